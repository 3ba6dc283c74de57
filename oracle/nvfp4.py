"""NVFP4 element and scale codecs (oracle; test infrastructure only).

The Jet-QSparse abstract stores the key history in NVFP4 and names no further
detail of the format. NVFP4 is
the public 4-bit format with

* E2M1 elements: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; the
  exponent field 0 encodes the subnormal 0.5 * mantissa; no infinity or NaN;
  magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6;
* E4M3 block scales (the OCP E4M3FN variant): 1 sign bit, 4 exponent bits
  (bias 7), 3 mantissa bits; subnormals m * 2^-9; the all-ones pattern
  S.1111.111 is NaN; no infinity; largest finite value 448;
* one scale per 16 consecutive elements and one FP32 scale per tensor.

Encoding is round-to-nearest, ties to the even code, saturating to the largest
finite magnitude (reading chosen for the packer; the pages give no rounding
rule). Values here are derived from the bit fields, not from a table.
"""

from __future__ import annotations

import numpy as np


def e2m1_value(code: int) -> float:
    """Real value of one 4-bit E2M1 code, from its sign/exponent/mantissa fields."""
    sign = -1.0 if (code >> 3) & 1 else 1.0
    exp = (code >> 1) & 3
    man = code & 1
    if exp == 0:
        return sign * 0.5 * man
    return sign * 2.0 ** (exp - 1) * (1.0 + 0.5 * man)


def e4m3_value(code: int) -> float:
    """Real value of one E4M3FN byte (NaN for S.1111.111)."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    exp = (code >> 3) & 15
    man = code & 7
    if exp == 15 and man == 7:
        return float("nan")
    if exp == 0:
        return sign * man * 2.0 ** -9
    return sign * 2.0 ** (exp - 7) * (1.0 + man / 8.0)


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e2m1_decode(codes) -> np.ndarray:
    return E2M1_TABLE[np.asarray(codes, dtype=np.int64)]


def e4m3_decode(codes) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.int64)]


def _nearest_even(x: np.ndarray, values: np.ndarray, codes: np.ndarray,
                  chunk: int = 1 << 16) -> np.ndarray:
    """Index into ``codes`` of the value nearest to each x; ties go to the even code."""
    x = np.asarray(x, dtype=np.float64).ravel()
    out = np.empty(x.shape, dtype=np.int64)
    for lo in range(0, x.size, chunk):
        xs = x[lo:lo + chunk, None]
        dist = np.abs(xs - values[None, :])
        best = dist == dist.min(axis=1, keepdims=True)
        # among equally near values prefer the even code (mantissa LSB 0)
        pref = best * (2 - (codes[None, :] & 1))
        out[lo:lo + chunk] = np.argmax(pref, axis=1)
    return out


_E2M1_POS_CODES = np.arange(8, dtype=np.int64)
_E2M1_POS_VALUES = E2M1_TABLE[:8]
_E4M3_POS_CODES = np.arange(0x7F, dtype=np.int64)  # 0x00 .. 0x7E, all finite
_E4M3_POS_VALUES = E4M3_TABLE[:0x7F]


def e2m1_encode(x) -> np.ndarray:
    """Nearest E2M1 code (ties to even, saturating at 6); sign copied from x."""
    x = np.asarray(x, dtype=np.float32)
    # saturation: magnitudes beyond the largest finite value take that value
    mag = np.minimum(np.abs(x.astype(np.float64)).ravel(), _E2M1_POS_VALUES[-1])
    idx = _nearest_even(mag, _E2M1_POS_VALUES, _E2M1_POS_CODES)
    code = _E2M1_POS_CODES[idx] | (np.signbit(x.ravel()).astype(np.int64) << 3)
    return code.astype(np.uint8).reshape(x.shape)


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3FN code of a signed value (ties to even, saturating at 448,
    never NaN); the sign bit is copied from x, so -0 is 0x80."""
    x = np.asarray(x, dtype=np.float32)
    if np.any(np.isnan(x)):
        raise ValueError("no NaN input")
    mag = np.minimum(np.abs(x.astype(np.float64)).ravel(), _E4M3_POS_VALUES[-1])
    idx = _nearest_even(mag, _E4M3_POS_VALUES, _E4M3_POS_CODES)
    code = _E4M3_POS_CODES[idx] | (np.signbit(x.ravel()).astype(np.int64) << 7)
    return code.astype(np.uint8).reshape(x.shape)


def e4m3_encode_nonneg(x) -> np.ndarray:
    """Nearest non-negative E4M3FN code (ties to even, saturating at 448)."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(x < 0) or np.any(np.isnan(x)):
        raise ValueError("block scales are non-negative")
    idx = _nearest_even(np.minimum(x.ravel(), _E4M3_POS_VALUES[-1]),
                        _E4M3_POS_VALUES, _E4M3_POS_CODES)
    return _E4M3_POS_CODES[idx].astype(np.uint8).reshape(x.shape)
