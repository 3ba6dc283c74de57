"""Pins of the oracle's NVFP4 codecs against the format definitions (CPU)."""

import math
import os

import numpy as np
import pytest

from oracle import nvfp4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nvfp4_codec_points.txt")


def _golden(kind):
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            k, a, b = line.split()
            if k == kind:
                rows.append((a, b))
    assert rows, kind
    return rows


def _same(a, b):
    if math.isnan(b):
        return math.isnan(a)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


@pytest.mark.parametrize("kind,fn", [("e2m1", nvfp4.e2m1_value), ("e4m3", nvfp4.e4m3_value)])
def test_decode_matches_format_points(kind, fn):
    for code, val in _golden(kind):
        assert _same(fn(int(code, 16)), float(val)), (kind, code, val)


def test_e2m1_encode_points():
    for x, code in _golden("e2m1_enc"):
        got = int(nvfp4.e2m1_encode(np.float32(float(x))))
        assert got == int(code, 16), (x, code, got)


def test_e4m3_encode_points():
    for x, code in _golden("e4m3_enc"):
        got = int(nvfp4.e4m3_encode_nonneg(np.float64(float(x))))
        assert got == int(code, 16), (x, code, got)


def test_every_finite_code_round_trips():
    for c in range(16):
        v = nvfp4.e2m1_value(c)
        assert int(nvfp4.e2m1_encode(np.float32(v))) == c
    for c in range(0x7F):
        assert int(nvfp4.e4m3_encode_nonneg(nvfp4.e4m3_value(c))) == c


def test_e4m3_table_is_strictly_increasing_and_bounded():
    v = nvfp4.E4M3_TABLE[:0x7F]
    assert np.all(np.diff(v) > 0)
    assert v[-1] == 448.0 and v[1] == 2.0 ** -9
    # negative half mirrors the positive half
    assert np.array_equal(nvfp4.E4M3_TABLE[0x80:0xFF], -v)


def test_encoders_are_optimal_brute_force():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.uniform(-8, 8, 4000), rng.uniform(-1, 1, 2000)]).astype(np.float32)
    codes = nvfp4.e2m1_encode(x)
    err = np.abs(x.astype(np.float64) - nvfp4.e2m1_decode(codes))
    all_err = np.abs(x.astype(np.float64)[:, None] - nvfp4.E2M1_TABLE[None, :])
    assert np.all(err <= all_err.min(axis=1))
    s = np.exp(rng.uniform(np.log(1e-4), np.log(600), 5000))
    sc = nvfp4.e4m3_encode_nonneg(s)
    err = np.abs(s - nvfp4.e4m3_decode(sc))
    all_err = np.abs(s[:, None] - nvfp4.E4M3_TABLE[None, :0x7F])
    assert np.all(err <= all_err.min(axis=1))


def test_encoders_monotone():
    x = np.linspace(-7, 7, 20001).astype(np.float32)
    v = nvfp4.e2m1_decode(nvfp4.e2m1_encode(x))
    assert np.all(np.diff(v) >= 0)
    s = np.linspace(0, 500, 20001)
    v = nvfp4.e4m3_decode(nvfp4.e4m3_encode_nonneg(s))
    assert np.all(np.diff(v) >= 0)


def test_e2m1_sign_copied_and_negative_zero():
    assert int(nvfp4.e2m1_encode(np.float32(-0.0))) == 8
    assert int(nvfp4.e2m1_encode(np.float32(-0.2))) == 8
    assert int(nvfp4.e2m1_encode(np.float32(0.2))) == 0


def test_signed_e4m3_encode_points():
    for x, code in _golden("e4m3s_enc"):
        got = int(nvfp4.e4m3_encode(np.float32(float(x))))
        assert got == int(code, 16), (x, code, got)


def test_signed_e4m3_every_finite_code_round_trips():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        v = nvfp4.e4m3_value(c)
        assert int(nvfp4.e4m3_encode(np.float32(-0.0 if c == 0x80 else v))) == c


def test_signed_e4m3_is_nearest_with_even_ties_brute_force():
    # the definition, written out: the finite value nearest to x, the code with
    # an even mantissa among equally near ones, the sign of x
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.standard_normal(3000) * 3, rng.uniform(-500, 500, 1000),
                        rng.uniform(-0.02, 0.02, 1000),
                        (rng.integers(-900, 900, 1000) * 2.0 ** -10)]).astype(np.float32)
    mags = [nvfp4.e4m3_value(c) for c in range(0x7F)]
    for xi, ci in zip(x, nvfp4.e4m3_encode(x)):
        a = min(abs(float(xi)), 448.0)
        d = [abs(a - m) for m in mags]
        best = [c for c in range(0x7F) if d[c] == min(d)]
        want = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]
        want |= 0x80 if np.signbit(xi) else 0
        assert int(ci) == want, (float(xi), int(ci), want)
