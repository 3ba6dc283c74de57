"""Pins of the oracle's NVFP4 packer and block scan (CPU)."""

import math
import os

import numpy as np
import pytest

from oracle import decode as O
from oracle import nvfp4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pack_worked_example.txt")
SIGMA = 1.0 / math.sqrt(128)


def _load_worked():
    keys, codes, scales, meta = [], {}, {}, {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            p = line.split()
            if p[0] == "key":
                keys.append((int(p[1]), int(p[2]), float(p[3])))
            elif p[0] == "code":
                codes[int(p[1])] = int(p[2], 16)
            elif p[0] == "scale":
                scales[int(p[1])] = int(p[2], 16)
            else:
                meta[p[0]] = float(p[1])
    return keys, codes, scales, meta


def test_pack_worked_example_bytes():
    keys, codes, scales, meta = _load_worked()
    k = np.zeros((128, 128), dtype=np.float16)
    for t, d, v in keys:
        k[t, d] = v
    rec_c, rec_s = O.pack_unit_blocks(k, np.zeros(128, np.float32), meta["global_scale"], 0, 1)
    exp_c = np.zeros(8192, np.uint8)
    for off, b in codes.items():
        exp_c[off] = b
    exp_s = np.zeros(1024, np.uint8)
    for off, b in scales.items():
        exp_s[off] = b
    assert np.array_equal(rec_c[0], exp_c)
    assert np.array_equal(rec_s[0], exp_s)


def test_scan_worked_example():
    keys, _, _, meta = _load_worked()
    k = np.zeros((128, 128), dtype=np.float16)
    for t, d, v in keys:
        k[t, d] = v
    c = np.zeros(128, np.float32)
    rc, rs = O.pack_unit_blocks(k, c, meta["global_scale"], 0, 1)
    q = np.zeros((1, 128), np.float16)
    q[0, 0] = 1.0
    s = O.scan_block_unit(q, rc, rs, meta["global_scale"], c, 128, 0, SIGMA)
    assert abs(s[0] - meta["block_score_q_e0"]) < 1e-15


def test_layout_is_a_bijection():
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 16, (3, 128, 128)).astype(np.uint8)
    assert np.array_equal(O.cache_layout_to_codes(O.codes_to_cache_layout(codes)), codes)
    sb = rng.integers(0, 256, (3, 128, 8)).astype(np.uint8)
    assert np.array_equal(O.cache_layout_to_scales(O.scales_to_cache_layout(sb)), sb)
    # every byte of a record is written by exactly one (token, channel pair)
    rec = O.codes_to_cache_layout(np.arange(128 * 128).reshape(128, 128) % 16)
    assert rec.shape == (8192,)


def _exact_keys(rng, T, center, st, sb_range=(0x38, 0x48)):
    """Keys whose centered values are exactly e2m1 * e4m3 * s_t, one 6 per group.

    The scale codes stay in a narrow range so that key = value + center is
    exact in fp16 (checked below).
    """
    sb = rng.integers(*sb_range, (T, 8))
    e = rng.integers(0, 16, (T, 8, 16))
    e[e == 8] = 0  # avoid -0
    e[..., 0] = 7  # largest magnitude sits in every group
    vals = (nvfp4.e2m1_decode(e) * nvfp4.e4m3_decode(sb)[..., None] * st).reshape(T, 128)
    k = (vals + center[None, :]).astype(np.float16)
    assert np.array_equal(k.astype(np.float64) - center[None, :], vals)  # exact in fp16
    return k, e.reshape(T, 128).astype(np.uint8), sb.astype(np.uint8), vals


def test_pack_round_trips_representable_keys():
    rng = np.random.default_rng(1)
    st = 2.0 ** -6
    center = (rng.integers(-4, 5, 128) * 0.125).astype(np.float32)
    k, e, sb, _ = _exact_keys(rng, 256, center.astype(np.float64), st)
    codes, scales = O.pack_nvfp4(k, center, st)
    assert np.array_equal(scales, sb)
    assert np.array_equal(codes, e)
    # without centering the whole scale range is exact, subnormal scales included
    zero = np.zeros(128)
    k, e, sb, _ = _exact_keys(rng, 256, zero, st, sb_range=(0x01, 0x7F))
    codes, scales = O.pack_nvfp4(k, zero.astype(np.float32), st)
    assert np.array_equal(scales, sb)
    assert np.array_equal(codes, e)


def test_pack_error_bound_random_keys():
    rng = np.random.default_rng(2)
    k = (rng.standard_normal((512, 128)) * 3 + 1).astype(np.float16)
    c = k.astype(np.float64).mean(axis=0).astype(np.float32)
    y = k.astype(np.float32) - c
    st = np.float32(np.abs(y).max() / np.float32(2688.0))
    codes, sb = O.pack_nvfp4(k, c, st)
    S = (nvfp4.e4m3_decode(sb).astype(np.float32) * st).astype(np.float32).astype(np.float64)
    Sx = np.repeat(S, 16, axis=-1)
    xq = nvfp4.e2m1_decode(codes)
    x = y.astype(np.float64) / Sx
    assert np.all(np.abs(x) <= 6 * (1 + 2 ** -3))  # no group is far into saturation
    # half the local E2M1 gap: 0.25 below 2, 0.5 below 4, 1 up to 6
    gap = np.where(np.abs(xq) < 2, 0.25, np.where(np.abs(xq) < 4, 0.5, 1.0))
    assert np.all(np.abs(x - xq) <= gap + 1e-6)


def test_scan_equals_exact_logits_for_representable_keys():
    rng = np.random.default_rng(3)
    st = 2.0 ** -6
    center = (rng.integers(-4, 5, 128) * 0.125)
    T, G = 640, 4  # 5 blocks
    k, _, _, _ = _exact_keys(rng, T, center, st)
    q = rng.standard_normal((G, 128)).astype(np.float16)
    rc, rs = O.pack_unit_blocks(k, center.astype(np.float32), st, 0, T // 128)
    for L, n_tail in [(T, 0), (600, 0), (600, 2), (129, 1)]:
        s = O.scan_block_unit(q, rc, rs, st, center.astype(np.float32), L, n_tail, SIGMA,
                              max_blocks=T // 128)
        # brute force: best exact logit over heads and valid tokens of each scanned block
        npg = -(-L // 128)
        for blk in range(T // 128):
            if blk >= max(0, npg - n_tail):
                assert s[blk] == -np.inf
                continue
            best = -np.inf
            for t in range(blk * 128, min(L, blk * 128 + 128)):
                for h in range(G):
                    best = max(best, SIGMA * float(np.dot(q[h].astype(np.float64),
                                                          k[t].astype(np.float64))))
            assert abs(s[blk] - best) <= 1e-12 * max(1.0, abs(best)), (L, n_tail, blk)


def test_scan_max_over_group_heads():
    rng = np.random.default_rng(4)
    k = rng.standard_normal((256, 128)).astype(np.float16)
    c = np.zeros(128, np.float32)
    st = np.float32(np.abs(k.astype(np.float32)).max() / 2688)
    rc, rs = O.pack_unit_blocks(k, c, st, 0, 2)
    q = rng.standard_normal((4, 128)).astype(np.float16)
    full = O.scan_block_unit(q, rc, rs, st, c, 256, 0, SIGMA)
    per_head = np.stack([O.scan_block_unit(q[h:h + 1], rc, rs, st, c, 256, 0, SIGMA)
                         for h in range(4)])
    assert np.array_equal(full, per_head.max(axis=0))


# ---- the NVFP4 query (scan only) -------------------------------------------

def _exact_query(rng, G, sq_exp=-12):
    """Heads whose values are exactly e2m1 * e4m3 * 2^sq_exp, every group holding
    a +-6 and one group per head at scale 448, so amax = 2688 * 2^sq_exp and
    s_q = 2^sq_exp."""
    sb = rng.integers(0x08, 0x7E, (G, 8))
    top = rng.integers(0, 8, G)
    sb[np.arange(G), top] = 0x7E
    e = rng.integers(0, 16, (G, 8, 16))
    e[e == 8] = 0  # no -0
    # every group holds a +-6, so its amax sets its scale
    e[np.arange(G)[:, None], np.arange(8)[None, :], rng.integers(0, 16, (G, 8))] = \
        7 + 8 * rng.integers(0, 2, (G, 8))
    vals = nvfp4.e2m1_decode(e) * nvfp4.e4m3_decode(sb)[..., None] * 2.0 ** sq_exp
    q = vals.reshape(G, 128).astype(np.float16)
    assert np.array_equal(q.astype(np.float64), vals.reshape(G, 128))  # exact in fp16
    return q, e.reshape(G, 128).astype(np.uint8), sb.astype(np.uint8)


def test_query_quantizer_round_trips_representable_heads():
    rng = np.random.default_rng(11)
    q, e, sb = _exact_query(rng, 16)
    codes, scales, s_q = O.quantize_query(q)
    assert np.array_equal(s_q, np.full(16, 2.0 ** -12, np.float32))
    assert np.array_equal(scales, sb)
    assert np.array_equal(codes, e)
    assert np.array_equal(O.dequant_query(codes, scales, s_q), q.astype(np.float64))
    assert np.array_equal(O.scan_query(q, "nvfp4"), q.astype(np.float64))


def test_query_scale_puts_the_largest_group_at_448():
    rng = np.random.default_rng(12)
    q = (rng.standard_normal((64, 128)) * rng.uniform(0.01, 30, (64, 1))).astype(np.float16)
    codes, sb, s_q = O.quantize_query(q)
    amax = np.abs(q.astype(np.float32)).max(axis=1)
    assert np.array_equal(s_q, (amax / np.float32(2688.0)).astype(np.float32))
    g = np.abs(q.astype(np.float32)).reshape(64, 8, 16).max(axis=2).argmax(axis=1)
    assert np.all(sb[np.arange(64), g] == 0x7E)
    assert np.all(sb <= 0x7E)


def test_query_quantizer_is_scale_invariant_by_powers_of_two():
    rng = np.random.default_rng(13)
    q = (rng.standard_normal((8, 128)) * 0.5).astype(np.float16)
    c0, s0, q0 = O.quantize_query(q)
    for k in (-3, 2, 5):
        c1, s1, q1 = O.quantize_query((q.astype(np.float32) * 2.0 ** k).astype(np.float16))
        assert np.array_equal(c0, c1) and np.array_equal(s0, s1)
        assert np.array_equal(q1, (q0 * np.float32(2.0 ** k)).astype(np.float32))


def test_query_quantizer_error_bound():
    rng = np.random.default_rng(14)
    q = (rng.standard_normal((256, 128)) * 2).astype(np.float16)
    codes, sb, s_q = O.quantize_query(q)
    S = nvfp4.e4m3_decode(sb) * s_q.astype(np.float64)[:, None]
    x = q.astype(np.float64) / np.repeat(S, 16, axis=1)
    xq = nvfp4.e2m1_decode(codes)
    assert np.all(np.abs(x) <= 6 * (1 + 2 ** -3))
    gap = np.where(np.abs(xq) < 2, 0.25, np.where(np.abs(xq) < 4, 0.5, 1.0))
    assert np.all(np.abs(x - xq) <= gap + 1e-6)
    qt = O.scan_query(q, "nvfp4")
    assert np.all(np.abs(qt - q) <= np.repeat(S, 16, axis=1) * (gap + 1e-6))


def test_zero_query_head_scores_zero():
    rng = np.random.default_rng(15)
    k = rng.standard_normal((256, 128)).astype(np.float16)
    c = rng.standard_normal(128).astype(np.float32)
    codes, sb, s_q = O.quantize_query(np.zeros((2, 128), np.float16))
    assert not codes.any() and not sb.any() and not s_q.any()
    st = np.float32(2.0 ** -6)
    rc, rs = O.pack_unit_blocks(k, c, st, 0, 2)
    s = O.scan_block_unit(O.scan_query(np.zeros((2, 128), np.float16), "nvfp4"), rc, rs, st, c,
                          256, 0, SIGMA)
    assert np.array_equal(s, np.zeros(2))


def test_quantized_query_scan_equals_exact_logits():
    """Representable keys and a non-representable query: the scores are the exact
    logits of qtilde, which differ from those of q."""
    rng = np.random.default_rng(16)
    st = 2.0 ** -6
    center = rng.integers(-4, 5, 128) * 0.125
    k, _, _, _ = _exact_keys(rng, 256, center, st)
    q = rng.standard_normal((4, 128)).astype(np.float16)
    qt = O.scan_query(q, "nvfp4")
    rc, rs = O.pack_unit_blocks(k, center.astype(np.float32), st, 0, 2)
    s = O.scan_block_unit(qt, rc, rs, st, center.astype(np.float32), 256, 0, SIGMA)
    for blk in range(2):
        rows = k[blk * 128:(blk + 1) * 128].astype(np.float64)
        best = SIGMA * (rows @ qt.T).max()
        assert abs(s[blk] - best) <= 1e-12 * max(1.0, abs(best))
        assert best != SIGMA * (rows @ q.astype(np.float64).T).max()
