"""The oracle's NVFP4 value store (the 4-bit values of the Jet-QSparse
abstract's NVFP4 cache, aggregated in FP16 with FP32 accumulation), pinned to a
hand-packed row, exact round trips, the E2M1 error bound and the attention over
its rows (CPU)."""

import os

import numpy as np

from oracle import decode as O
from oracle import nvfp4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "value_store_worked_example.txt")
SIGMA = 1.0 / np.sqrt(128.0)


def _golden():
    out = {"code": {}, "scale": {}, "deq": {}}
    for line in open(GOLDEN):
        f = line.split("#")[0].split()
        if len(f) == 3:
            out[f[0]][int(f[1])] = float.fromhex(f[2]) if f[2].startswith("0x") and f[0] == "deq" \
                else (int(f[2], 16) if f[2].startswith("0x") else float(f[2]))
    return out


def test_hand_packed_row():
    g = _golden()
    v = np.zeros((1, 128), np.float32)
    v[0, :5] = [6, 3, -1.5, 0.5, 0]
    v[0, 16:18] = [1.0, 0.75]
    cb, sb = O.pack_values(v, np.float32(1.0))
    want_c = np.zeros(64, np.uint8)
    for i, x in g["code"].items():
        want_c[i] = x
    want_s = np.zeros(8, np.uint8)
    for i, x in g["scale"].items():
        want_s[i] = x
    assert np.array_equal(cb[0], want_c) and np.array_equal(sb[0], want_s)
    deq = O.dequant_values(cb, sb, 1.0)[0]
    want_d = np.zeros(128)
    for i, x in g["deq"].items():
        want_d[i] = x
    assert np.array_equal(deq, want_d)


def test_representable_rows_round_trip_exactly():
    """Rows built as s_v * e2m1 * e4m3 with a +-6 in every group (so the
    group's amax selects its scale exactly) pack to those codes and read back
    bit for bit, for power-of-two s_v."""
    rng = np.random.default_rng(3)
    T = 64
    for s_v in (1.0, 2.0 ** -7, 8.0):
        codes = rng.integers(0, 16, size=(T, 128)).astype(np.uint8)
        codes[:, ::16] = rng.choice([0x7, 0xF], size=(T, 8))  # +-6 per group
        sb = rng.integers(0x08, 0x7F, size=(T, 8)).astype(np.uint8)  # normal E4M3 scales
        vals = nvfp4.e2m1_decode(codes) * np.repeat(nvfp4.e4m3_decode(sb), 16, axis=-1) * s_v
        v = vals.astype(np.float32)
        assert np.array_equal(v.astype(np.float64), vals)
        cb, got_sb = O.pack_values(v, np.float32(s_v))
        assert np.array_equal(got_sb, sb)
        assert np.array_equal(O.dequant_values(cb, got_sb, s_v), vals)
        # the nibble order: channel 2i in the low nibble of byte i
        assert np.array_equal(cb & 0xF, codes[:, 0::2]) and np.array_equal(cb >> 4, codes[:, 1::2])


def test_random_rows_meet_the_e2m1_error_bound():
    """Each element is within half the local E2M1 step of its group's scale S
    (a step is 0.5 S below 2 S, S below 4 S, 2 S above), plus the saturation
    past 6 S the E4M3 rounding of the ratio can cause (at most S / 16 * 6)."""
    rng = np.random.default_rng(4)
    v = (rng.standard_normal((256, 128)) * rng.uniform(0.01, 50, size=(256, 1))).astype(np.float32)
    s_v = O.value_scale(v)
    cb, sb = O.pack_values(v, s_v)
    deq = O.dequant_values(cb, sb, s_v)
    S = np.repeat(nvfp4.e4m3_decode(sb), 16, axis=-1) * float(s_v)
    a = np.abs(v.astype(np.float64)) / S
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    bound = 0.5 * step * S + np.maximum(a - 6.0, 0.0) * S + 1e-12
    assert np.all(np.abs(deq - v) <= bound)
    assert float(s_v) == np.float32(np.abs(v).max()) / np.float32(2688.0)


def test_attention_over_the_store_is_attention_over_its_values():
    """The gather reads the store's dequantized values (tail pages from the
    BF16 store as before); with every block selected this is dense
    attention over those values."""
    rng = np.random.default_rng(5)
    T, L = 1024, 900
    q = rng.standard_normal((4, 128)).astype(np.float16)
    k = rng.standard_normal((T, 128)).astype(np.float16)
    v = rng.standard_normal((T, 128)).astype(np.float16)
    s_v = O.value_scale(v[:L])
    cb, sb = O.pack_values(v, s_v)
    blocks = list(range(O.n_pages(L)))
    kr, vr = O.gather_rows_block(k, v, blocks, L, 0, v_store=(cb, sb, s_v))
    vq = O.dequant_values(cb, sb, s_v)[:L]
    assert np.array_equal(vr, vq)
    o, lse = O.attend(q, kr, vr, SIGMA)
    logits = SIGMA * q.astype(np.float64) @ k[:L].astype(np.float64).T
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    dense = (w @ vq) / w.sum(axis=1, keepdims=True)
    assert np.abs(o - dense).max() < 1e-12
    # token mode: rows read at their tokens
    toks = [3, 77, 511, 899]
    _, vt = O.gather_rows_token(k, v, toks, v_store=(cb, sb, s_v))
    assert np.array_equal(vt, vq[toks])
