"""Pins of the oracle's selection, attention, combine and token path (CPU)."""

import math

import os

import numpy as np
import pytest
import torch

from oracle import decode as O

SIGMA = 1.0 / math.sqrt(128)


def _rank_select(scores, n_cand, picks):
    """Brute force: candidate i is chosen iff fewer than `picks` candidates beat it."""
    chosen = []
    for i in range(n_cand):
        beat = sum(1 for j in range(n_cand)
                   if scores[j] > scores[i] or (scores[j] == scores[i] and j < i))
        if beat < picks:
            chosen.append(i)
    return chosen


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_select_matches_rank_counting_with_ties(seed):
    rng = np.random.default_rng(seed)
    n = 97
    s = np.round(rng.standard_normal(n) * 2) / 2  # many exact ties
    for budget in [1, 5, 20, 96, 97, 120]:
        idx, cnt = O.select_unit(s, n, budget)
        exp = _rank_select(s, n, budget)
        assert cnt == len(exp)
        assert list(idx[:cnt]) == exp  # ascending
        assert np.all(idx[cnt:] == -1)


def test_select_blocks_forced_tail_pages():
    rng = np.random.default_rng(5)
    L = 128 * 10 + 7  # 11 pages, the last partial
    scores = rng.standard_normal(16)
    idx, cnt = O.select_blocks_unit(scores, L, 2, 5)
    # 3 picks among the 9 scanned blocks plus pages 9 and 10
    exp = sorted(_rank_select(scores, 9, 3) + [9, 10])
    assert cnt == 5 and list(idx) == exp
    # fewer pages than tail slots
    idx, cnt = O.select_blocks_unit(scores, 100, 2, 4)
    assert cnt == 1 and list(idx) == [0, -1, -1, -1]
    # empty sequence
    idx, cnt = O.select_blocks_unit(scores, 0, 2, 4)
    assert cnt == 0 and np.all(idx == -1)


def test_budget_all_blocks_is_dense_attention():
    rng = np.random.default_rng(6)
    T, G = 1024, 4
    q = rng.standard_normal((G, 128)).astype(np.float16)
    k = rng.standard_normal((T, 128)).astype(np.float16)
    v = rng.standard_normal((T, 128)).astype(np.float16)
    idx = np.arange(T // 128)
    kr, vr = O.gather_rows_block(k, v, idx, T, 0)
    o, lse = O.attend(q, kr, vr, SIGMA)
    qt = torch.from_numpy(q.astype(np.float64))
    kt = torch.from_numpy(k.astype(np.float64))
    vt = torch.from_numpy(v.astype(np.float64))
    logits = SIGMA * qt @ kt.T
    ref = torch.softmax(logits, dim=-1) @ vt
    assert np.abs(o - ref.numpy()).max() < 1e-12
    assert np.abs(lse - torch.logsumexp(logits, dim=-1).numpy()).max() < 1e-12


def test_attention_brute_force_loops():
    rng = np.random.default_rng(7)
    T, G = 300, 2
    q = rng.standard_normal((G, 128)).astype(np.float16)
    k = rng.standard_normal((T, 128)).astype(np.float16)
    v = rng.standard_normal((T, 128)).astype(np.float16)
    sel = [0, 2]  # blocks 0 and 2 (tokens 0..127, 256..299)
    kr, vr = O.gather_rows_block(k, v, sel, T, 0)
    o, lse = O.attend(q, kr, vr, SIGMA)
    toks = list(range(0, 128)) + list(range(256, 300))
    for h in range(G):
        w = [math.exp(SIGMA * sum(float(q[h, d]) * float(k[t, d]) for d in range(128)))
             for t in toks]
        z = sum(w)
        for d in (0, 17, 127):
            od = sum(wi * float(v[t, d]) for wi, t in zip(w, toks)) / z
            assert abs(o[h, d] - od) < 1e-12
        assert abs(lse[h] - math.log(z)) < 1e-12


def test_centering_does_not_change_attention():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((4, 128)).astype(np.float16)
    k = rng.standard_normal((512, 128))
    v = rng.standard_normal((512, 128))
    c = rng.standard_normal(128) * 3
    o1, _ = O.attend(q, k, v, SIGMA)
    o2, _ = O.attend(q, k - c[None, :], v, SIGMA)
    assert np.abs(o1 - o2).max() < 1e-12


@pytest.mark.parametrize("splits", [1, 2, 3, 8, 16])
def test_combine_independent_of_split_count(splits):
    rng = np.random.default_rng(9)
    T = 1280
    q = rng.standard_normal((4, 128)).astype(np.float16)
    k = rng.standard_normal((T, 128)).astype(np.float16)
    v = rng.standard_normal((T, 128)).astype(np.float16)
    idx = np.array([0, 3, 4, 7, 9, -1, -1], dtype=np.int32)
    rows = lambda sel: O.gather_rows_block(k, v, sel, T, 0)
    po, pl = O.attend_splits(q, idx, splits, rows, SIGMA)
    o, lse = O.combine(po, pl)
    kr, vr = rows([0, 3, 4, 7, 9])
    o1, l1 = O.attend(q, kr, vr, SIGMA)
    assert np.abs(o - o1).max() < 1e-12 and np.abs(lse - l1).max() < 1e-12
    if splits == 1:
        assert np.array_equal(po[0], o1)


@pytest.mark.parametrize("n,splits", [(0, 3), (1, 8), (5, 2), (62, 8), (64, 8), (2048, 8), (7, 16)])
def test_split_ranges_share_the_selected_entries(n, splits):
    """The splits tile [0, n) in order, each at most ceil(n / S) entries, and
    the empty ones come last."""
    r = O.split_ranges(n, splits)
    assert len(r) == splits
    per = -(-n // splits)
    cover = []
    for lo, hi in r:
        assert 0 <= lo <= hi <= n and hi - lo <= per
        cover.extend(range(lo, hi))
    assert cover == list(range(n))
    sizes = [hi - lo for lo, hi in r]
    assert sizes == sorted(sizes, reverse=True)


def test_empty_selection_gives_zero_and_minus_inf():
    q = np.ones((4, 128), np.float16)
    po, pl = O.attend_splits(q, np.full(4, -1, np.int32), 2,
                             lambda sel: (np.zeros((0, 128)), np.zeros((0, 128))), SIGMA)
    o, lse = O.combine(po, pl)
    assert np.all(o == 0) and np.all(lse == -np.inf)


def test_tail_pages_read_from_bf16_store():
    rng = np.random.default_rng(10)
    L = 128 * 5 + 40  # 6 pages; pages 4, 5 live in the tail store
    T = 1024
    q = rng.standard_normal((4, 128)).astype(np.float16)
    x = rng.standard_normal((T, 128)).astype(np.float32)
    xv = rng.standard_normal((T, 128)).astype(np.float32)
    k = x.astype(np.float16)
    v = xv.astype(np.float16)
    tk = np.zeros((2, 128, 128), np.uint16)
    tv = np.zeros((2, 128, 128), np.uint16)
    for s, page in enumerate([4, 5]):
        tk[s] = O.f32_to_bf16_bits(x[page * 128:(page + 1) * 128])
        tv[s] = O.f32_to_bf16_bits(xv[page * 128:(page + 1) * 128])
    k[512:] = 1000  # the main buffer at tail pages is never read
    kr, vr = O.gather_rows_block(k, v, [1, 4, 5], L, 2, tk, tv)
    assert kr.shape[0] == 128 + 128 + 40
    assert np.array_equal(kr[128:256], O.bf16_bits_to_f64(tk[0]))
    assert np.array_equal(kr[256:], O.bf16_bits_to_f64(tk[1, :40]))
    xk = torch.from_numpy(x[512:512 + 168]).to(torch.bfloat16).double().numpy()
    assert np.array_equal(kr[128:], xk)


# ---------------------------------------------------------------- token path

def test_identity_projection_gives_bf16_keys():
    rng = np.random.default_rng(11)
    k = rng.standard_normal((300, 128)).astype(np.float16)
    P = np.eye(128, dtype=np.float32)
    bits = O.project_keys(k, P)
    ref = torch.from_numpy(k.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(bits.view(np.int16), ref)


def test_projection_within_float32_error_bound():
    rng = np.random.default_rng(12)
    k = rng.standard_normal((500, 128)).astype(np.float16)
    g = rng.standard_normal((128, 32))
    P = np.linalg.qr(g)[0].astype(np.float32)
    got = O.bf16_bits_to_f64(O.project_keys(k, P))
    exact = k.astype(np.float64) @ P.astype(np.float64)
    absterm = np.abs(k.astype(np.float64)) @ np.abs(P.astype(np.float64))
    u32 = 2.0 ** -24
    bound = 129 * u32 * absterm + 2.0 ** -8 * np.abs(exact) * 1.01
    assert np.all(np.abs(got - exact) <= bound)


def test_token_scores_follow_mean_query_and_rotation():
    rng = np.random.default_rng(13)
    T, G = 400, 4
    k = rng.standard_normal((T, 128)).astype(np.float16)
    q = rng.standard_normal((G, 128)).astype(np.float16)
    P = np.linalg.qr(rng.standard_normal((128, 128)))[0].astype(np.float32)
    s = O.scan_token_unit(q, O.project_keys(k, P), P, T, SIGMA)
    qbar = q.astype(np.float64).mean(axis=0)
    exact = SIGMA * (k.astype(np.float64) @ qbar)
    # full-rank orthonormal P: scores are sigma * qbar . k up to BF16 rounding of P^T k
    bound = SIGMA * (np.abs(k.astype(np.float64)) @ np.abs(P.astype(np.float64))
                     ) @ np.abs(P.astype(np.float64).T @ qbar) * 2.0 ** -7
    assert np.all(np.abs(s - exact) <= bound + 1e-9)
    # the score depends on the group only through its mean query
    qm = np.repeat(qbar[None, :], G, axis=0)
    s2 = O.scan_token_unit(qm, O.project_keys(k, P), P, T, SIGMA)
    assert np.abs(s - s2).max() < 1e-12
    # masking beyond the sequence length
    s3 = O.scan_token_unit(q, O.project_keys(k, P), P, 250, SIGMA)
    assert np.all(s3[250:] == -np.inf) and np.array_equal(s3[:250], s[:250])


def test_token_select_and_gather_free_rows():
    rng = np.random.default_rng(14)
    T = 512
    s = np.round(rng.standard_normal(T), 1)
    idx, cnt = O.select_tokens_unit(s, 400, 37)
    assert cnt == 37 and list(idx) == _rank_select(s, 400, 37)
    k = rng.standard_normal((T, 128)).astype(np.float16)
    v = rng.standard_normal((T, 128)).astype(np.float16)
    kr, vr = O.gather_rows_token(k, v, idx[:cnt])
    assert np.array_equal(kr, k[idx[:cnt]].astype(np.float64))


# ---------------------------------------------------------------- FP8 projected cache

def _e4m3_nearest_even(x):
    """Brute-force E4M3FN encode of float32 values (the format definition)."""
    from oracle import nvfp4

    mags = np.array([nvfp4.e4m3_value(c) for c in range(0x7F)])
    out = []
    for xi in np.asarray(x, dtype=np.float32).ravel():
        a = min(abs(float(xi)), 448.0)
        d = np.abs(mags - a)
        best = np.flatnonzero(d == d.min())
        c = int(best[0]) if best.size == 1 else int(best[best % 2 == 0][0])
        out.append(c | (0x80 if np.signbit(xi) else 0))
    return np.array(out, dtype=np.uint8).reshape(np.shape(x))


def test_fp8_identity_projection_gives_e4m3_of_keys():
    rng = np.random.default_rng(21)
    k = (rng.standard_normal((200, 128)) * np.array([0.01, 1.0, 40.0, 600.0]).repeat(32)
         ).astype(np.float16)
    P = np.eye(128, dtype=np.float32)[:, :32]
    got = O.project_keys(k, P, "fp8")
    assert got.dtype == np.uint8 and np.array_equal(got, _e4m3_nearest_even(k[:, :32]))


def test_fp8_projection_within_error_bound():
    rng = np.random.default_rng(22)
    k = rng.standard_normal((500, 128)).astype(np.float16)
    P = np.linalg.qr(rng.standard_normal((128, 32)))[0].astype(np.float32)
    got = O.proj_values(O.project_keys(k, P, "fp8"), "fp8")
    exact = k.astype(np.float64) @ P.astype(np.float64)
    absterm = np.abs(k.astype(np.float64)) @ np.abs(P.astype(np.float64))
    # float32 accumulation, then E4M3: half a unit in the last place (2^-4
    # relative for normal values, 2^-10 absolute among subnormals)
    acc_err = 129 * 2.0 ** -24 * absterm
    bound = acc_err + 2.0 ** -4 * (np.abs(exact) + acc_err) + 2.0 ** -10
    assert np.all(np.abs(got - exact) <= bound)


def test_fp8_token_scores_exact_for_representable_keys():
    from oracle import nvfp4

    rng = np.random.default_rng(23)
    T, G = 300, 4
    finite = np.array([nvfp4.e4m3_value(c) for c in range(256) if c not in (0x7F, 0xFF)])
    k = np.zeros((T, 128), dtype=np.float16)
    k[:, :32] = rng.choice(finite, size=(T, 32)).astype(np.float16)  # exact in fp16
    q = rng.standard_normal((G, 128)).astype(np.float16)
    P = np.eye(128, dtype=np.float32)[:, :32]
    s = O.scan_token_unit(q, O.project_keys(k, P, "fp8"), P, 250, SIGMA, "fp8")
    qbar = q.astype(np.float64).mean(axis=0)
    exact = SIGMA * (k[:, :32].astype(np.float64) @ qbar[:32])
    assert np.abs(s[:250] - exact[:250]).max() < 1e-12 and np.all(s[250:] == -np.inf)


BF16_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bf16_rne_points.txt")


def _bf16_golden():
    pts = []
    for line in open(BF16_GOLDEN):
        line = line.split("#")[0].split()
        if len(line) >= 2:
            pts.append((int(line[0], 16), int(line[1], 16)))
    return pts


def test_bf16_rounding_matches_hand_derived_points():
    pts = _bf16_golden()
    f = np.array([p[0] for p in pts], dtype=np.uint32).view(np.float32)
    got = O.f32_to_bf16_bits(f)
    for (fb, want), g in zip(pts, got):
        if want & 0x7F80 == 0x7F80 and want & 0x7F:  # NaN: any quiet NaN of that sign
            assert g & 0x7FC0 == 0x7FC0 and (g >> 15) == (want >> 15), hex(fb)
        else:
            assert int(g) == want, (hex(fb), hex(int(g)), hex(want))


def test_bf16_rounding_is_the_nearest_value_ties_to_even():
    """Brute force by value on random and crafted patterns: the result is the
    nearer of the two bfloat16 values around x (exact in float64), the even one
    on a tie, and infinity past the largest finite one's midpoint."""
    rng = np.random.default_rng(12)
    bits = rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32)
    edges = np.array([0x7F7F8000, 0x7F7FFFFF, 0x7F7F7FFF, 0xFF7F8000, 0x00008000, 0x80018000],
                     dtype=np.uint32)
    bits = np.concatenate([bits, (bits & 0xFFFF0000) | 0x8000, bits & 0xFFFF0000, edges])
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    got = O.f32_to_bf16_bits(x)
    lo = (x.view(np.uint32) >> 16).astype(np.uint32)  # truncation toward zero
    hi = lo + 1

    def val(b):
        # the pattern one step past the largest finite value stands for 2^128,
        # as if the exponent range went on: rounding there gives infinity
        v = (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        past = (b & 0x7FFF) == 0x7F80
        return np.where(past, np.where(b & 0x8000, -2.0**128, 2.0**128), v)

    xv = x.astype(np.float64)
    dlo, dhi = np.abs(xv - val(lo)), np.abs(val(hi) - xv)
    with np.errstate(invalid="ignore"):
        pick_hi = (dhi < dlo) | ((dhi == dlo) & (lo % 2 == 1))
    want = np.where(pick_hi, hi, lo).astype(np.uint16)
    assert np.array_equal(got, want)


def test_tail_store_from_cache_worked_example():
    # 130 tokens, two tail pages: slot 0 is page 0 (rows 0..127), slot 1 page 1
    # (rows 128, 129, then zeros); one tail page at 128 tokens is page 0 whole.
    # Rows hold float16 values whose bfloat16 roundings are hand-derived points:
    # 1 + 4/1024 (a tie, to 1.0), 1 + 12/1024 (a tie, up), 1 + 9/1024 (down),
    # 65504 (up to 65536), and small integers (exact).
    vals = np.array([1 + 4 / 1024, 1 + 12 / 1024, 1 + 9 / 1024, 65504.0, -3.0, 7.0], np.float16)
    want = {1 + 4 / 1024: 0x3F80, 1 + 12 / 1024: 0x3F82, 1 + 9 / 1024: 0x3F81, 65504.0: 0x4780,
            -3.0: 0xC040, 7.0: 0x40E0}
    rows = vals[np.arange(300 * 128).reshape(300, 128) % len(vals)]
    bf = np.vectorize(lambda v: want[float(v)])(rows).astype(np.uint16)
    t = O.tail_store_from_cache(rows, 130, 2)
    assert np.array_equal(t[0], bf[:128])
    assert np.array_equal(t[1, :2], bf[128:130]) and not t[1, 2:].any()
    t1 = O.tail_store_from_cache(rows, 128, 1)
    assert np.array_equal(t1[0], bf[:128])
    # fewer pages than slots: the leading slots stay zero
    t3 = O.tail_store_from_cache(rows, 5, 2)
    assert not t3[0].any() and np.array_equal(t3[1, :5], bf[:5]) and not t3[1, 5:].any()

