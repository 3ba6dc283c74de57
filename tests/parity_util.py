"""Stage-by-stage comparison of the HIP path with the oracle, one unit at a time.

Tolerances (the oracle is float64):
  pack           bit-exact bytes (key copy, projected keys, 4-bit value store)
  block scores   |gpu - oracle| <= 8e-6 * A + 1e-6, A = sigma * (s_t * sum|q| |dequant k|
                 + sum |q| |c|) maximised over the block: FP32 accumulation of at
                 most 130 exactly formed products (error <= 130 * 2^-24 * A)
  token scores   same form with A = sigma * sum_j |p_j| |kproj_j| (float32 p = P^T qbar)
  selection      integer work: the oracle's selection run on the GPU's own scores
                 must equal the GPU's bit for bit; against the oracle's scores the
                 two may differ only on entries whose oracle score lies within
                 1e-4 relative of the boundary score
  attention      max |O_gpu - O_oracle| <= 2e-3 and |lse_gpu - lse_oracle| <= 2e-3,
                 both sides on the GPU's selection
  cluster index  offsets and members bit-exact; centroids (FP32 sums of up to a few
                 hundred FP16 keys) within 1e-5 of the max |key| plus 1e-5 relative
  cluster scores |gpu - oracle| <= 2e-5 * A + 1e-6, A = sigma * max_h sum |q_h| |centroid|
                 (the GPU scores its own FP32 centroids)
  cluster choice bit-exact on the GPU's own scores; against the oracle's scores the
                 rankings may part only between blocks whose scores lie within 1e-4
                 relative of each other
"""

from __future__ import annotations

import numpy as np

from oracle import decode as O
from oracle import nvfp4

SCORE_REL = 8e-6
SCORE_ABS = 1e-6
BOUNDARY_REL = 1e-4
OUT_TOL = 2e-3


def q_group(w, b, h):
    G = w.spec.group
    return w.q[b, h * G:(h + 1) * G]


def scan_q(w, b, h):
    """The query the block scan scores with (the FP16 query, or its NVFP4 form)."""
    return O.scan_query(q_group(w, b, h), w.spec.query_fmt)


def check_pack_block(w, b, h, codes_gpu, scales_gpu):
    nb = w.spec.max_blocks
    rc, rs = O.pack_unit_blocks(w.k[b, h], w.key_center[h], w.global_scale[h], 0, nb)
    assert np.array_equal(codes_gpu, rc), f"code bytes differ at unit {(b, h)}: " \
        f"{int((codes_gpu != rc).sum())} of {rc.size}"
    assert np.array_equal(scales_gpu, rs), f"scale bytes differ at unit {(b, h)}"
    return rc, rs


def check_pack_token(w, b, h, kproj_gpu, tokens=None):
    fmt = w.spec.proj_fmt
    k = w.k[b, h] if tokens is None else w.k[b, h][tokens]
    ref = O.project_keys(k, w.proj[h], fmt)
    got = kproj_gpu if tokens is None else kproj_gpu[tokens]
    got = got.view(ref.dtype)
    assert np.array_equal(got, ref), \
        f"kproj differs at unit {(b, h)}: {int((got != ref).sum())} entries"
    return ref


def store_views(d):
    """The 4-bit value store of a DeviceStep as (codes [B, Hkv, T, 64], scales
    [B, Hkv, T, 8], s_v [Hkv]) device views (the buffer layout of bsa_value_store_size)."""
    s = d.w.spec
    R = s.batch * s.kv_heads * s.max_tokens
    codes = d.v[:64 * R].view(s.batch, s.kv_heads, s.max_tokens, 64)
    scales = d.v[64 * R:72 * R].view(s.batch, s.kv_heads, s.max_tokens, 8)
    s_v = d.v[72 * R:72 * R + 4 * s.kv_heads].view(torch_float32())
    return codes, scales, s_v


def torch_float32():
    import torch

    return torch.float32


def oracle_value_store(w, b, h):
    """(code bytes, scale bytes, s_v) of one unit's values, packed by the oracle."""
    s_v = np.float32(w.value_scale[h])
    cb, sb = O.pack_values(w.v[b, h], s_v)
    return cb, sb, s_v


def check_pack_values(w, b, h, codes_gpu, scales_gpu, s_v_gpu):
    cb, sb, s_v = oracle_value_store(w, b, h)
    assert np.float32(s_v_gpu) == s_v, f"value store scale differs at {(b, h)}"
    assert np.array_equal(codes_gpu, cb), f"value code bytes differ at unit {(b, h)}: " \
        f"{int((codes_gpu != cb).sum())} of {cb.size}"
    assert np.array_equal(scales_gpu, sb), f"value scale bytes differ at unit {(b, h)}"
    return cb, sb, s_v


def block_score_bound(w, b, h, rc, rs):
    """Per-block magnitude A of the estimated logits (see the module docstring)."""
    nb = w.spec.max_blocks
    qg = np.abs(scan_q(w, b, h))
    deq = np.abs(O.dequant_blocks(rc, rs)).reshape(nb, 128, 128)
    sigma = w.softmax_scale
    a = sigma * (float(w.global_scale[h]) * (deq @ qg.T) +
                 (qg @ np.abs(w.key_center[h].astype(np.float64)))[None, None, :])
    return a.reshape(nb, -1).max(axis=1)


def check_block_scores(w, b, h, scores_gpu, rc, rs):
    s = w.spec
    ref = O.scan_block_unit(scan_q(w, b, h), rc, rs, w.global_scale[h], w.key_center[h],
                            int(w.seq_lens[b]), s.n_tail, w.softmax_scale, s.max_blocks)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(scores_gpu)), f"-inf pattern differs at {(b, h)}"
    assert np.all(scores_gpu[~fin] == -np.inf)
    A = block_score_bound(w, b, h, rc, rs)
    err = np.abs(scores_gpu[fin].astype(np.float64) - ref[fin])
    lim = SCORE_REL * A[fin] + SCORE_ABS
    assert np.all(err <= lim), f"block scores at {(b, h)}: max err {err.max():.3e}, " \
        f"worst ratio {(err / lim).max():.2f}"
    return ref


def check_token_scores(w, b, h, scores_gpu, kproj_ref):
    fmt = w.spec.proj_fmt
    ref = O.scan_token_unit(q_group(w, b, h), kproj_ref, w.proj[h], int(w.seq_lens[b]),
                            w.softmax_scale, fmt)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(scores_gpu))
    qbar = np.abs(q_group(w, b, h).astype(np.float64)).mean(axis=0)
    p = np.abs(w.proj[h].astype(np.float64)).T @ qbar
    A = w.softmax_scale * (np.abs(O.proj_values(kproj_ref, fmt)) @ p)
    err = np.abs(scores_gpu[fin].astype(np.float64) - ref[fin])
    lim = SCORE_REL * A[fin] + SCORE_ABS
    assert np.all(err <= lim), f"token scores at {(b, h)}: max err {err.max():.3e}"
    return ref


def check_selection(w, b, h, idx_gpu, count_gpu, scores_gpu, scores_ref):
    s = w.spec
    L = int(w.seq_lens[b])
    if s.granularity == "block":
        exact_idx, exact_cnt = O.select_blocks_unit(scores_gpu.astype(np.float64), L, s.n_tail,
                                                    s.budget)
        ref_idx, ref_cnt = O.select_blocks_unit(scores_ref, L, s.n_tail, s.budget)
        picks = s.budget - s.n_tail
    elif s.top_p > 0:
        n = check_top_p_selection(scores_gpu, L, s.budget, s.top_p, idx_gpu, count_gpu)
        check_top_p_against_oracle(scores_ref, L, s.budget, s.top_p, idx_gpu, count_gpu)
        return n
    else:
        exact_idx, exact_cnt = O.select_tokens_unit(scores_gpu.astype(np.float64), L, s.budget)
        ref_idx, ref_cnt = O.select_tokens_unit(scores_ref, L, s.budget)
        picks = s.budget
    assert int(count_gpu) == exact_cnt == ref_cnt, (b, h, int(count_gpu), exact_cnt, ref_cnt)
    assert np.array_equal(idx_gpu, exact_idx), f"selection on the GPU's scores differs at {(b, h)}"
    got = set(int(x) for x in idx_gpu[:exact_cnt])
    exp = set(int(x) for x in ref_idx[:ref_cnt])
    diff = got ^ exp
    if diff:
        cand = scores_ref[np.isfinite(scores_ref)]
        tau = np.sort(cand)[::-1][min(picks, cand.size) - 1]
        for x in diff:
            assert abs(scores_ref[x] - tau) <= BOUNDARY_REL * abs(tau), \
                f"selection differs beyond the boundary band at {(b, h)}: entry {x}"
    return len(diff)


# The adaptive budget's cut is a count decided by float sums (float32 on the
# GPU, float64 in the oracle): a count is accepted when the oracle's shares of
# its prefix lie within TOP_P_REL of top_p on the right sides; the set must then
# be exactly the oracle's top-count set.
TOP_P_REL = 1e-4


def check_top_p_selection(scores_gpu, L, budget, top_p, idx_gpu, count_gpu):
    """Adaptive-budget selection on the GPU's own scores (one unit)."""
    s = np.asarray(scores_gpu, dtype=np.float64)
    n = min(int(L), s.shape[0])
    picks = max(0, min(int(budget), n))
    m = int(count_gpu)
    assert 0 <= m <= picks, (m, picks)
    top_idx, top_cnt = O.select_tokens_unit(s, L, m) if m > 0 else (np.zeros(0, np.int32), 0)
    assert top_cnt == m
    assert np.array_equal(idx_gpu[:m], top_idx[:m]), "the kept tokens are not the top-ranked ones"
    assert np.all(idx_gpu[m:] == -1), "padding"
    ref_idx, ref_m = O.select_tokens_top_p(s, L, budget, top_p)
    if m == ref_m:
        assert np.array_equal(idx_gpu, ref_idx)
        return 0
    w = O.token_weights(s[:n])
    z = w.sum()
    assert z > 0 and np.isfinite(z), "the fixed budget applies when nothing has weight"
    order = np.lexsort((np.arange(n), -s[:n]))
    cum = np.cumsum(w[order[:picks]]) / z
    assert m == picks or cum[m - 1] >= top_p * (1 - TOP_P_REL), (m, ref_m, cum[m - 1], top_p)
    assert m == 1 or cum[m - 2] < top_p * (1 + TOP_P_REL), (m, ref_m, cum[m - 2], top_p)
    return abs(m - ref_m)


def check_top_p_against_oracle(scores_ref, L, budget, top_p, idx_gpu, count_gpu):
    """Adaptive-budget selection against the oracle's float64 scores (one unit).

    The kept count m is accepted when the oracle's shares (softmax weights of
    its own scores, ranked by them) of the top m reach top_p within TOP_P_REL
    and those of the top m - 1 do not; the kept set may differ from the
    oracle's top-m set only on tokens whose oracle score lies within
    BOUNDARY_REL of the oracle's m-th score, as for a fixed budget."""
    s = np.asarray(scores_ref, dtype=np.float64)
    n = min(int(L), s.shape[0])
    picks = max(0, min(int(budget), n))
    m = int(count_gpu)
    w = O.token_weights(s[:n])
    z = w.sum()
    if not (z > 0 and np.isfinite(z)):
        assert m == picks, "the fixed budget applies when nothing has weight"
        return
    order = np.lexsort((np.arange(n), -s[:n]))
    cum = np.cumsum(w[order[:picks]]) / z
    assert 1 <= m <= picks, (m, picks)
    assert m == picks or cum[m - 1] >= top_p * (1 - TOP_P_REL), (m, cum[m - 1], top_p)
    assert m == 1 or cum[m - 2] < top_p * (1 + TOP_P_REL), (m, cum[m - 2], top_p)
    got = set(int(x) for x in idx_gpu[:m])
    exp = set(int(x) for x in order[:m])
    tau = s[order[m - 1]]
    for x in got ^ exp:
        assert abs(s[x] - tau) <= BOUNDARY_REL * abs(tau), \
            f"adaptive selection differs beyond the boundary band: token {x}"


def oracle_partials(w, b, h, idx, splits, v_store=None):
    """The oracle's split partials on the given selection; v_store = the unit's
    (code bytes, scale bytes, s_v) when the values come from the 4-bit store."""
    s = w.spec
    L = int(w.seq_lens[b])
    qg = q_group(w, b, h)
    if s.value_fmt == "nvfp4" and v_store is None:
        v_store = oracle_value_store(w, b, h)
    if s.granularity == "block":
        tk = w.tail_k[b, h] if s.n_tail else None
        tv = w.tail_v[b, h] if s.n_tail else None
        rows = lambda sel: O.gather_rows_block(w.k[b, h], w.v[b, h], sel, L, s.n_tail, tk, tv,
                                               v_store=v_store)
    else:
        rows = lambda sel: O.gather_rows_token(w.k[b, h], w.v[b, h],
                                               [t for t in sel if t < L], v_store=v_store)
    return O.attend_splits(qg, np.asarray(idx), splits, rows, w.softmax_scale)


def check_attention(w, b, h, idx_gpu, splits, part_o_gpu, part_lse_gpu, out_gpu, lse_gpu,
                    v_store=None):
    """part_o_gpu [G, S, D], part_lse_gpu [G, S], out_gpu [G, D], lse_gpu [G]."""
    po, pl = oracle_partials(w, b, h, idx_gpu, splits, v_store)  # [S, G, D], [S, G]
    o, lse = O.combine(po, pl)
    fin = np.isfinite(pl)
    assert np.array_equal(fin, np.isfinite(part_lse_gpu.T)), f"empty splits differ at {(b, h)}"
    assert np.abs(part_lse_gpu.T[fin] - pl[fin]).max(initial=0) <= OUT_TOL
    assert np.abs(np.transpose(part_o_gpu, (1, 0, 2)) - po).max() <= OUT_TOL
    err = np.abs(out_gpu - o).max()
    assert err <= OUT_TOL, f"output error {err:.3e} at {(b, h)}"
    lf = np.isfinite(lse)
    assert np.array_equal(lf, np.isfinite(lse_gpu))
    assert np.abs(lse_gpu[lf] - lse[lf]).max(initial=0) <= OUT_TOL
    return err


def check_cluster_index(w, b, h, cent_gpu, off_gpu, mem_gpu):
    s = w.spec
    cent, off, mem = O.cluster_index(w.k[b, h], w.assign[b, h], s.n_clusters, int(w.seq_lens[b]))
    assert np.array_equal(off_gpu, off), f"cluster offsets differ at {(b, h)}"
    assert np.array_equal(mem_gpu[:off[-1]], mem), f"cluster members differ at {(b, h)}"
    kmax = float(np.abs(w.k[b, h].astype(np.float64)).max())
    err = np.abs(cent_gpu.astype(np.float64) - cent)
    assert np.all(err <= 1e-5 * kmax + 1e-5 * np.abs(cent)), \
        f"centroids at {(b, h)}: max err {err.max():.3e}"
    return cent, off, mem


def check_cluster_scores(w, b, h, scores_gpu, cent, off):
    sizes = np.diff(off)
    ref = O.cluster_scores(q_group(w, b, h), cent, sizes, w.softmax_scale)
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(scores_gpu)), f"-inf pattern differs at {(b, h)}"
    A = w.softmax_scale * (np.abs(cent) @ np.abs(q_group(w, b, h).astype(np.float64)).T).max(axis=1)
    err = np.abs(scores_gpu[fin].astype(np.float64) - ref[fin])
    lim = 2e-5 * A[fin] + 1e-6
    assert np.all(err <= lim), f"cluster scores at {(b, h)}: worst ratio {(err / lim).max():.2f}"
    return ref


def check_cluster_choice(w, b, h, idx_gpu, count_gpu, scores_gpu, scores_ref, off, mem):
    s = w.spec
    sizes = np.diff(off)
    ch, tot = O.select_clusters(scores_gpu.astype(np.float64), sizes, s.budget)
    toks, n = O.cluster_tokens(ch, off, mem, s.budget)
    assert int(count_gpu) == n == tot, (b, h, int(count_gpu), n)
    assert np.array_equal(idx_gpu, toks), f"cluster choice on the GPU's scores differs at {(b, h)}"
    ch_ref, _ = O.select_clusters(scores_ref, sizes, s.budget)
    if not np.array_equal(ch, ch_ref):
        # the first rank where the two parts: its two blocks tie within 1e-4
        k = next(i for i in range(min(len(ch), len(ch_ref)) + 1)
                 if i >= len(ch) or i >= len(ch_ref) or ch[i] != ch_ref[i])
        pair = [c for c in (ch[k] if k < len(ch) else None, ch_ref[k] if k < len(ch_ref) else None)
                if c is not None]
        if len(pair) == 2:
            a, c = scores_ref[pair[0]], scores_ref[pair[1]]
            assert abs(a - c) <= BOUNDARY_REL * max(abs(a), abs(c)), \
                f"cluster ranking parts beyond the tie band at {(b, h)}"
    return n


def check_units(w, d, units=None):
    """Compare every stage of a DeviceStep with the oracle for the given units
    (all by default); w must hold the K and V the GPU holds. Device buffers are
    copied to the host one unit at a time."""
    s = w.spec
    G = s.group
    if units is None:
        units = [(b, h) for b in range(s.batch) for h in range(s.kv_heads)]
    host = lambda t: t.cpu().numpy()
    store = store_views(d) if s.value_fmt == "nvfp4" else None
    for b, h in units:
        v_store = None
        if store is not None:
            v_store = check_pack_values(w, b, h, host(store[0][b, h]), host(store[1][b, h]),
                                        host(store[2])[h])
        scores = host(d.scores[b, h])
        if s.granularity == "cluster":
            cent, off, mem = check_cluster_index(w, b, h, host(d.centroids[b, h]),
                                                 host(d.offsets[b, h]), host(d.members[b, h]))
            ref = check_cluster_scores(w, b, h, scores, cent, off)
            check_cluster_choice(w, b, h, host(d.idx[b, h]), host(d.count[b, h]), scores, ref,
                                 off, mem)
            rows = slice(h * G, (h + 1) * G)
            check_attention(w, b, h, host(d.idx[b, h]), d.splits, host(d.part_o[b, rows]),
                            host(d.part_lse[b, rows]), host(d.out[b, rows]),
                            host(d.out_lse[b, rows]), v_store)
            continue
        if s.granularity == "block":
            rc, rs = check_pack_block(w, b, h, host(d.codes[b, h]), host(d.scales[b, h]))
            ref = check_block_scores(w, b, h, scores, rc, rs)
        else:
            kref = check_pack_token(w, b, h, host(d.kproj[b, h]))
            ref = check_token_scores(w, b, h, scores, kref)
        check_selection(w, b, h, host(d.idx[b, h]), host(d.count[b, h]), scores, ref)
        rows = slice(h * G, (h + 1) * G)
        check_attention(w, b, h, host(d.idx[b, h]), d.splits, host(d.part_o[b, rows]),
                        host(d.part_lse[b, rows]), host(d.out[b, rows]), host(d.out_lse[b, rows]),
                        v_store)


STEP_OUT = ("scores", "idx", "count", "part_o", "part_lse", "out", "out_lse")


def check_forms_match(d):
    """score_select + attend_combine, score_scan + select_attend_combine, and
    decode_step reproduce the four calls' bits (and leave every counter at
    zero); d has just run the four calls."""
    import torch

    host = lambda t: t.cpu().numpy()
    ref = [host(getattr(d, n)).copy() for n in STEP_OUT]
    for run in (d.run_fused, d.run_two, d.decode_step):
        for n in STEP_OUT:
            getattr(d, n).fill_(7)
        run()
        torch.cuda.synchronize()
        for n, a in zip(STEP_OUT, ref):
            assert np.array_equal(a, host(getattr(d, n)), equal_nan=True), (run.__name__, n)
        assert int(d.counters.abs().sum()) == 0
