"""Parity of the HIP path (through the C ABI) with the CPU oracle, stage by stage.

Every workload runs at a reduced size where the oracle checks every unit
(several tiles, ragged tails) and, in test_gpu_full_size.py, at its full size
on sampled units. Edge cases: empty and sub-block sequences, one tail page,
query-group sizes 1..16, a BF16 cache, exact score ties, all-equal scores,
budgets at and above the candidate count, one split and one split per entry.
"""

import dataclasses
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from block_sparse_attention_pack_amd import workloads as W
from block_sparse_attention_pack_amd.step import upload

import parity_util as PU

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_sparse_attention_pack_amd import binding

    binding.load()  # fails loudly when the library is missing


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_step(w, splits=None, kv_dtype="f16"):
    d = upload(w, splits=splits, kv_dtype=kv_dtype)
    d.pack()
    d.run()
    torch.cuda.synchronize()
    return d


def host(t):
    return t.cpu().numpy()


def check_all(w, d, units=None):
    PU.check_units(w, d, units)


REDUCED = {
    "tiny": W.SPECS["tiny"],
    "llama8b": W.reduced("llama8b", 8192),
    "jetqsparse": W.reduced("jetqsparse", 8192, batch=2),
    "ragged": W.reduced("ragged", 16384, batch=3, budget=24),
    "token": W.reduced("token", 16384, batch=2),
    "token_fp8": W.reduced("token_fp8", 16384, batch=2),
    "jetqsparse_q4": W.reduced("jetqsparse_q4", 8192, batch=2),
    "token_topp": W.reduced("token_topp", 16384, batch=2),
}


@pytest.mark.parametrize("name", list(REDUCED))
def test_reduced_workloads_match_oracle(name):
    spec = REDUCED[name]
    _say(f"[parity] {spec.name}")
    w = W.generate(spec)
    d = run_step(w)
    check_all(w, d)


@pytest.mark.parametrize("splits", [1, 3, 8])
def test_split_count_does_not_matter(splits):
    spec = W.reduced("jetqsparse", 4096, batch=1, budget=8)
    w = W.generate(spec)
    d = run_step(w, splits=splits)
    check_all(w, d)


@pytest.mark.parametrize("G", [1, 2, 8, 16])
def test_query_group_sizes(G):
    spec = dataclasses.replace(W.SPECS["tiny"], name=f"group{G}", seed=20 + G, batch=2,
                               kv_heads=2, q_heads=2 * G, max_tokens=2048, budget=5)
    w = W.generate(spec)
    d = run_step(w)
    check_all(w, d)
    _two_calls_match(d)
    tspec = dataclasses.replace(W.SPECS["token"], name=f"tgroup{G}", seed=30 + G, batch=1,
                                kv_heads=2, q_heads=2 * G, max_tokens=4096, budget=96)
    w = W.generate(tspec)
    d = run_step(w)
    check_all(w, d)
    _two_calls_match(d)


def _two_calls_match(d):
    PU.check_forms_match(d)


def test_select_attend_combine_above_the_in_kernel_budget():
    """Budgets above 1024 blocks (more than 4 candidates per selecting thread
    re-read from memory): same results in every form."""
    spec = dataclasses.replace(W.SPECS["jetqsparse"], name="big_budget", seed=90, batch=1,
                               kv_heads=1, q_heads=4, max_tokens=1280 * 128, budget=1100,
                               needle_count=5, key_offset_std=0.0)
    w = W.generate(spec)
    d = run_step(w, splits=8)
    check_all(w, d)
    _two_calls_match(d)


def test_short_and_empty_sequences_with_tail_pages():
    lengths = (0, 1, 127, 128, 129, 300, 2000, 4096)
    for n_tail in (0, 1, 2):
        spec = dataclasses.replace(W.SPECS["ragged"], name=f"short{n_tail}", seed=40 + n_tail,
                                   batch=len(lengths), kv_heads=2, q_heads=8, max_tokens=4096,
                                   budget=6, n_tail=n_tail, needle_count=2, lengths=lengths)
        _say(f"[parity] {spec.name}")
        w = W.generate(spec)
        d = run_step(w)
        check_all(w, d)
        cnt = host(d.count)
        assert np.all(cnt[0] == 0)  # empty sequence: nothing selected, output 0, lse -inf
        assert np.all(host(d.out)[0] == 0) and np.all(host(d.out_lse)[0] == -np.inf)


def test_token_mode_ragged_lengths():
    lengths = (0, 5, 100, 4097, 8192)
    spec = dataclasses.replace(W.SPECS["token"], name="tok_ragged", seed=50, batch=len(lengths),
                               kv_heads=2, q_heads=8, max_tokens=8192, budget=256,
                               lengths=lengths)
    w = W.generate(spec)
    check_all(w, run_step(w))


def test_bf16_cache():
    spec = W.reduced("jetqsparse", 4096, batch=2, budget=10)
    w = W.generate(spec)
    d = run_step(w, kv_dtype="bf16")
    # the oracle sees the bf16-rounded keys and values the GPU holds
    w16 = dataclasses.replace(w, k=host(d.k.float()), v=host(d.v.float()))
    check_all(w16, d)


def test_exact_ties_go_to_the_lower_index():
    spec = dataclasses.replace(W.SPECS["tiny"], name="ties", seed=60, needle_count=0, budget=3)
    w = W.generate(spec)
    k = w.k.copy()
    qm = w.q[0].astype(np.float64).mean(axis=0)
    k[0, 0, 5 * 128:6 * 128] += (3.0 * qm / np.linalg.norm(qm)).astype(np.float16)
    # blocks 3, 9, 20 and 30 become copies of block 5: five identical top scores
    for dst in (3, 9, 20, 30):
        k[0, 0, dst * 128:(dst + 1) * 128] = k[0, 0, 5 * 128:6 * 128]
    w = dataclasses.replace(w, k=k)
    d = run_step(w)
    sc = host(d.scores)[0, 0]
    assert len(set(sc[[3, 5, 9, 20, 30]])) == 1 and sc[5] == sc.max()
    assert list(host(d.idx)[0, 0]) == [3, 5, 9]
    check_all(w, d)


@pytest.mark.parametrize("name", ["tiny", "token"])
def test_all_equal_scores_take_lowest_indices(name):
    base = W.SPECS["tiny"] if name == "tiny" else W.reduced("token", 4096, batch=1)
    w = W.generate(base)
    w = dataclasses.replace(w, q=np.zeros_like(w.q))
    d = run_step(w)
    s = w.spec
    picks = s.budget - s.n_tail
    assert list(host(d.idx)[0, 0][:picks]) == list(range(picks))
    check_all(w, d)


def test_budget_at_and_above_candidates():
    lengths = (128 * 5, 128 * 3 + 7)
    spec = dataclasses.replace(W.SPECS["ragged"], name="budget_all", seed=70, batch=2,
                               kv_heads=1, q_heads=4, max_tokens=2048, budget=8, n_tail=2,
                               needle_count=1, lengths=lengths)
    w = W.generate(spec)
    d = run_step(w, splits=8)
    check_all(w, d)
    assert list(host(d.count)[:, 0]) == [5, 4]
    # budget == n_tail: only the tail pages
    w2 = dataclasses.replace(w, spec=dataclasses.replace(spec, budget=2))
    d2 = run_step(w2, splits=2)
    check_all(w2, d2)
    assert list(host(d2.idx)[0, 0]) == [3, 4]


def test_budget_all_blocks_is_dense_attention():
    spec = dataclasses.replace(W.SPECS["tiny"], name="dense", budget=32)
    w = W.generate(spec)
    d = run_step(w, splits=4)
    check_all(w, d)
    q = torch.from_numpy(w.q[0].astype(np.float64))
    k = torch.from_numpy(w.k[0, 0].astype(np.float64))
    v = torch.from_numpy(w.v[0, 0].astype(np.float64))
    ref = torch.softmax(w.softmax_scale * q @ k.T, dim=-1) @ v
    assert np.abs(host(d.out)[0] - ref.numpy()).max() <= PU.OUT_TOL


def test_repeat_runs_are_bitwise_identical():
    w = W.generate(W.reduced("ragged", 8192, batch=2, budget=12))
    d = run_step(w)
    first = [host(t).copy() for t in (d.scores, d.idx, d.count, d.part_o, d.out, d.out_lse)]
    for _ in range(3):
        d.run()
        torch.cuda.synchronize()
        again = [host(t) for t in (d.scores, d.idx, d.count, d.part_o, d.out, d.out_lse)]
        for a, b in zip(first, again):
            assert np.array_equal(a, b, equal_nan=True)


@pytest.mark.parametrize("name", list(REDUCED))
def test_fused_calls_match_the_four_calls(name):
    """score_select + attend_combine, and score_scan + select_attend_combine,
    give the four calls' bits, call after call."""
    w = W.generate(REDUCED[name])
    d = run_step(w)
    ref = [host(t).copy() for t in (d.scores, d.idx, d.count, d.out, d.out_lse)]
    for t in (d.scores, d.idx, d.count, d.out, d.out_lse):
        t.fill_(7)
    for run in (d.run_fused, d.run_two, d.decode_step):
        for rep in range(3):  # the arrival counters must return to zero every call
            for t in (d.idx, d.count, d.out, d.out_lse):
                t.fill_(7)
            run()
            torch.cuda.synchronize()
            got = [host(t) for t in (d.scores, d.idx, d.count, d.out, d.out_lse)]
            for a, b in zip(ref, got):
                assert np.array_equal(a, b, equal_nan=True), (name, run.__name__, rep)
            assert int(d.counters.abs().sum()) == 0
    check_all(w, d)


def test_fused_calls_with_short_sequences_and_many_splits():
    lengths = (0, 1, 129, 300, 2000, 4096)
    spec = dataclasses.replace(W.SPECS["ragged"], name="fused_short", seed=80, batch=len(lengths),
                               kv_heads=2, q_heads=8, max_tokens=4096, budget=12, n_tail=2,
                               needle_count=2, lengths=lengths)
    w = W.generate(spec)
    for splits in (6, 12):
        d = upload(w, splits=splits)
        d.pack()
        d.run_fused()
        torch.cuda.synchronize()
        check_all(w, d)
        d.run_two()
        torch.cuda.synchronize()
        check_all(w, d)


@pytest.mark.parametrize("splits", [8, 9, 16, 17, 32, 33, 48])
def test_attend_combine_on_both_sides_of_the_merge_limit(splits):
    """Up to 8 splits the merge runs in the attention launch, beyond in its own
    launch: the same bits either way."""
    w = W.generate(W.reduced("ragged", 16384, batch=2, budget=48))
    d = run_step(w, splits=splits)
    ref = [host(t).copy() for t in (d.out, d.out_lse)]
    for t in (d.out, d.out_lse):
        t.fill_(7)
    for rep in range(2):
        d.attend_combine()
        torch.cuda.synchronize()
        for a, b in zip(ref, (host(d.out), host(d.out_lse))):
            assert np.array_equal(a, b, equal_nan=True), (splits, rep)
        assert int(d.counters.abs().sum()) == 0
    check_all(w, d)


def test_decode_step_with_short_sequences_tails_and_many_splits():
    """The whole step: empty, sub-block and ragged sequences, 0-2 tail pages, and
    split counts on both sides of the in-kernel merge, call after call."""
    lengths = (0, 1, 129, 300, 2000, 4096)
    for n_tail in (0, 2):
        spec = dataclasses.replace(W.SPECS["ragged"], name=f"step_short{n_tail}", seed=85 + n_tail,
                                   batch=len(lengths), kv_heads=2, q_heads=8, max_tokens=4096,
                                   budget=12, n_tail=n_tail, needle_count=2, lengths=lengths)
        w = W.generate(spec)
        for splits in (1, 6, 12):
            _say(f"[parity] {spec.name} splits {splits}")
            d = run_step(w, splits=splits)
            _two_calls_match(d)
            _two_calls_match(d)
            check_all(w, d)


def test_decode_step_bf16_cache_and_large_group():
    for G, kv_dtype in ((4, "bf16"), (16, "f16")):
        spec = dataclasses.replace(W.reduced("jetqsparse", 8192, batch=2), name=f"step_g{G}",
                                   seed=95 + G, q_heads=4 * G)
        w = W.generate(spec)
        d = run_step(w, kv_dtype=kv_dtype)
        _two_calls_match(d)
        # the oracle sees the keys and values the GPU holds
        check_all(dataclasses.replace(w, k=host(d.k.float()), v=host(d.v.float())), d)


@pytest.mark.parametrize("splits", [16, 32, 64])
def test_decode_step_merges_many_splits(splits):
    """More splits than the attention launch merges itself: the merge launch
    gives the four calls' bits."""
    spec = W.reduced("jetqsparse", 16384, batch=2, budget=64)
    w = W.generate(spec)
    d = run_step(w, splits=splits)
    _two_calls_match(d)
    check_all(w, d)


def test_fp8_projected_cache_decodes_every_code():
    """The scan widens every finite E4M3 code exactly: crafted cache rows, token t
    holding code t (NaN codes replaced by 0) in every column, against the oracle."""
    spec = dataclasses.replace(W.SPECS["token_fp8"], name="fp8_codes", batch=1, kv_heads=1,
                               q_heads=4, max_tokens=512, budget=32)
    w = W.generate(spec)
    d = run_step(w)
    codes = np.arange(512, dtype=np.int64) % 256
    codes[(codes == 0x7F) | (codes == 0xFF)] = 0
    rows = np.repeat(codes.astype(np.uint8)[:, None], spec.rank, axis=1)
    d.kproj[0, 0].copy_(torch.from_numpy(rows))
    d.scan()
    torch.cuda.synchronize()
    PU.check_token_scores(w, 0, 0, host(d.scores[0, 0]), rows)



APPEND_CASES = {
    # name: (spec, cache dtype)
    "block": (dataclasses.replace(W.SPECS["ragged"], name="append_block", seed=111, batch=5,
                                  kv_heads=2, q_heads=8, max_tokens=2048, budget=8, n_tail=0,
                                  needle_count=2, lengths=(0, 127, 250, 1900, 2048)), "f16"),
    "block_tail1": (dataclasses.replace(W.SPECS["ragged"], name="append_tail1", seed=112, batch=5,
                                        kv_heads=2, q_heads=8, max_tokens=2048, budget=8,
                                        n_tail=1, needle_count=2,
                                        lengths=(0, 127, 250, 1900, 2048)), "f16"),
    "block_tail2_bf16": (dataclasses.replace(W.SPECS["ragged"], name="append_tail2", seed=113,
                                             batch=5, kv_heads=2, q_heads=8, max_tokens=2048,
                                             budget=8, n_tail=2, needle_count=2,
                                             lengths=(0, 127, 250, 1900, 2048)), "bf16"),
    "token": (dataclasses.replace(W.SPECS["token"], name="append_token", seed=114, batch=3,
                                  kv_heads=2, q_heads=8, max_tokens=2048, budget=256,
                                  lengths=(0, 1000, 2000)), "f16"),
    "token_fp8": (dataclasses.replace(W.SPECS["token_fp8"], name="append_fp8", seed=115, batch=3,
                                      kv_heads=2, q_heads=8, max_tokens=2048, budget=256,
                                      lengths=(0, 1000, 2000)), "f16"),
    # the 4-bit value store: appended values packed into it (tail pages still BF16)
    "block_tail2_v4": (dataclasses.replace(W.SPECS["ragged"], name="append_tail2_v4", seed=116,
                                           batch=5, kv_heads=2, q_heads=8, max_tokens=2048,
                                           budget=8, n_tail=2, needle_count=2,
                                           lengths=(0, 127, 250, 1900, 2048),
                                           value_fmt="nvfp4"), "f16"),
    "token_v4_bf16": (dataclasses.replace(W.SPECS["token"], name="append_token_v4", seed=117,
                                          batch=3, kv_heads=2, q_heads=8, max_tokens=2048,
                                          budget=256, lengths=(0, 1000, 2000),
                                          value_fmt="nvfp4"), "bf16"),
}


@pytest.mark.parametrize("case", list(APPEND_CASES))
def test_append_tokens_match_the_bulk_build(case):
    """bsa_append_token, one call per decode step, from lengths that start empty,
    inside a page, at a page edge and full (page starts, tail shifts, sequences
    that fill up on the way): the cache rows, the key copy and the BF16 tail
    store end bit-identical to the oracle's build of the final cache, and a step
    on the appended cache matches the oracle."""
    from oracle import decode as O

    spec, kv_dtype = APPEND_CASES[case]
    w = W.generate(spec)
    d = upload(w, kv_dtype=kv_dtype)
    d.pack()
    B, Hkv, T, nt = spec.batch, spec.kv_heads, spec.max_tokens, spec.n_tail
    lens = np.asarray(w.seq_lens, dtype=np.int64).copy()
    k_exp = d.k.cpu().clone()  # the cache dtype
    v_exp = (d.v_src if d.value_store else d.v).cpu().clone()
    if nt:  # the tail store the appends keep up: BF16 pages of the cache rows
        kf, vf = k_exp.float().numpy(), v_exp.float().numpy()
        for name, rows in (("tail_k", kf), ("tail_v", vf)):
            st = np.stack([np.stack([O.tail_store_from_cache(rows[b, h], int(lens[b]), nt)
                                     for h in range(Hkv)]) for b in range(B)])
            getattr(d, name).copy_(torch.from_numpy(st.view(np.int16)))
    n_app = 300
    rng = np.random.default_rng([spec.seed, 7])
    dt = d.k.dtype
    k_new = torch.from_numpy(rng.standard_normal((n_app, B, Hkv, 128), dtype=np.float32)).to(dt)
    v_new = torch.from_numpy(rng.standard_normal((n_app, B, Hkv, 128), dtype=np.float32)).to(dt)
    k_new_d, v_new_d = k_new.cuda(), v_new.cuda()
    _say(f"[append] {case}: {n_app} tokens from lengths {lens.tolist()}")
    for i in range(n_app):
        d.append(k_new_d[i], v_new_d[i])
        for b in range(B):
            if lens[b] < T:
                k_exp[b, :, lens[b]] = k_new[i, b]
                v_exp[b, :, lens[b]] = v_new[i, b]
        lens = np.minimum(lens + 1, T)
        d.seq_lens.add_(1).clamp_(max=T)
    torch.cuda.synchronize()
    assert np.array_equal(host(d.seq_lens), lens)
    assert torch.equal(d.k.cpu(), k_exp)
    if not d.value_store:
        assert torch.equal(d.v.cpu(), v_exp)
    kf, vf = k_exp.float().numpy(), v_exp.float().numpy()
    store = PU.store_views(d) if d.value_store else None
    for b in range(B):
        for h in range(Hkv):
            if store is not None:
                # every row of the store: the appended ones and those the bulk pack wrote
                PU.check_pack_values(dataclasses.replace(w, v=vf), b, h, host(store[0][b, h]),
                                     host(store[1][b, h]), host(store[2])[h])
            if spec.granularity == "block":
                # every token's records: the appended ones and those the bulk pack wrote
                PU.check_pack_block(dataclasses.replace(w, k=kf), b, h, host(d.codes[b, h]),
                                    host(d.scales[b, h]))
            else:
                PU.check_pack_token(dataclasses.replace(w, k=kf), b, h, host(d.kproj[b, h]))
            if nt:
                for name, rows in (("tail_k", kf), ("tail_v", vf)):
                    exp = O.tail_store_from_cache(rows[b, h], int(lens[b]), nt)
                    got = host(getattr(d, name)[b, h]).view(np.uint16)
                    assert np.array_equal(got, exp), f"{name} differs at {(b, h)}"
    # a decode step on the appended cache
    tails = {}
    if nt:
        tails = dict(tail_k=host(d.tail_k).view(np.uint16), tail_v=host(d.tail_v).view(np.uint16))
    w2 = dataclasses.replace(w, k=kf, v=vf, seq_lens=lens.astype(np.int32), **tails)
    d.run()
    torch.cuda.synchronize()
    check_all(w2, d)


def test_nvfp4_query_reads_back_every_element():
    """The scan's NVFP4 query, element by element: block i of a unit holds the
    one-hot key e_i (center 0), so block score i is a positive multiple of
    qtilde_i. Head 0 puts elements on every E2M1 tie and spreads the group scales
    over normal and subnormal E4M3 codes; head 1 is all zeros."""
    T = 128 * 128
    spec = dataclasses.replace(W.SPECS["jetqsparse_q4"], name="q4_elements", batch=1, kv_heads=2,
                               q_heads=2, max_tokens=T, budget=8, needle_count=0,
                               key_offset_std=0.0)
    w = W.generate(spec)
    k = np.zeros((1, 2, T, 128), np.float16)
    for i in range(128):
        k[0, :, i * 128:(i + 1) * 128, i] = 1.0
    # head 0: s_q = 2^-12 (group 5 at scale 448 holds the largest 6); in units of
    # its group's scale, every group holds a 6 and the E2M1 ties
    x = np.array([6, -0.25, 0.75, -1.25, 1.75, 2.5, -3.5, 5, 0.375, 1, -1.5, 2, 3, 4.5, -6, 0])
    scale_codes = [0x7D, 0x40, 0x31, 0x03, 0x09, 0x7E, 0x22, 0x58]
    from oracle import nvfp4
    q = np.zeros((1, 2, 128), np.float64)
    for g, code in enumerate(scale_codes):
        q[0, 0, 16 * g:16 * (g + 1)] = np.roll(x, g) * nvfp4.e4m3_value(code) * 2.0 ** -12
    q16 = q.astype(np.float16)
    assert np.array_equal(q16.astype(np.float64), q)  # exact in fp16
    st = np.full(2, np.float32(1.0) / np.float32(2688.0), np.float32)
    w2 = dataclasses.replace(w, k=k, q=q16, key_center=np.zeros((2, 128), np.float32),
                             global_scale=st)
    d = run_step(w2)
    check_all(w2, d)
    got = host(d.scores[0, 0]).astype(np.float64)
    qt = PU.scan_q(w2, 0, 0)[0]
    assert np.all(np.sign(got) == np.sign(qt))
    assert np.allclose(got, got[np.argmax(qt)] / qt.max() * qt, rtol=1e-6, atol=0)
    assert np.array_equal(host(d.scores[0, 1]), np.zeros(128, np.float32))


@pytest.mark.parametrize("G", [1, 2, 8, 16])
def test_nvfp4_query_group_sizes(G):
    """The NVFP4 query staged by 16 threads per head, from 1 to 16 heads per KV
    head (all 256 threads at 16): scores against the oracle's quantized query,
    and the combined calls give the four calls' bits."""
    spec = dataclasses.replace(W.SPECS["jetqsparse_q4"], name=f"q4group{G}", seed=120 + G, batch=2,
                               kv_heads=2, q_heads=2 * G, max_tokens=4096, budget=6,
                               needle_count=2)
    w = W.generate(spec)
    d = run_step(w)
    check_all(w, d)
    _two_calls_match(d)


@pytest.mark.parametrize("rank,fmt", [(8, "bf16"), (16, "bf16"), (64, "bf16"), (128, "bf16"),
                                      (16, "fp8"), (64, "fp8"), (128, "fp8")])
def test_token_mode_every_rank(rank, fmt):
    """The projected-key pack, scan and attention at every supported rank (a row
    of 16 to 256 bytes: 1 to 16 lanes per token), BF16 and FP8, ragged lengths."""
    spec = dataclasses.replace(W.SPECS["token"], name=f"rank{rank}{fmt}", seed=140 + rank,
                               batch=2, kv_heads=2, q_heads=8, max_tokens=8192, budget=160,
                               rank=rank, proj_fmt=fmt, lengths=(8192, 5003))
    w = W.generate(spec)
    d = run_step(w)
    check_all(w, d)
    _two_calls_match(d)


@pytest.mark.parametrize("name", ["ragged", "token"])
def test_token_major_interleaved_kv_layout(name):
    """K and V in one token-major buffer [B][T][2][Hkv][128] (head stride 128,
    token stride 2 * Hkv * 128): every stage through the layout's strides."""
    from block_sparse_attention_pack_amd import binding as bsa

    spec = REDUCED[name]
    w = W.generate(spec)
    d = upload(w)
    B, Hkv, T = spec.batch, spec.kv_heads, spec.max_tokens
    buf = torch.empty((B, T, 2, Hkv, 128), dtype=d.k.dtype, device=d.k.device)
    kview = buf[:, :, 0].permute(0, 2, 1, 3)  # [B, Hkv, T, 128]
    vview = buf[:, :, 1].permute(0, 2, 1, 3)
    kview.copy_(d.k)
    vview.copy_(d.v)
    layout = bsa.layout_for(kview, spec.q_heads)
    assert (layout.kv_stride_h, layout.kv_stride_t) == (128, 2 * Hkv * 128)
    d = dataclasses.replace(d, k=kview, v=vview, layout=layout)
    d.pack()
    d.run()
    torch.cuda.synchronize()
    check_all(w, d)
    _two_calls_match(d)
