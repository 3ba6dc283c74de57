"""select_topk on crafted score rows, through the C ABI, against the oracle.

The scores are written straight into the score buffer, so the selection is
tested on rows no scan would give: exact ties spread over many 8192-key chunks,
keys that differ only in their lowest bits (every radix digit is needed), NaN,
signed zeros, infinities and subnormals, all-equal rows, and budgets from 1 to
above the candidate count. The result must be bit-exact: the same indices, in
ascending order, and the same count.
"""

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from block_sparse_attention_pack_amd import binding as bsa

from oracle import decode as O

import parity_util as PU

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bsa.load()


def _layout(B, Hkv, T):
    # select_topk reads no K: a contiguous [B, Hkv, T, 128] layout with no buffer
    return bsa.KvLayout(B, Hkv, Hkv, 128, 128, T, Hkv * T * 128, T * 128, 128, bsa.DTYPE_F16)


def _rows(pattern, n, rng):
    if pattern == "random":
        return rng.standard_normal(n).astype(np.float32)
    if pattern == "low_bits":  # one exponent, 700 neighbouring mantissas, each ~n/700 times
        return (np.float32(1.5) + (rng.integers(0, 700, n) * np.float32(2.0 ** -23))).astype(np.float32)
    if pattern == "few_values":  # four values: every boundary is a tie spread over all chunks
        return rng.integers(0, 4, n).astype(np.float32)
    if pattern == "specials":
        pool = np.array([np.nan, -0.0, 0.0, -np.inf, np.inf, 1e-45, -1e-45, 3.0, -3.0, 1e30,
                         -1e30, 2.0 ** -126], dtype=np.float32)
        return pool[rng.integers(0, len(pool), n)]
    if pattern == "all_equal":
        return np.full(n, 0.25, dtype=np.float32)
    if pattern == "peaked":  # logits spread over ~40: the softmax mass sits in a few hundred keys
        return (rng.standard_normal(n) * 5.0).astype(np.float32)
    raise ValueError(pattern)


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _histograms_back_at_zero(ws, units, T, one_group=False):
    """After a call each unit's histogram in the token workspace is zero again
    (per unit: 4096 histogram words; a slot of 8 + 3 words per 16384-key chunk,
    rounded up to 64; two bitmaps of ceil(T/64)*2 words rounded up to 64).
    With the one-launch select (budget <= 2048, T <= 131072) a
    second region follows, 64 + 2 * 8192 words per unit and 32768-token chunk:
    its arrival counter (word 0) is zero again too."""
    w = ws.view(torch.int32).cpu().numpy()
    W = -(-T // 64) * 2
    slot = -(-(8 + 3 * -(-T // 16384)) // 64) * 64
    per = 4096 + slot + 2 * (-(-W // 64) * 64)
    one = 64 + -(-T // 32768) * 2 * 8192 if one_group else 0
    assert w.size == units * (per + one), (w.size, units, per, one)
    for u in range(units):
        assert not w[u * per:u * per + 4096].any(), f"histogram of unit {u}"
        if one_group:
            assert w[units * per + u * one] == 0, f"arrival counter of unit {u}"


@pytest.mark.parametrize("pattern", ["random", "low_bits", "few_values", "specials", "all_equal"])
@pytest.mark.parametrize("budget", [1, 300, 2048, 40000])
def test_token_select_matches_oracle(pattern, budget):
    T = 40960  # five 8192-key chunks
    lengths = [T, 40001, 8193, 8192, 8191, 2049, 1, 0]
    B, Hkv = len(lengths), 2
    rng = np.random.default_rng([7, budget, len(pattern)])
    scores = np.stack([_rows(pattern, T, rng) for _ in range(B * Hkv)]).reshape(B, Hkv, T)
    _say(f"[select] token pattern={pattern} budget={budget} T={T}")
    layout = _layout(B, Hkv, T)
    cfg = bsa.select_cfg(bsa.TOKEN, budget, 0, 32, 0.1)
    ws_bytes = bsa.workspace_size(layout, cfg)
    dev = torch.device("cuda")
    ws = torch.zeros((ws_bytes,), dtype=torch.uint8, device=dev)  # zero before the first use
    sc = torch.from_numpy(scores).to(dev)
    lens = torch.tensor(lengths, dtype=torch.int32, device=dev)
    idx = torch.full((B, Hkv, budget), 5, dtype=torch.int32, device=dev)
    count = torch.full((B, Hkv), 5, dtype=torch.int32, device=dev)
    for rep in range(2):  # a second call on the same workspace
        bsa.select_topk(layout, cfg, sc, lens, ws, ws_bytes, idx, count)
        torch.cuda.synchronize()
        _histograms_back_at_zero(ws, B * Hkv, T, one_group=budget <= 2048)
        gi, gc = idx.cpu().numpy(), count.cpu().numpy()
        for b in range(B):
            for h in range(Hkv):
                ri, rc = O.select_tokens_unit(scores[b, h].astype(np.float64), lengths[b], budget)
                assert int(gc[b, h]) == rc, (pattern, budget, b, h, rep)
                assert np.array_equal(gi[b, h], ri), (pattern, budget, b, h, rep)


def _sample_positions(C):
    """Tokens whose scores the one-launch token select samples for its
    threshold (1024 evenly spaced ones when a row has more than 16384
    candidates)."""
    return (np.arange(1024, dtype=np.int64) * C) // 1024


@pytest.mark.parametrize("case", ["sampled_high", "unsampled_high"])
def test_token_select_when_the_sample_misleads(case):
    """Rows built against the threshold sample: only the sampled tokens score
    high (far fewer than the budget lie above the sampled threshold), or only
    the unsampled ones do (far more candidates than the list holds). Both take
    the selection over the scores in memory and must still be exact."""
    T = 131072
    lengths = [T, 65536, 16385, 16384]
    B, Hkv, budget = len(lengths), 1, 2048
    rng = np.random.default_rng([12, len(case)])
    scores = np.zeros((B, Hkv, T), dtype=np.float32)
    for b, C in enumerate(lengths):
        pos = _sample_positions(C)
        row = np.full(T, -5.0, dtype=np.float32)
        if case == "sampled_high":
            row[:C] = -1.0 - rng.random(C).astype(np.float32)
            row[pos] = 1.0 + rng.random(len(pos)).astype(np.float32)
        else:
            row[:C] = 1.0 + rng.random(C).astype(np.float32)
            row[pos] = -1.0 - rng.random(len(pos)).astype(np.float32)
        scores[b, 0] = row
    _say(f"[select] token sample case={case} T={T}")
    layout = _layout(B, Hkv, T)
    cfg = bsa.select_cfg(bsa.TOKEN, budget, 0, 32, 0.1)
    ws_bytes = bsa.workspace_size(layout, cfg)
    dev = torch.device("cuda")
    ws = torch.zeros((ws_bytes,), dtype=torch.uint8, device=dev)
    sc = torch.from_numpy(scores).to(dev)
    lens = torch.tensor(lengths, dtype=torch.int32, device=dev)
    idx = torch.full((B, Hkv, budget), 5, dtype=torch.int32, device=dev)
    count = torch.full((B, Hkv), 5, dtype=torch.int32, device=dev)
    for rep in range(2):  # the arrival counters are left at zero for the second
        bsa.select_topk(layout, cfg, sc, lens, ws, ws_bytes, idx, count)
        torch.cuda.synchronize()
        _histograms_back_at_zero(ws, B * Hkv, T, one_group=True)
    gi, gc = idx.cpu().numpy(), count.cpu().numpy()
    for b in range(B):
        ri, rc = O.select_tokens_unit(scores[b, 0].astype(np.float64), lengths[b], budget)
        assert int(gc[b, 0]) == rc, (case, b)
        assert np.array_equal(gi[b, 0], ri), (case, b)


@pytest.mark.parametrize("pattern", ["random", "low_bits", "few_values", "specials", "all_equal"])
@pytest.mark.parametrize("nb,budget,n_tail", [(1024, 64, 0), (1000, 37, 1), (256, 256, 2),
                                              (2048, 130, 2), (4096, 1000, 1), (4096, 4096, 0)])
def test_block_select_matches_oracle(pattern, nb, budget, n_tail):
    T = nb * 128  # 2048 blocks fill the per-thread registers; 4096 re-read memory
    lengths = [T, T - 1, T // 2 + 5, 129, 128, 1, 0]
    B, Hkv = len(lengths), 2
    rng = np.random.default_rng([8, nb, budget, len(pattern)])
    scores = np.stack([_rows(pattern, nb, rng) for _ in range(B * Hkv)]).reshape(B, Hkv, nb)
    _say(f"[select] block pattern={pattern} blocks={nb} budget={budget} tail={n_tail}")
    layout = _layout(B, Hkv, T)
    cfg = bsa.select_cfg(bsa.BLOCK, budget, n_tail, 0, 0.1)
    dev = torch.device("cuda")
    sc = torch.from_numpy(scores).to(dev)
    lens = torch.tensor(lengths, dtype=torch.int32, device=dev)
    idx = torch.full((B, Hkv, budget), 5, dtype=torch.int32, device=dev)
    count = torch.full((B, Hkv), 5, dtype=torch.int32, device=dev)
    bsa.select_topk(layout, cfg, sc, lens, None, 0, idx, count)
    torch.cuda.synchronize()
    gi, gc = idx.cpu().numpy(), count.cpu().numpy()
    for b in range(B):
        for h in range(Hkv):
            ri, rc = O.select_blocks_unit(scores[b, h].astype(np.float64), lengths[b], n_tail,
                                          budget)
            assert int(gc[b, h]) == rc, (pattern, b, h)
            assert np.array_equal(gi[b, h], ri), (pattern, b, h)


@pytest.mark.parametrize("pattern", ["random", "few_values"])
def test_token_select_over_several_bitmap_windows(pattern):
    """Rows longer than 131072 tokens: the bitmaps are compacted in several windows."""
    T = 262144
    lengths = [T, 140000, 131073]
    B, Hkv, budget = len(lengths), 2, 3000
    rng = np.random.default_rng([9, len(pattern)])
    scores = np.stack([_rows(pattern, T, rng) for _ in range(B * Hkv)]).reshape(B, Hkv, T)
    _say(f"[select] token windows pattern={pattern} T={T}")
    layout = _layout(B, Hkv, T)
    cfg = bsa.select_cfg(bsa.TOKEN, budget, 0, 32, 0.1)
    ws_bytes = bsa.workspace_size(layout, cfg)
    dev = torch.device("cuda")
    ws = torch.zeros((ws_bytes,), dtype=torch.uint8, device=dev)
    sc = torch.from_numpy(scores).to(dev)
    lens = torch.tensor(lengths, dtype=torch.int32, device=dev)
    idx = torch.full((B, Hkv, budget), 5, dtype=torch.int32, device=dev)
    count = torch.full((B, Hkv), 5, dtype=torch.int32, device=dev)
    bsa.select_topk(layout, cfg, sc, lens, ws, ws_bytes, idx, count)
    torch.cuda.synchronize()
    _histograms_back_at_zero(ws, B * Hkv, T)
    gi, gc = idx.cpu().numpy(), count.cpu().numpy()
    for b in range(B):
        for h in range(Hkv):
            ri, rc = O.select_tokens_unit(scores[b, h].astype(np.float64), lengths[b], budget)
            assert int(gc[b, h]) == rc, (pattern, b, h)
            assert np.array_equal(gi[b, h], ri), (pattern, b, h)


@pytest.mark.parametrize("pattern", ["random", "peaked", "few_values", "specials", "all_equal"])
@pytest.mark.parametrize("budget", [1, 300, 4096])
@pytest.mark.parametrize("top_p", [0.05, 0.5, 0.9, 1.0])
def test_token_top_p_matches_oracle(pattern, budget, top_p):
    """The adaptive budget: the kept tokens are the top-ranked ones, the count
    is a valid cut of the softmax shares, and the workspace is left reusable."""
    T = 40960
    lengths = [T, 40001, 8193, 8192, 8191, 2049, 1, 0]
    B, Hkv = len(lengths), 2
    rng = np.random.default_rng([11, budget, len(pattern), int(top_p * 100)])
    scores = np.stack([_rows(pattern, T, rng) for _ in range(B * Hkv)]).reshape(B, Hkv, T)
    _say(f"[select] top-p pattern={pattern} budget={budget} p={top_p}")
    layout = _layout(B, Hkv, T)
    cfg = bsa.select_cfg(bsa.TOKEN, budget, 0, 32, 0.1, top_p=top_p)
    ws_bytes = bsa.workspace_size(layout, cfg)
    dev = torch.device("cuda")
    ws = torch.zeros((ws_bytes,), dtype=torch.uint8, device=dev)
    sc = torch.from_numpy(scores).to(dev)
    lens = torch.tensor(lengths, dtype=torch.int32, device=dev)
    idx = torch.full((B, Hkv, budget), 5, dtype=torch.int32, device=dev)
    count = torch.full((B, Hkv), 5, dtype=torch.int32, device=dev)
    for rep in range(2):
        bsa.select_topk(layout, cfg, sc, lens, ws, ws_bytes, idx, count)
        torch.cuda.synchronize()
        _histograms_back_at_zero(ws, B * Hkv, T, one_group=budget <= 2048)
        gi, gc = idx.cpu().numpy(), count.cpu().numpy()
        for b in range(B):
            for h in range(Hkv):
                PU.check_top_p_selection(scores[b, h], lengths[b], budget, top_p, gi[b, h],
                                         gc[b, h])
