"""Parity of the coarse-semantic-block path (Coarse Semantic Blocks abstract:
blocks of noncontiguous tokens picked by their centroids, attention over the
picked blocks' keys and values) with the oracle, through the C ABI.

Index (offsets, members bit-exact; centroids within FP32 summation error),
centroid scores, the choice (bit-exact on the GPU's own scores), the
attention (2e-3); the four calls against the fused two; query-group sizes
1..16; ragged and empty sequences, blocks with no token, assignments outside
[0, C); budgets below the largest block (nothing fits) and above the length
(every block: dense attention); crafted scores with ties, NaN and infinities.
"""

import dataclasses
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from block_sparse_attention_pack_amd import binding as bsa
from block_sparse_attention_pack_amd import workloads as W
from block_sparse_attention_pack_amd.step import step_calls, upload

import parity_util as PU

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bsa.load()


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    return t.cpu().numpy()


OUT = ("scores", "idx", "count", "part_o", "part_lse", "out", "out_lse")


def run_and_check(w, splits=None, kv_dtype="f16"):
    d = upload(w, splits=splits, kv_dtype=kv_dtype)
    assert d.cluster_mode
    d.pack()
    d.run()
    torch.cuda.synchronize()
    PU.check_units(w, d)
    # the fused form (score_select_clusters, attend_combine) gives the same bits
    ref = [host(getattr(d, n)).copy() for n in OUT]
    for n in OUT:
        getattr(d, n).fill_(7)
    for c in step_calls(d, "fused"):
        c()
    torch.cuda.synchronize()
    for n, a in zip(OUT, ref):
        assert np.array_equal(a, host(getattr(d, n)), equal_nan=True), n
    assert int(d.counters.abs().sum()) == 0
    return d


def test_reduced_cluster_workload():
    spec = W.reduced("cluster", 16384, batch=2)
    _say(f"[cluster] {spec.name}")
    run_and_check(W.generate(spec))


@pytest.mark.parametrize("G", [1, 2, 8, 16])
def test_cluster_group_sizes(G):
    spec = dataclasses.replace(W.SPECS["cluster"], name=f"cgroup{G}", seed=80 + G, batch=1,
                               kv_heads=2, q_heads=2 * G, max_tokens=4096, budget=256,
                               n_clusters=40, needle_count=2)
    run_and_check(W.generate(spec))


def test_cluster_ragged_lengths_empty_blocks_and_stray_ids():
    spec = dataclasses.replace(W.SPECS["cluster"], name="cragged", seed=90, batch=4, kv_heads=2,
                               q_heads=8, max_tokens=4096, budget=300, n_clusters=64,
                               needle_count=2, lengths=(0, 1, 1000, 4096))
    w = W.generate(spec)
    a = w.assign.copy()
    a[:, :, ::7] = -1          # tokens in no block
    a[:, :, 3::11] = 64 + 5    # ids outside [0, C): in no block either
    a[a == 17] = 18            # block 17 empty
    w = dataclasses.replace(w, assign=a)
    run_and_check(w, splits=3)


@pytest.mark.parametrize("budget", [1, 4096])
def test_cluster_budget_extremes(budget):
    """budget 1: no block fits (count 0, out 0, lse -inf); budget >= length:
    every block, i.e. dense attention."""
    spec = dataclasses.replace(W.SPECS["cluster"], name=f"cbudget{budget}", seed=95, batch=2,
                               kv_heads=2, q_heads=8, max_tokens=4096, budget=budget,
                               n_clusters=32, needle_count=1)
    d = run_and_check(W.generate(spec), splits=1)
    if budget == 1:
        assert int(d.count.abs().sum()) == 0
        assert not host(d.out).any() and np.all(host(d.out_lse) == -np.inf)
    else:
        assert np.array_equal(host(d.count), np.full((2, 2), 4096))


def test_cluster_choice_on_crafted_scores():
    """bsa_select_clusters on given scores: exact ties (lower id first), NaN
    (last), -inf, +inf, -0 / +0, against the oracle's choice."""
    from oracle import decode as O

    spec = dataclasses.replace(W.SPECS["cluster"], name="ccraft", seed=99, batch=1, kv_heads=4,
                               q_heads=4, max_tokens=2048, budget=700, n_clusters=50,
                               needle_count=0)
    w = W.generate(spec)
    d = upload(w)
    d.pack()
    rng = np.random.default_rng(5)
    pool = np.array([np.nan, -np.inf, np.inf, -0.0, 0.0, 1.0, 1.0, 2.5, -3.0], dtype=np.float32)
    sc = rng.choice(pool, size=(1, 4, 50)).astype(np.float32)
    d.scores.copy_(torch.from_numpy(sc))
    d.select_clusters()
    torch.cuda.synchronize()
    for h in range(4):
        off, mem = host(d.offsets[0, h]), host(d.members[0, h])
        sizes = np.diff(off)
        s_eff = np.where(sizes > 0, sc[0, h].astype(np.float64), -np.inf)
        ch, tot = O.select_clusters(s_eff, sizes, spec.budget)
        toks, n = O.cluster_tokens(ch, off, mem, spec.budget)
        assert int(host(d.count)[0, h]) == n
        assert np.array_equal(host(d.idx[0, h]), toks), h
