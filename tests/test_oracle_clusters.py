"""The oracle's coarse semantic blocks (Coarse Semantic Blocks abstract: keys
clustered into blocks of noncontiguous tokens, blocks picked by their
centroids' scores, attention over the picked blocks' original keys and
values), pinned to hand-worked cases, brute force and the dense limit (CPU)."""

import itertools

import numpy as np

from oracle import decode as O


def test_index_worked_example():
    # 12 tokens, one-hot keys e_t; tokens at or past the length (11) are not
    # indexed; token 4 belongs to no block; block 4 is empty
    k = np.zeros((12, 128))
    for t in range(12):
        k[t, t] = 1.0
    assign = np.array([2, 0, 2, 1, -1, 0, 3, 2, 1, 0, 3, 3])
    cent, off, mem = O.cluster_index(k, assign, 5, 11)
    assert off.tolist() == [0, 3, 5, 8, 10, 10]
    assert mem.tolist() == [1, 5, 9, 3, 8, 0, 2, 7, 6, 10]
    third = 1.0 / 3.0
    assert np.allclose(cent[0][:12], [0, third, 0, 0, 0, third, 0, 0, 0, third, 0, 0], atol=0)
    assert cent[1][3] == 0.5 and cent[1][8] == 0.5 and cent[1].sum() == 1.0
    assert cent[3][6] == 0.5 and cent[3][10] == 0.5 and cent[3][11] == 0.0
    assert not cent[4].any()


def test_scores_brute_force():
    rng = np.random.default_rng(1)
    G, C = 3, 6
    q = rng.standard_normal((G, 128)).astype(np.float16)
    cent = rng.standard_normal((C, 128))
    sizes = np.array([4, 0, 1, 7, 2, 9])
    sigma = 0.125
    got = O.cluster_scores(q, cent, sizes, sigma)
    for c in range(C):
        if sizes[c] == 0:
            assert got[c] == -np.inf
            continue
        best = max(sum(float(q[h, d]) * float(cent[c, d]) for d in range(128)) for h in range(G))
        assert abs(got[c] - sigma * best) <= 1e-12 * max(1.0, abs(best))


def test_selection_worked_example():
    scores = np.array([0.5, 0.9, 0.9, -1.0, 3.0])
    sizes = np.array([3, 2, 3, 2, 0])  # block 4 is empty: never chosen
    # ranking 1 (0.9, the lower id), 2 (0.9), 0, 3: sizes 2, 3, 3, 2
    ch, tot = O.select_clusters(scores, sizes, 5)
    assert ch.tolist() == [1, 2] and tot == 5
    ch, tot = O.select_clusters(scores, sizes, 4)  # block 2 does not fit: the prefix ends
    assert ch.tolist() == [1] and tot == 2
    ch, tot = O.select_clusters(scores, sizes, 1)
    assert ch.tolist() == [] and tot == 0
    ch, tot = O.select_clusters(np.array([np.nan, 0.0, -np.inf]), np.array([1, 1, 1]), 3)
    assert ch.tolist() == [1, 2, 0] and tot == 3  # NaN ranks last, below -inf
    off = np.array([0, 3, 5, 8, 10, 10])
    mem = np.array([1, 5, 9, 3, 8, 0, 2, 7, 6, 10])
    toks, n = O.cluster_tokens(np.array([2, 0]), off, mem, 8)
    assert toks.tolist() == [0, 2, 7, 1, 5, 9, -1, -1] and n == 6


def test_selection_is_the_longest_fitting_prefix():
    rng = np.random.default_rng(2)
    for _ in range(200):
        C = int(rng.integers(1, 9))
        scores = rng.choice([-1.0, 0.0, 0.5, 2.0, np.nan], size=C)
        sizes = rng.integers(0, 6, size=C)
        budget = int(rng.integers(0, 20))
        ch, tot = O.select_clusters(scores, sizes, budget)
        # brute force: rank by (NaN last, score desc, id), drop empties, prefix
        ranked = sorted((c for c in range(C) if sizes[c] > 0),
                        key=lambda c: (np.isnan(scores[c]),
                                       -(scores[c] if not np.isnan(scores[c]) else 0), c))
        want, run = [], 0
        for c in ranked:
            if run + sizes[c] > budget:
                break
            want.append(c)
            run += sizes[c]
        assert ch.tolist() == want and tot == run


def test_every_block_within_budget_is_dense_attention():
    rng = np.random.default_rng(3)
    T, L, C = 300, 257, 7
    q = rng.standard_normal((4, 128)).astype(np.float16)
    k = rng.standard_normal((T, 128)).astype(np.float16)
    v = rng.standard_normal((T, 128)).astype(np.float16)
    assign = rng.integers(0, C, size=T)
    cent, off, mem = O.cluster_index(k, assign, C, L)
    sizes = np.diff(off)
    sc = O.cluster_scores(q, cent, sizes, 0.1)
    ch, tot = O.select_clusters(sc, sizes, L)
    assert tot == L and sorted(ch.tolist()) == [c for c in range(C) if sizes[c]]
    toks, n = O.cluster_tokens(ch, off, mem, L)
    assert sorted(toks[:n].tolist()) == list(range(L))
    kr, vr = O.gather_rows_token(k, v, toks[:n])
    o, lse = O.attend(q, kr, vr, 0.1)
    od, lsed = O.attend(q, k[:L].astype(np.float64), v[:L].astype(np.float64), 0.1)
    assert np.abs(o - od).max() < 1e-12 and np.abs(lse - lsed).max() < 1e-12
