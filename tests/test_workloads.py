"""Input generators: determinism, shapes and the structure each workload states (CPU)."""

import numpy as np

from block_sparse_attention_pack_amd import workloads as W


def test_specs_shapes_and_budgets():
    s = W.SPECS
    assert (s["tiny"].batch, s["tiny"].kv_heads, s["tiny"].q_heads, s["tiny"].max_tokens,
            s["tiny"].budget) == (1, 1, 4, 4096, 8)
    assert (s["llama8b"].kv_heads, s["llama8b"].q_heads, s["llama8b"].max_blocks,
            s["llama8b"].budget) == (8, 32, 256, 64)
    assert (s["jetqsparse"].batch, s["jetqsparse"].kv_heads, s["jetqsparse"].q_heads,
            s["jetqsparse"].max_blocks, s["jetqsparse"].budget) == (16, 4, 16, 1024, 64)
    assert s["ragged"].budget == 128 and s["ragged"].n_tail == 2
    # token budget at the fixed 1.5625% density (JSSA Figure 3): 2048 of 131072
    assert s["token"].budget == s["token"].max_tokens * 0.015625 == 2048
    assert s["token"].rank == 32
    for sp in s.values():
        assert sp.q_heads % sp.kv_heads == 0


def test_generation_is_deterministic_and_unit_redrawable():
    spec = W.reduced("jetqsparse", 2048, batch=2)
    a = W.generate(spec)
    b = W.generate(spec, threads=1)
    for name in ("q", "k", "v", "key_center", "global_scale", "seq_lens"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
    assert a.k.dtype == np.float16 and a.k.shape == (2, 4, 2048, 128)


def test_needles_align_with_group_mean_query():
    w = W.generate(W.SPECS["tiny"])
    qm = w.q[0].astype(np.float64).mean(axis=0)
    qm /= np.linalg.norm(qm)
    proj = (w.k[0, 0].astype(np.float64) @ qm).reshape(-1, 128).mean(axis=1)
    needles = set(int(x) for x in w.needles[0][0])
    assert len(needles) == 3
    others = [proj[i] for i in range(32) if i not in needles]
    for n in needles:  # +2.0 along the mean query direction
        assert proj[n] > max(others) + 1.0


def test_ragged_lengths_tail_pages_and_calibration():
    spec = W.reduced("ragged", 8192, batch=3)
    w = W.generate(spec)
    assert np.all(w.seq_lens >= 4096) and np.all(w.seq_lens <= 8192)
    for b in range(3):
        npg = w.n_pages(b)
        for h in range(4):
            assert np.all(w.needles[b][h] < npg - 2)
            page = npg - 1
            tail = (w.tail_k[b, h, 1].astype(np.uint32) << 16).view(np.float32)
            main = w.k[b, h, page * 128:(page + 1) * 128].astype(np.float32)
            assert np.abs(tail - main).max() <= 2.0 ** -7 * np.abs(main).max() + 1e-3
    assert w.global_scale.dtype == np.float32 and np.all(w.global_scale > 0)
    # the largest centered key magnitude maps onto 6 * 448
    y = np.abs(w.k[0, 0, :(w.n_pages(0) - 2) * 128].astype(np.float32) - w.key_center[0])
    assert y.max() <= w.global_scale[0] * 2688 * (1 + 1e-6)


def test_token_projection_orthonormal_and_shared():
    w = W.generate(W.reduced("token", 1024, batch=1))
    P = w.proj
    assert P.shape == (8, 128, 32)
    assert np.abs(P[0].T.astype(np.float64) @ P[0] - np.eye(32)).max() < 1e-6
    assert all(np.array_equal(P[0], P[h]) for h in range(8))


def test_algorithmic_bytes_of_the_full_shapes():
    # block mode: 72 B per scanned token and 512 B per attended token
    s = W.SPECS["jetqsparse"]
    scan = s.units * 72 * s.max_tokens
    attn = s.units * 512 * s.budget * 128
    assert (scan, attn, scan + attn) == (603979776, 268435456, 872415232)
    t = W.SPECS["token"]
    assert t.units * 64 * t.max_tokens + t.units * 512 * t.budget == 603979776
