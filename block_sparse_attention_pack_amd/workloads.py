"""Seeded synthetic decode-step workloads, shared by the oracle and the HIP path.

This module only draws inputs. It holds none of the decode-step arithmetic
(no quantization, scoring, selection or attention); both the CPU oracle and
the GPU path receive exactly the arrays built here.

The workloads follow the sparse-decode settings the pages evaluate:

* ``tiny``        B1  Hkv1 Hq4  T4096   block budget 8     (3 needle blocks, +2.0)
* ``llama8b``     B1  Hkv8 Hq32 T32768  block budget 64    (1% needle blocks, norm 3)
* ``jetqsparse``  B16 Hkv4 Hq16 T131072 block budget 64    (per-channel key offset,
                  Zipf-profile needles over 2% of blocks); the decode shape of the
                  Jet-QSparse abstract (128K context, batch 16, 64 blocks per KV head)
* ``ragged``      the jetqsparse shape with budget 128, lengths uniform in
                  [64K, 128K], 4 outlier channels x8, and the two newest pages kept
                  in BF16 (Jet-QSparse abstract: up to two BF16 pages per sequence)
* ``token``       B8 Hkv8 Hq32 T131072, rank-32 projected keys from a seeded
                  orthonormal P, top-2048 tokens (JSSA abstract and Figure 1;
                  1.5625% density of JSSA Figure 3: 2048 of 131072)
* ``token_topp``  the token shape with 8 strong needle blocks per unit (key
                  component of norm 96 along the group's mean query, so most of
                  the softmax mass sits in about 1000 tokens) and the adaptive
                  budget at top_p 0.9 (RaBitQCache abstract): of at most 2048
                  tokens, about 860 are kept
* ``jetqsparse_v4`` the jetqsparse inputs with the values held in a 4-bit
                  NVFP4 store (the Jet-QSparse abstract's NVFP4 cache with values
                  compressed too): 72 B per attended value row instead of 256
* ``jetqsparse_g16`` the jetqsparse shape with 64 query heads (16 per KV head,
                  the largest group the kernels take)
* ``cluster``     B8 Hkv8 Hq32 T131072 in 1024 coarse blocks of noncontiguous
                  tokens (each token's block drawn uniformly, about 128 tokens a
                  block; keys = the block's center + unit noise), 4 needle blocks
                  whose centers lean towards the group's mean query, a token
                  budget of 2048 (Coarse Semantic Blocks abstract: blocks picked
                  by their centroids under a token budget)

Every workload also exists at reduced size (``scale_tokens`` / ``batch``) so the
oracle finishes in seconds while still spanning many tiles and a ragged tail.

Random streams are drawn per (sequence, KV head) from
``numpy.random.default_rng([seed, stream, b, h])``, so any unit can be redrawn
on its own (the full-size sampled checks rely on that).

Calibration inputs (the key-centering vector and the per-KV-head FP32 scales)
are produced here too: the centering vector is the per-channel mean of the
keys over the packed region (the tiny workload states exactly that), and the
per-KV-head scale maps the largest centered key magnitude onto the largest
NVFP4 magnitude (6 x 448 = 2688), so that no block scale saturates; the value
store's scale does the same for the largest |v| of the KV head.
"""

from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional

import numpy as np

HEAD_DIM = 128
BLOCK = 128
# Largest NVFP4 magnitude: E2M1 max (6) times E4M3 max (448).
NVFP4_MAX = 2688.0

# stream ids for default_rng([seed, stream, ...])
_S_Q, _S_K, _S_V, _S_NEEDLE, _S_OFFSET, _S_OUTLIER, _S_LENS, _S_PROJ, _S_ASSIGN = range(1, 10)


@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape and structure of one synthetic workload."""

    name: str
    seed: int
    batch: int
    kv_heads: int
    q_heads: int
    max_tokens: int
    granularity: str  # "block", "token" or "cluster"
    budget: int  # blocks (block mode) or tokens (token mode), forced pages included
    n_tail: int = 0  # BF16 tail pages per (sequence, KV head), always selected
    needle_count: int = 0  # needle blocks per unit
    needle_profile: str = "none"  # "const" or "zipf"
    needle_strength: float = 0.0
    key_offset_std: float = 0.0  # per (KV head, channel) offset, shared over b and t
    outlier_channels: int = 0
    outlier_gain: float = 1.0
    ragged: bool = False  # lengths uniform in [max_tokens/2, max_tokens]
    rank: int = 0  # projection rank in token mode
    proj_fmt: str = "bf16"  # token mode: projected-key cache storage, "bf16" or "fp8"
    query_fmt: str = "f16"  # block mode: the query the scan scores with, "f16" or "nvfp4"
    top_p: float = 0.0  # token mode: 0 keeps the budget; else the adaptive (top-p) budget
    value_fmt: str = "f16"  # "f16": V from the cache; "nvfp4": V from the 4-bit value store
    n_clusters: int = 0  # cluster mode: coarse blocks per unit
    lengths: Optional[tuple] = None  # explicit sequence lengths (edge cases), one per sequence

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def max_blocks(self) -> int:
        return self.max_tokens // BLOCK

    @property
    def units(self) -> int:
        return self.batch * self.kv_heads


SPECS: Dict[str, Spec] = {
    "tiny": Spec("tiny", 0, 1, 1, 4, 4096, "block", 8,
                 needle_count=3, needle_profile="const", needle_strength=2.0),
    "llama8b": Spec("llama8b", 1, 1, 8, 32, 32768, "block", 64,
                    needle_count=3, needle_profile="const", needle_strength=3.0),
    "jetqsparse": Spec("jetqsparse", 2, 16, 4, 16, 131072, "block", 64,
                       needle_count=20, needle_profile="zipf", needle_strength=3.0,
                       key_offset_std=2.0),
    "ragged": Spec("ragged", 3, 16, 4, 16, 131072, "block", 128, n_tail=2,
                   needle_count=20, needle_profile="zipf", needle_strength=3.0,
                   key_offset_std=2.0, outlier_channels=4, outlier_gain=8.0, ragged=True),
    "token": Spec("token", 4, 8, 8, 32, 131072, "token", 2048, rank=32),
    # the token workload's inputs (same seed) with an FP8 projected-key cache
    "token_fp8": Spec("token_fp8", 4, 8, 8, 32, 131072, "token", 2048, rank=32,
                      proj_fmt="fp8"),
    # the Jet-QSparse decode shape's inputs (same seed), scanned with an NVFP4 query
    "jetqsparse_q4": Spec("jetqsparse_q4", 2, 16, 4, 16, 131072, "block", 64,
                          needle_count=20, needle_profile="zipf", needle_strength=3.0,
                          key_offset_std=2.0, query_fmt="nvfp4"),
    # the token shape with the adaptive budget (top-p retrieval, RaBitQCache
    # abstract): 8 strong needle blocks per unit hold most of the softmax mass,
    # so keeping 90% of it takes fewer than the 2048 tokens
    "token_topp": Spec("token_topp", 4, 8, 8, 32, 131072, "token", 2048, rank=32,
                       needle_count=8, needle_profile="const", needle_strength=96.0,
                       top_p=0.9),
    # the Jet-QSparse decode shape's inputs (same seed), values in the 4-bit store
    "jetqsparse_v4": Spec("jetqsparse_v4", 2, 16, 4, 16, 131072, "block", 64,
                          needle_count=20, needle_profile="zipf", needle_strength=3.0,
                          key_offset_std=2.0, value_fmt="nvfp4"),
    # the Jet-QSparse decode shape with 16 query heads per KV head
    "jetqsparse_g16": Spec("jetqsparse_g16", 2, 16, 4, 64, 131072, "block", 64,
                           needle_count=20, needle_profile="zipf", needle_strength=3.0,
                           key_offset_std=2.0),
    # coarse semantic blocks picked by their centroids, at the token shape
    "cluster": Spec("cluster", 5, 8, 8, 32, 131072, "cluster", 2048, n_clusters=1024,
                    needle_count=4, needle_profile="const", needle_strength=8.0),
}

ORDER = ["tiny", "llama8b", "jetqsparse", "ragged", "token", "token_fp8", "jetqsparse_q4",
         "token_topp", "jetqsparse_v4", "cluster", "jetqsparse_g16"]


def reduced(name: str, max_tokens: int, batch: Optional[int] = None,
            budget: Optional[int] = None) -> Spec:
    """A smaller copy of a workload: fewer tokens (and optionally sequences).

    Needle counts and token budgets keep the full workload's density.
    """
    s = SPECS[name]
    assert max_tokens % BLOCK == 0
    frac = max_tokens / s.max_tokens
    kw = dict(max_tokens=max_tokens, name=f"{s.name}@{max_tokens}")
    if batch is not None:
        kw["batch"] = batch
    if s.needle_count:
        kw["needle_count"] = max(1, int(round(s.needle_count * frac)))
    if s.n_clusters:
        kw["n_clusters"] = max(4, int(round(s.n_clusters * frac)))
    if budget is not None:
        kw["budget"] = budget
    elif s.granularity in ("token", "cluster"):
        kw["budget"] = max(1, int(round(s.budget * frac)))
    else:
        kw["budget"] = min(s.budget, max(s.n_tail + 1, max_tokens // BLOCK // 4))
    return dataclasses.replace(s, **kw)


@dataclasses.dataclass
class Workload:
    spec: Spec
    q: np.ndarray  # float16 [B, Hq, D]
    k: np.ndarray  # float16 [B, Hkv, T, D]
    v: np.ndarray  # float16 [B, Hkv, T, D]
    seq_lens: np.ndarray  # int32 [B]
    key_center: np.ndarray  # float32 [Hkv, D]
    global_scale: np.ndarray  # float32 [Hkv]
    tail_k: Optional[np.ndarray]  # uint16 BF16 bits [B, Hkv, 2, 128, D]
    tail_v: Optional[np.ndarray]
    proj: Optional[np.ndarray]  # float32 [Hkv, D, r]
    needles: List[List[np.ndarray]]  # [b][h] -> block ids carrying needles
    value_scale: Optional[np.ndarray] = None  # float32 [Hkv], the 4-bit value store's scale
    assign: Optional[np.ndarray] = None  # int32 [B, Hkv, T]: each token's coarse block (cluster)

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(HEAD_DIM)

    def n_pages(self, b: int) -> int:
        return -(-int(self.seq_lens[b]) // BLOCK)

    def packed_blocks(self, b: int) -> int:
        """Blocks of sequence b held in the 4-bit copy (all but the tail pages)."""
        return max(0, self.n_pages(b) - self.spec.n_tail)


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest-even) and return the raw 16-bit patterns."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _seq_lens(spec: Spec) -> np.ndarray:
    if spec.lengths is not None:
        assert len(spec.lengths) == spec.batch
        return np.asarray(spec.lengths, dtype=np.int32)
    if not spec.ragged:
        return np.full(spec.batch, spec.max_tokens, dtype=np.int32)
    rng = np.random.default_rng([spec.seed, _S_LENS])
    lo = spec.max_tokens // 2
    return rng.integers(lo, spec.max_tokens, size=spec.batch, endpoint=True).astype(np.int32)


def _needle_blocks(spec: Spec, seq_lens: np.ndarray) -> List[List[np.ndarray]]:
    rng = np.random.default_rng([spec.seed, _S_NEEDLE])
    out = []
    for b in range(spec.batch):
        n_pages = -(-int(seq_lens[b]) // BLOCK)
        packed = max(0, n_pages - spec.n_tail)
        row = []
        for _h in range(spec.kv_heads):
            cnt = min(spec.needle_count, packed)
            row.append(np.sort(rng.choice(packed, size=cnt, replace=False)) if cnt else
                       np.zeros(0, dtype=np.int64))
        out.append(row)
    return out


def _needle_strengths(spec: Spec, count: int, rng: np.random.Generator) -> np.ndarray:
    if spec.needle_profile == "zipf":
        # Rank profile s_i = s_1 * i^-1.1 (a Zipf(1.1) law over needle ranks),
        # ranks assigned to the needle blocks in random order.
        s = spec.needle_strength * np.arange(1, count + 1, dtype=np.float64) ** -1.1
        return rng.permutation(s)
    return np.full(count, spec.needle_strength, dtype=np.float64)


def _unit_keys(spec: Spec, b: int, h: int, qdir: np.ndarray, offset: Optional[np.ndarray],
               outliers: Optional[np.ndarray], needles: np.ndarray) -> np.ndarray:
    """float32 keys of one (sequence, KV head) before rounding to the cache dtype."""
    rng = np.random.default_rng([spec.seed, _S_K, b, h])
    x = rng.standard_normal((spec.max_tokens, HEAD_DIM), dtype=np.float32)
    if outliers is not None:
        x[:, outliers[h]] *= np.float32(spec.outlier_gain)
    if offset is not None:
        x += offset[h][None, :]
    if len(needles):
        srng = np.random.default_rng([spec.seed, _S_NEEDLE, b, h])
        strengths = _needle_strengths(spec, len(needles), srng)
        for blk, s in zip(needles, strengths):
            x[blk * BLOCK:(blk + 1) * BLOCK] += (s * qdir).astype(np.float32)[None, :]
    return x


def _cluster_keys(spec: Spec, b: int, h: int, qdir: np.ndarray):
    """(keys float32 [T, D], assignment int32 [T]) of one unit in cluster mode:
    each token's block uniform over the n_clusters, keys = the block's center
    (N(0, 1) per channel) + N(0, 1) noise; needle blocks' centers gain
    needle_strength along qdir."""
    rng = np.random.default_rng([spec.seed, _S_ASSIGN, b, h])
    C = spec.n_clusters
    assign = rng.integers(0, C, size=spec.max_tokens).astype(np.int32)
    centers = rng.standard_normal((C, HEAD_DIM), dtype=np.float32)
    if spec.needle_count:
        nrng = np.random.default_rng([spec.seed, _S_NEEDLE, b, h])
        picks = nrng.choice(C, size=min(spec.needle_count, C), replace=False)
        strengths = _needle_strengths(spec, len(picks), nrng)
        for c, st in zip(picks, strengths):
            centers[c] += (st * qdir).astype(np.float32)
    krng = np.random.default_rng([spec.seed, _S_K, b, h])
    x = krng.standard_normal((spec.max_tokens, HEAD_DIM), dtype=np.float32)
    x += centers[assign]
    return x, assign


def _unit_values(spec: Spec, b: int, h: int) -> np.ndarray:
    rng = np.random.default_rng([spec.seed, _S_V, b, h])
    return rng.standard_normal((spec.max_tokens, HEAD_DIM), dtype=np.float32)


def _proj(spec: Spec) -> np.ndarray:
    """One seeded orthonormal P (D x r), shared by all KV heads, columns sign-fixed."""
    rng = np.random.default_rng([spec.seed, _S_PROJ])
    g = rng.standard_normal((HEAD_DIM, spec.rank))
    qm, rm = np.linalg.qr(g)
    qm = qm * np.sign(np.diag(rm))[None, :]
    p = qm.astype(np.float32)
    return np.ascontiguousarray(np.broadcast_to(p, (spec.kv_heads, HEAD_DIM, spec.rank)))


def generate(spec: Spec, threads: int = 8) -> Workload:
    """Draw every input of one workload (deterministic in ``spec``)."""
    B, Hkv, Hq, T, D = spec.batch, spec.kv_heads, spec.q_heads, spec.max_tokens, HEAD_DIM
    G = spec.group
    qrng = np.random.default_rng([spec.seed, _S_Q])
    q = qrng.standard_normal((B, Hq, D), dtype=np.float32).astype(np.float16)
    seq_lens = _seq_lens(spec)
    needles = _needle_blocks(spec, seq_lens)
    offset = None
    if spec.key_offset_std:
        offset = (np.random.default_rng([spec.seed, _S_OFFSET])
                  .standard_normal((Hkv, D)) * spec.key_offset_std).astype(np.float32)
    outliers = None
    if spec.outlier_channels:
        orng = np.random.default_rng([spec.seed, _S_OUTLIER])
        outliers = np.stack([np.sort(orng.choice(D, spec.outlier_channels, replace=False))
                             for _ in range(Hkv)])

    k = np.empty((B, Hkv, T, D), dtype=np.float16)
    v = np.empty((B, Hkv, T, D), dtype=np.float16)
    assign = np.empty((B, Hkv, T), dtype=np.int32) if spec.granularity == "cluster" else None
    tail_k = tail_v = None
    if spec.n_tail:
        tail_k = np.zeros((B, Hkv, spec.n_tail, BLOCK, D), dtype=np.uint16)
        tail_v = np.zeros_like(tail_k)
    col_sum = np.zeros((B, Hkv, D), dtype=np.float64)
    col_cnt = np.zeros((B,), dtype=np.int64)

    def work(bh):
        b, h = bh
        qm = q[b, h * G:(h + 1) * G].astype(np.float64).mean(axis=0)
        qdir = qm / max(np.linalg.norm(qm), 1e-30)
        if assign is not None:
            xk, assign[b, h] = _cluster_keys(spec, b, h, qdir)
        else:
            xk = _unit_keys(spec, b, h, qdir, offset, outliers, needles[b][h])
        xv = _unit_values(spec, b, h)
        k[b, h] = xk.astype(np.float16)
        v[b, h] = xv.astype(np.float16)
        n_pages = -(-int(seq_lens[b]) // BLOCK)
        packed = max(0, n_pages - spec.n_tail)
        if spec.n_tail:
            for s in range(spec.n_tail):
                page = n_pages - spec.n_tail + s
                if page >= 0:
                    sl = slice(page * BLOCK, (page + 1) * BLOCK)
                    tail_k[b, h, s] = _bf16_bits(xk[sl])
                    tail_v[b, h, s] = _bf16_bits(xv[sl])
        col_sum[b, h] = k[b, h, :packed * BLOCK].astype(np.float64).sum(axis=0)
        col_cnt[b] = packed * BLOCK

    units = [(b, h) for b in range(B) for h in range(Hkv)]
    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(work, units))

    proj = None
    if spec.granularity != "block":
        key_center = np.zeros((Hkv, D), dtype=np.float32)
        global_scale = np.ones((Hkv,), dtype=np.float32)
        proj = _proj(spec) if spec.granularity == "token" else None
    else:
        total = max(int(col_cnt.sum()), 1)
        key_center = (col_sum.sum(axis=0) / total).astype(np.float32)
        global_scale = calibrate_scale(spec, k, seq_lens, key_center, threads)
    value_scale = None
    if spec.value_fmt == "nvfp4":
        value_scale = calibrate_value_scale(spec, v, seq_lens, threads)
    return Workload(spec, q, k, v, seq_lens, key_center, global_scale,
                    tail_k, tail_v, proj, needles, value_scale, assign)


def calibrate_scale(spec: Spec, k: np.ndarray, seq_lens: np.ndarray,
                    key_center: np.ndarray, threads: int = 8) -> np.ndarray:
    """Per-KV-head FP32 scale: largest |key - center| over the packed region / 2688."""
    Hkv = spec.kv_heads
    amax = np.zeros((spec.batch, Hkv), dtype=np.float32)

    def work(bh):
        b, h = bh
        n_pages = -(-int(seq_lens[b]) // BLOCK)
        packed = max(0, n_pages - spec.n_tail) * BLOCK
        if packed:
            y = k[b, h, :packed].astype(np.float32) - key_center[h][None, :]
            amax[b, h] = np.abs(y).max()

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(work, [(b, h) for b in range(spec.batch) for h in range(Hkv)]))
    s = (amax.max(axis=0) / np.float32(NVFP4_MAX)).astype(np.float32)
    s[s == 0] = np.float32(1.0)
    return s


def calibrate_value_scale(spec: Spec, v: np.ndarray, seq_lens: np.ndarray,
                          threads: int = 8) -> np.ndarray:
    """Per-KV-head FP32 scale of the value store: largest |v| over t < L_b / 2688."""
    amax = np.zeros((spec.batch, spec.kv_heads), dtype=np.float32)

    def work(bh):
        b, h = bh
        L = int(seq_lens[b])
        if L:
            amax[b, h] = np.abs(v[b, h, :L].astype(np.float32)).max()

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        list(ex.map(work, [(b, h) for b in range(spec.batch) for h in range(spec.kv_heads)]))
    s = (amax.max(axis=0) / np.float32(NVFP4_MAX)).astype(np.float32)
    s[s == 0] = np.float32(1.0)
    return s


def algorithmic_bytes(w: Workload, kept_tokens: Optional[int] = None) -> Dict[str, int]:
    """Bytes the method must move per decode step (scan + selected K,V), per stage.

    Block mode: 72 B per scanned token (64 B of E2M1 codes + 8 B of E4M3 scales)
    and 2 x 256 B per attended token (FP16 K and V rows; BF16 tail rows also
    count 512 B), or 256 + 72 B with the 4-bit value store (tail rows still
    512 B). Token mode: 2r B (BF16) or r B (FP8) per scanned token (the
    projected key) and 512 B per selected token. With the adaptive budget the
    number of selected tokens depends on the scores: pass it as kept_tokens
    (the sum of the step's counts over all units); likewise in cluster mode
    (512 B of FP32 centroid and 4 B of offset per block scanned, then the chosen
    blocks' tokens, whose number depends on their sizes).
    """
    s = w.spec
    scan = attn = 0
    for b in range(s.batch):
        L = int(w.seq_lens[b])
        if s.granularity == "block":
            packed = w.packed_blocks(b)
            scanned_tokens = min(packed * BLOCK, L)
            scan += s.kv_heads * 72 * scanned_tokens
            n_pages = w.n_pages(b)
            forced = min(s.n_tail, n_pages)
            chosen = min(s.budget - s.n_tail, packed) + forced
            # every chosen page is a full 128-token tile except the newest one
            tail_tokens = 0
            for p in range(n_pages - forced, n_pages):
                tail_tokens += min(BLOCK, L - p * BLOCK)
            main_tokens = (chosen - forced) * BLOCK if forced else min(chosen * BLOCK, L)
            row = 256 + (72 if s.value_fmt == "nvfp4" else 256)
            attn += s.kv_heads * (512 * tail_tokens + row * main_tokens)
        elif s.granularity == "token":
            scan += s.kv_heads * (1 if s.proj_fmt == "fp8" else 2) * s.rank * L
            attn += s.kv_heads * (256 + (72 if s.value_fmt == "nvfp4" else 256)) * min(s.budget, L)
        else:  # cluster: FP32 centroids and the offsets; the chosen tokens' K, V rows
            scan += s.kv_heads * (512 * s.n_clusters + 4 * (s.n_clusters + 1))
            attn += s.kv_heads * (256 + (72 if s.value_fmt == "nvfp4" else 256)) * min(s.budget, L)
    if kept_tokens is not None:
        attn = (256 + (72 if s.value_fmt == "nvfp4" else 256)) * int(kept_tokens)
    q_bytes = s.batch * s.q_heads * HEAD_DIM * 2
    return {"scan": scan, "attn": attn, "q": q_bytes, "total": scan + attn}
