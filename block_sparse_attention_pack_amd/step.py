"""Device buffers of one decode step and the four-call hot path.

PyTorch only provides device memory and the stream here; every step of the
path runs in libbsa.so kernels through :mod:`block_sparse_attention_pack_amd.binding`.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

from . import binding as bsa
from .workloads import BLOCK, HEAD_DIM, Workload


def default_splits(units: int, budget: int, granularity: str) -> int:
    """Split count of the attention: about 512 work-groups, two per CU (the
    kernel's pipeline runs two waves per SIMD), so every CU streams from the
    first group on. A split keeps at least two blocks (block mode, from 8 units
    up; fewer units are latency-bound and gain from one block per split) or 64
    tokens (token mode)."""
    s = max(1, math.ceil(512 / max(units, 1)))
    if granularity in ("token", "cluster"):
        s = min(s, max(1, budget // 64))  # at least one 16-row group per wave
    elif units >= 8:
        s = min(s, max(1, budget // 2))
    return max(1, min(s, budget))


# Forms of the step as calls of the C ABI (bench.py times one of them).
STEP_FORMS = {
    "scoresel": ["score_select", "attend_combine"],
    "fused": ["scan", "select_attend_combine"],
    "three": ["scan", "select", "attend_combine"],
    "split": ["scan", "select", "attend", "combine"],
    "step": ["decode_step"],
}


# The same for coarse semantic blocks (cluster mode).
CLUSTER_FORMS = {
    "fused": ["score_select_clusters", "attend_combine"],
    "split": ["score_clusters", "select_clusters", "attend", "combine"],
}


def default_form(granularity: str) -> str:
    """The form bench.py times by default: score_scan, then
    select_attend_combine (the selection, the attention and its merge), so
    that the scan is a launch of its own whose rate is timed alone; in cluster
    mode the centroid scoring with the choice, then the attention."""
    return "fused"


def forms_of(granularity: str):
    return CLUSTER_FORMS if granularity == "cluster" else STEP_FORMS


def step_calls(d: "DeviceStep", form: str):
    """The bound methods of one step in the given form."""
    forms = CLUSTER_FORMS if d.cluster_mode else STEP_FORMS
    return [getattr(d, name) for name in forms[form]]


@dataclasses.dataclass
class DeviceStep:
    """Inputs, the key copy and the step's outputs, resident on one GPU."""

    w: Workload
    layout: bsa.KvLayout
    cfg: bsa.SelectCfg
    splits: int
    q: "torch.Tensor"
    k: "torch.Tensor"
    v: "torch.Tensor"  # the V cache, or the 4-bit value store (layout.value_dtype)
    seq_lens: "torch.Tensor"
    key_center: "torch.Tensor"
    global_scale: "torch.Tensor"
    tail_k: Optional["torch.Tensor"]
    tail_v: Optional["torch.Tensor"]
    proj: Optional["torch.Tensor"]
    codes: Optional["torch.Tensor"]
    scales: Optional["torch.Tensor"]
    kproj: Optional["torch.Tensor"]
    scores: "torch.Tensor"
    workspace: Optional["torch.Tensor"]
    ws_bytes: int
    idx: "torch.Tensor"
    count: "torch.Tensor"
    part_o: "torch.Tensor"
    part_lse: "torch.Tensor"
    out: "torch.Tensor"
    out_lse: "torch.Tensor"
    counters: "torch.Tensor"  # arrival counters of the in-kernel merge (zero between calls)
    v_src: Optional["torch.Tensor"] = None  # full-precision V the value store is packed from
    value_scale: Optional["torch.Tensor"] = None  # the value store's FP32 scale per KV head
    assign: Optional["torch.Tensor"] = None  # cluster mode: each token's block, and the index
    centroids: Optional["torch.Tensor"] = None
    offsets: Optional["torch.Tensor"] = None
    members: Optional["torch.Tensor"] = None

    @property
    def cluster_mode(self) -> bool:
        return self.cfg.granularity == bsa.CLUSTER

    @property
    def value_store(self) -> bool:
        return self.layout.value_dtype == bsa.VALUE_NVFP4

    @property
    def block_mode(self) -> bool:
        return self.cfg.granularity == bsa.BLOCK

    # -- the cache build (not part of the timed step) ------------------------
    def pack(self, stream=None) -> None:
        nb = self.w.spec.max_blocks
        if self.cluster_mode:
            bsa.build_cluster_index(self.layout, self.cfg, self.k, self.assign, self.seq_lens,
                                    self.centroids, self.offsets, self.members, stream)
            return
        bsa.pack_kv_cache(self.layout, self.cfg, self.k, self.key_center, self.global_scale,
                          self.proj, 0, nb, self.codes, self.scales, self.kproj, stream)
        if self.value_store:
            bsa.pack_values(self.layout, self.v_src, self.value_scale, 0, nb, self.v, stream)

    # -- the decode step ------------------------------------------------------
    def scan(self, stream=None) -> None:
        bsa.score_scan(self.layout, self.cfg, self.q, self.codes, self.scales,
                       self.global_scale, self.key_center, self.kproj, self.proj,
                       self.seq_lens, self.scores, stream)

    # -- cluster mode ---------------------------------------------------------
    def score_clusters(self, stream=None) -> None:
        bsa.score_clusters(self.layout, self.cfg, self.q, self.centroids, self.offsets,
                           self.scores, stream)

    def select_clusters(self, stream=None) -> None:
        bsa.select_clusters(self.layout, self.cfg, self.scores, self.offsets, self.members,
                            self.idx, self.count, stream)

    def score_select_clusters(self, stream=None) -> None:
        bsa.score_select_clusters(self.layout, self.cfg, self.q, self.centroids, self.offsets,
                                  self.members, self.scores, self.idx, self.count, stream)

    def select(self, stream=None) -> None:
        bsa.select_topk(self.layout, self.cfg, self.scores, self.seq_lens, self.workspace,
                        self.ws_bytes, self.idx, self.count, stream)

    def attend(self, stream=None) -> None:
        bsa.sparse_decode_attn(self.layout, self.cfg, self.q, self.k, self.v, self.seq_lens,
                               self.idx, self.count, self.tail_k, self.tail_v, self.splits,
                               self.part_o, self.part_lse, stream)

    def combine(self, stream=None) -> None:
        rows = self.w.spec.batch * self.w.spec.q_heads
        bsa.combine(rows, self.splits, HEAD_DIM, self.part_o, self.part_lse, self.out,
                    self.out_lse, stream)

    def run(self, stream=None) -> None:
        """The step as four calls: scan, select, attention, combine."""
        if self.cluster_mode:
            self.score_clusters(stream)
            self.select_clusters(stream)
        else:
            self.scan(stream)
            self.select(stream)
        self.attend(stream)
        self.combine(stream)

    # -- the same step as two combined calls ----------------------------------
    def score_select(self, stream=None) -> None:
        bsa.score_select(self.layout, self.cfg, self.q, self.codes, self.scales,
                         self.global_scale, self.key_center, self.kproj, self.proj,
                         self.seq_lens, self.scores, self.workspace, self.ws_bytes,
                         self.idx, self.count, stream)

    def attend_combine(self, stream=None) -> None:
        bsa.attend_combine(self.layout, self.cfg, self.q, self.k, self.v, self.seq_lens,
                           self.idx, self.count, self.tail_k, self.tail_v, self.splits,
                           self.part_o, self.part_lse, self.counters, self.out, self.out_lse,
                           stream)

    def select_attend_combine(self, stream=None) -> None:
        bsa.select_attend_combine(self.layout, self.cfg, self.q, self.k, self.v, self.seq_lens,
                                  self.scores, self.workspace, self.ws_bytes, self.tail_k,
                                  self.tail_v, self.splits, self.idx, self.count, self.part_o,
                                  self.part_lse, self.counters, self.out, self.out_lse, stream)

    def run_two(self, stream=None) -> None:
        """The step as two calls: score_scan, select_attend_combine."""
        self.scan(stream)
        self.select_attend_combine(stream)

    def with_budget(self, budget: int, splits: Optional[int] = None) -> "DeviceStep":
        """The same cache and inputs with another budget (new selection and
        partial buffers); budget = every block or token gives dense attention."""
        import torch

        L = self.layout
        B, Hkv, Hq = L.batch, L.num_kv_heads, L.num_q_heads
        gran = "block" if self.block_mode else ("cluster" if self.cluster_mode else "token")
        cfg = bsa.select_cfg(self.cfg.granularity, budget, self.cfg.n_tail_pages,
                             self.cfg.proj_rank, self.cfg.softmax_scale,
                             proj_dtype=self.cfg.proj_dtype, query_dtype=self.cfg.query_dtype,
                             num_clusters=self.cfg.num_clusters)
        if splits is None:
            splits = default_splits(B * Hkv, budget, gran)
        dev = self.q.device
        ws_bytes = bsa.workspace_size(L, cfg)
        return dataclasses.replace(
            self, cfg=cfg, splits=splits,
            workspace=torch.zeros((ws_bytes,), dtype=torch.uint8, device=dev) if ws_bytes else None,
            ws_bytes=ws_bytes,
            idx=torch.empty((B, Hkv, budget), dtype=torch.int32, device=dev),
            count=torch.empty((B, Hkv), dtype=torch.int32, device=dev),
            part_o=torch.empty((B, Hq, splits, HEAD_DIM), dtype=torch.float32, device=dev),
            part_lse=torch.empty((B, Hq, splits), dtype=torch.float32, device=dev),
            out=torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=dev),
            out_lse=torch.empty((B, Hq), dtype=torch.float32, device=dev))

    def run_fused(self, stream=None) -> None:
        """The step as two calls: score_select, attend_combine."""
        self.score_select(stream)
        self.attend_combine(stream)

    # -- decode-time cache maintenance (not part of the timed step) -----------
    def append(self, k_new, v_new, stream=None) -> None:
        """bsa_append_token: one new token per sequence at seq_lens (the caller
        advances seq_lens afterwards)."""
        bsa.append_token(self.layout, self.cfg, k_new, v_new, self.seq_lens, self.k, self.v,
                         self.key_center, self.global_scale, self.proj, self.codes,
                         self.scales, self.kproj, self.tail_k, self.tail_v, stream)

    # -- the whole step as one call -------------------------------------------
    def decode_step(self, stream=None) -> None:
        """bsa_decode_step: the whole step in one call."""
        bsa.decode_step(self.layout, self.cfg, self.q, self.codes, self.scales,
                        self.global_scale, self.key_center, self.kproj, self.proj, self.k,
                        self.v, self.seq_lens, self.tail_k, self.tail_v, self.splits,
                        self.scores, self.workspace, self.ws_bytes, self.idx, self.count,
                        self.part_o, self.part_lse, self.counters, self.out, self.out_lse,
                        stream)


def upload(w: Workload, device="cuda", splits: Optional[int] = None,
           kv_dtype: str = "f16") -> DeviceStep:
    """Copy a workload to the GPU and allocate every buffer of the step.

    ``kv_dtype="bf16"`` stores K and V as bfloat16 instead (values rounded from
    the fp16 draws), for the BF16-cache variant.
    """
    import torch

    s = w.spec
    B, Hkv, Hq, T = s.batch, s.kv_heads, s.q_heads, s.max_tokens
    dev = torch.device(device)
    t = lambda a: torch.from_numpy(np.array(a, order="C")).to(dev)  # a writable copy
    k = t(w.k)
    v = t(w.v)
    if kv_dtype == "bf16":
        k = k.to(torch.bfloat16)
        v = v.to(torch.bfloat16)
    v4 = s.value_fmt == "nvfp4"
    layout = bsa.layout_for(k, Hq, value_dtype=bsa.VALUE_NVFP4 if v4 else bsa.VALUE_CACHE)
    v_src = value_scale = None
    if v4:
        v_src = v
        value_scale = t(w.value_scale)
        v = torch.zeros((bsa.value_store_size(layout),), dtype=torch.uint8, device=dev)
    gran = {"block": bsa.BLOCK, "token": bsa.TOKEN, "cluster": bsa.CLUSTER}[s.granularity]
    fp8 = gran == bsa.TOKEN and s.proj_fmt == "fp8"
    cfg = bsa.select_cfg(gran, s.budget, s.n_tail, s.rank if gran == bsa.TOKEN else 0,
                         w.softmax_scale, proj_dtype=bsa.PROJ_FP8 if fp8 else bsa.PROJ_BF16,
                         query_dtype=bsa.QUERY_NVFP4 if s.query_fmt == "nvfp4" else bsa.QUERY_F16,
                         top_p=s.top_p, num_clusters=s.n_clusters)
    if splits is None:
        splits = default_splits(B * Hkv, s.budget, s.granularity)
    nb = s.max_blocks
    codes = scales = kproj = proj = None
    assign = centroids = offsets = members = None
    if gran == bsa.CLUSTER:
        C = s.n_clusters
        assign = t(w.assign)
        centroids = torch.empty((B, Hkv, C, HEAD_DIM), dtype=torch.float32, device=dev)
        offsets = torch.empty((B, Hkv, C + 1), dtype=torch.int32, device=dev)
        members = torch.empty((B, Hkv, T), dtype=torch.int32, device=dev)
        scores = torch.empty((B, Hkv, C), dtype=torch.float32, device=dev)
    elif gran == bsa.BLOCK:
        codes = torch.empty((B, Hkv, nb, 8192), dtype=torch.uint8, device=dev)
        scales = torch.empty((B, Hkv, nb, 1024), dtype=torch.uint8, device=dev)
        scores = torch.empty((B, Hkv, nb), dtype=torch.float32, device=dev)
    else:
        kproj = torch.empty((B, Hkv, T, s.rank), dtype=torch.uint8 if fp8 else torch.int16,
                            device=dev)
        proj = t(w.proj)
        scores = torch.empty((B, Hkv, T), dtype=torch.float32, device=dev)
    tail_k = tail_v = None
    if s.n_tail:
        tail_k = t(w.tail_k.view(np.int16))
        tail_v = t(w.tail_v.view(np.int16))
    ws_bytes = bsa.workspace_size(layout, cfg)
    # zero before the first use; every call leaves it so
    workspace = torch.zeros((ws_bytes,), dtype=torch.uint8, device=dev) if ws_bytes else None
    return DeviceStep(
        w=w, layout=layout, cfg=cfg, splits=splits,
        q=t(w.q), k=k, v=v, seq_lens=t(w.seq_lens), key_center=t(w.key_center),
        global_scale=t(w.global_scale), tail_k=tail_k, tail_v=tail_v, proj=proj,
        codes=codes, scales=scales, kproj=kproj, scores=scores, workspace=workspace,
        ws_bytes=ws_bytes,
        idx=torch.empty((B, Hkv, s.budget), dtype=torch.int32, device=dev),
        count=torch.empty((B, Hkv), dtype=torch.int32, device=dev),
        part_o=torch.empty((B, Hq, splits, HEAD_DIM), dtype=torch.float32, device=dev),
        part_lse=torch.empty((B, Hq, splits), dtype=torch.float32, device=dev),
        out=torch.empty((B, Hq, HEAD_DIM), dtype=torch.float32, device=dev),
        out_lse=torch.empty((B, Hq), dtype=torch.float32, device=dev),
        counters=torch.zeros((bsa.counters_size(layout) // 4,), dtype=torch.int32, device=dev),
        v_src=v_src, value_scale=value_scale,
        assign=assign, centroids=centroids, offsets=offsets, members=members,
    )
