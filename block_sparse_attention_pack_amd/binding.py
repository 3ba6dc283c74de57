"""ctypes binding of libbsa.so: argument marshalling only.

Every entry point of include/bsa.h has a function of the same name here (without
the ``bsa_`` prefix) taking torch tensors; it passes their device pointers and
the current HIP stream to the library and raises :class:`BsaError` on a non-zero
return code. No step of the decode path runs in Python.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbsa.so")

DTYPE_F16, DTYPE_BF16 = 0, 1
BLOCK, TOKEN, CLUSTER = 0, 1, 2
PROJ_BF16, PROJ_FP8 = 0, 1
QUERY_F16, QUERY_NVFP4 = 0, 1
VALUE_CACHE, VALUE_NVFP4 = 0, 1

ERRORS = {-1: "INVALID_ARG", -2: "UNSUPPORTED", -3: "HIP", -4: "WORKSPACE"}


class BsaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"bsa error {code} ({ERRORS.get(code, '?')}): {msg}")
        self.code = code


class KvLayout(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_tokens", ctypes.c_int32),
        ("kv_stride_b", ctypes.c_int64),
        ("kv_stride_h", ctypes.c_int64),
        ("kv_stride_t", ctypes.c_int64),
        ("kv_dtype", ctypes.c_int32),
        ("value_dtype", ctypes.c_int32),
    ]


class SelectCfg(ctypes.Structure):
    _fields_ = [
        ("granularity", ctypes.c_int32),
        ("budget", ctypes.c_int32),
        ("n_tail_pages", ctypes.c_int32),
        ("proj_rank", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("proj_dtype", ctypes.c_int32),
        ("query_dtype", ctypes.c_int32),
        ("top_p", ctypes.c_float),
        ("num_clusters", ctypes.c_int32),
    ]


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the library once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    try:
        # PyTorch ships its own libamdhip64.so.7; this library binds to whichever
        # copy the process loads first, and torch's kernels only run on its own
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m block_sparse_attention_pack_amd.build`")
    lib = ctypes.CDLL(path)
    LP, CP = ctypes.POINTER(KvLayout), ctypes.POINTER(SelectCfg)
    sig = {
        "bsa_pack_kv_cache": [LP, CP, _P, _P, _P, _P, _I32, _I32, _P, _P, _P, _P],
        "bsa_pack_values": [LP, _P, _P, _I32, _I32, _P, _P],
        "bsa_build_cluster_index": [LP, CP, _P, _P, _P, _P, _P, _P, _P],
        "bsa_score_clusters": [LP, CP, _P, _P, _P, _P, _P],
        "bsa_select_clusters": [LP, CP, _P, _P, _P, _P, _P, _P],
        "bsa_score_select_clusters": [LP, CP, _P, _P, _P, _P, _P, _P, _P, _P],
        "bsa_score_scan": [LP, CP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
        "bsa_select_topk": [LP, CP, _P, _P, _P, ctypes.c_size_t, _P, _P, _P],
        "bsa_sparse_decode_attn": [LP, CP, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P],
        "bsa_combine": [_I32, _I32, _I32, _P, _P, _P, _P, _P],
        "bsa_score_select": [LP, CP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                             _P, _P, _P],
        "bsa_attend_combine": [LP, CP, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _P, _P, _P, _P,
                               _P],
        "bsa_select_attend_combine": [LP, CP, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P, _P,
                                      _I32, _P, _P, _P, _P, _P, _P, _P, _P],
        "bsa_decode_step": [LP, CP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _P,
                            ctypes.c_size_t, _P, _P, _P, _P, _P, _P, _P, _P],
        "bsa_append_token": [LP, CP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
        "bsa_decode_step_noalloc": [LP, CP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32,
                                    _P, _P, _P],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.bsa_workspace_size.argtypes = [LP, CP]
    lib.bsa_workspace_size.restype = ctypes.c_size_t
    lib.bsa_counters_size.argtypes = [LP]
    lib.bsa_counters_size.restype = ctypes.c_size_t
    lib.bsa_value_store_size.argtypes = [LP]
    lib.bsa_value_store_size.restype = ctypes.c_size_t
    lib.bsa_last_error.argtypes = []
    lib.bsa_last_error.restype = ctypes.c_char_p
    lib.bsa_version.argtypes = []
    lib.bsa_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != 0:
        raise BsaError(rc, load().bsa_last_error().decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def layout_for(k, num_q_heads: int, dtype: Optional[int] = None,
               value_dtype: int = VALUE_CACHE) -> KvLayout:
    """Layout of a [B, Hkv, T, 128] K (or V) tensor (any strides with channel stride 1);
    value_dtype VALUE_NVFP4 says that the steps read V from a 4-bit value store."""
    import torch

    B, Hkv, T, D = k.shape
    if k.stride(3) != 1:
        raise ValueError("head_dim must be contiguous")
    if dtype is None:
        dtype = {torch.float16: DTYPE_F16, torch.bfloat16: DTYPE_BF16}[k.dtype]
    return KvLayout(B, Hkv, num_q_heads, D, 128, T, k.stride(0), k.stride(1), k.stride(2), dtype,
                    value_dtype)


def select_cfg(granularity: int, budget: int, n_tail_pages: int = 0, proj_rank: int = 0,
               softmax_scale: Optional[float] = None, head_dim: int = 128,
               proj_dtype: int = PROJ_BF16, query_dtype: int = QUERY_F16,
               top_p: float = 0.0, num_clusters: int = 0) -> SelectCfg:
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(head_dim)
    return SelectCfg(granularity, budget, n_tail_pages, proj_rank, softmax_scale, proj_dtype,
                     query_dtype, top_p, num_clusters)


def version() -> str:
    return load().bsa_version().decode()


def pack_kv_cache(layout, cfg, k, key_center, global_scale, proj, block_begin, block_end,
                  codes, scales, kproj, stream=None) -> None:
    lib = load()
    _check(lib.bsa_pack_kv_cache(ctypes.byref(layout), ctypes.byref(cfg), _ptr(k),
                                 _ptr(key_center), _ptr(global_scale), _ptr(proj), block_begin,
                                 block_end, _ptr(codes), _ptr(scales), _ptr(kproj),
                                 _stream(stream)))


def value_store_size(layout) -> int:
    return int(load().bsa_value_store_size(ctypes.byref(layout)))


def pack_values(layout, v, value_scale, block_begin, block_end, store, stream=None) -> None:
    lib = load()
    _check(lib.bsa_pack_values(ctypes.byref(layout), _ptr(v), _ptr(value_scale), block_begin,
                               block_end, _ptr(store), _stream(stream)))


def score_scan(layout, cfg, q, codes, scales, global_scale, key_center, kproj, proj, seq_lens,
               scores, stream=None) -> None:
    lib = load()
    _check(lib.bsa_score_scan(ctypes.byref(layout), ctypes.byref(cfg), _ptr(q), _ptr(codes),
                              _ptr(scales), _ptr(global_scale), _ptr(key_center), _ptr(kproj),
                              _ptr(proj), _ptr(seq_lens), _ptr(scores), _stream(stream)))


def workspace_size(layout, cfg) -> int:
    return int(load().bsa_workspace_size(ctypes.byref(layout), ctypes.byref(cfg)))


def select_topk(layout, cfg, scores, seq_lens, workspace, workspace_bytes, idx, count,
                stream=None) -> None:
    lib = load()
    _check(lib.bsa_select_topk(ctypes.byref(layout), ctypes.byref(cfg), _ptr(scores),
                               _ptr(seq_lens), _ptr(workspace), workspace_bytes, _ptr(idx),
                               _ptr(count), _stream(stream)))


def sparse_decode_attn(layout, cfg, q, k, v, seq_lens, idx, count, tail_k, tail_v, num_splits,
                       part_o, part_lse, stream=None) -> None:
    lib = load()
    _check(lib.bsa_sparse_decode_attn(ctypes.byref(layout), ctypes.byref(cfg), _ptr(q), _ptr(k),
                                      _ptr(v), _ptr(seq_lens), _ptr(idx), _ptr(count),
                                      _ptr(tail_k), _ptr(tail_v), num_splits, _ptr(part_o),
                                      _ptr(part_lse), _stream(stream)))


def combine(rows, num_splits, head_dim, part_o, part_lse, out, out_lse, stream=None) -> None:
    lib = load()
    _check(lib.bsa_combine(rows, num_splits, head_dim, _ptr(part_o), _ptr(part_lse), _ptr(out),
                           _ptr(out_lse), _stream(stream)))


def counters_size(layout) -> int:
    return int(load().bsa_counters_size(ctypes.byref(layout)))


def score_select(layout, cfg, q, codes, scales, global_scale, key_center, kproj, proj, seq_lens,
                 scores, workspace, workspace_bytes, idx, count, stream=None) -> None:
    lib = load()
    _check(lib.bsa_score_select(ctypes.byref(layout), ctypes.byref(cfg), _ptr(q), _ptr(codes),
                                _ptr(scales), _ptr(global_scale), _ptr(key_center), _ptr(kproj),
                                _ptr(proj), _ptr(seq_lens), _ptr(scores), _ptr(workspace),
                                workspace_bytes, _ptr(idx), _ptr(count), _stream(stream)))


def attend_combine(layout, cfg, q, k, v, seq_lens, idx, count, tail_k, tail_v, num_splits,
                   part_o, part_lse, counters, out, out_lse, stream=None) -> None:
    lib = load()
    _check(lib.bsa_attend_combine(ctypes.byref(layout), ctypes.byref(cfg), _ptr(q), _ptr(k),
                                  _ptr(v), _ptr(seq_lens), _ptr(idx), _ptr(count), _ptr(tail_k),
                                  _ptr(tail_v), num_splits, _ptr(part_o), _ptr(part_lse),
                                  _ptr(counters), _ptr(out), _ptr(out_lse), _stream(stream)))


def select_attend_combine(layout, cfg, q, k, v, seq_lens, scores, workspace, workspace_bytes,
                          tail_k, tail_v, num_splits, idx, count, part_o, part_lse, counters, out,
                          out_lse, stream=None) -> None:
    lib = load()
    _check(lib.bsa_select_attend_combine(
        ctypes.byref(layout), ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(seq_lens),
        _ptr(scores), _ptr(workspace), workspace_bytes, _ptr(tail_k), _ptr(tail_v), num_splits,
        _ptr(idx), _ptr(count), _ptr(part_o), _ptr(part_lse), _ptr(counters), _ptr(out),
        _ptr(out_lse), _stream(stream)))


def decode_step(layout, cfg, q, codes, scales, global_scale, key_center, kproj, proj, k, v,
                seq_lens, tail_k, tail_v, num_splits, scores, workspace, workspace_bytes, idx,
                count, part_o, part_lse, counters, out, out_lse, stream=None) -> None:
    lib = load()
    _check(lib.bsa_decode_step(
        ctypes.byref(layout), ctypes.byref(cfg), _ptr(q), _ptr(codes), _ptr(scales),
        _ptr(global_scale), _ptr(key_center), _ptr(kproj), _ptr(proj), _ptr(k), _ptr(v),
        _ptr(seq_lens), _ptr(tail_k), _ptr(tail_v), num_splits, _ptr(scores), _ptr(workspace),
        workspace_bytes, _ptr(idx), _ptr(count), _ptr(part_o), _ptr(part_lse), _ptr(counters),
        _ptr(out), _ptr(out_lse), _stream(stream)))


def append_token(layout, cfg, k_new, v_new, seq_lens, k, v, key_center, global_scale, proj,
                 codes, scales, kproj, tail_k, tail_v, stream=None) -> None:
    lib = load()
    _check(lib.bsa_append_token(
        ctypes.byref(layout), ctypes.byref(cfg), _ptr(k_new), _ptr(v_new), _ptr(seq_lens),
        _ptr(k), _ptr(v), _ptr(key_center), _ptr(global_scale), _ptr(proj), _ptr(codes),
        _ptr(scales), _ptr(kproj), _ptr(tail_k), _ptr(tail_v), _stream(stream)))


def decode_step_noalloc(layout, cfg, q, codes, scales, global_scale, key_center, kproj, proj, k,
                        v, seq_lens, tail_k, tail_v, num_splits, out, out_lse,
                        stream=None) -> None:
    lib = load()
    _check(lib.bsa_decode_step_noalloc(
        ctypes.byref(layout), ctypes.byref(cfg), _ptr(q), _ptr(codes), _ptr(scales),
        _ptr(global_scale), _ptr(key_center), _ptr(kproj), _ptr(proj), _ptr(k), _ptr(v),
        _ptr(seq_lens), _ptr(tail_k), _ptr(tail_v), num_splits, _ptr(out), _ptr(out_lse),
        _stream(stream)))


def build_cluster_index(layout, cfg, k, assign, seq_lens, centroids, offsets, members,
                        stream=None) -> None:
    lib = load()
    _check(lib.bsa_build_cluster_index(ctypes.byref(layout), ctypes.byref(cfg), _ptr(k),
                                       _ptr(assign), _ptr(seq_lens), _ptr(centroids),
                                       _ptr(offsets), _ptr(members), _stream(stream)))


def score_clusters(layout, cfg, q, centroids, offsets, scores, stream=None) -> None:
    lib = load()
    _check(lib.bsa_score_clusters(ctypes.byref(layout), ctypes.byref(cfg), _ptr(q),
                                  _ptr(centroids), _ptr(offsets), _ptr(scores), _stream(stream)))


def select_clusters(layout, cfg, scores, offsets, members, idx, count, stream=None) -> None:
    lib = load()
    _check(lib.bsa_select_clusters(ctypes.byref(layout), ctypes.byref(cfg), _ptr(scores),
                                   _ptr(offsets), _ptr(members), _ptr(idx), _ptr(count),
                                   _stream(stream)))


def score_select_clusters(layout, cfg, q, centroids, offsets, members, scores, idx, count,
                          stream=None) -> None:
    lib = load()
    _check(lib.bsa_score_select_clusters(ctypes.byref(layout), ctypes.byref(cfg), _ptr(q),
                                         _ptr(centroids), _ptr(offsets), _ptr(members),
                                         _ptr(scores), _ptr(idx), _ptr(count), _stream(stream)))
