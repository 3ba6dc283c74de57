"""The C ABI library: builds, loads without a GPU, exports every declared
entry point and rejects bad arguments before touching the device (CPU)."""

import ctypes
import os
import re

import pytest

from block_sparse_attention_pack_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from block_sparse_attention_pack_amd import build

        build.build()
    return B.load()


def declared_functions():
    text = "".join(open(os.path.join(ROOT, "include", h)).read()
                   for h in sorted(os.listdir(os.path.join(ROOT, "include"))) if h.endswith(".h"))
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?(bsa_[a-z_]+)\(", text, re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["bsa_pack_kv_cache", "bsa_score_scan", "bsa_select_topk",
              "bsa_sparse_decode_attn", "bsa_combine", "bsa_workspace_size",
              "bsa_decode_step", "bsa_append_token", "bsa_last_error", "bsa_version"]:
        assert n in names, n


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert "gfx950" in B.version()


def _layout(**kw):
    base = dict(batch=1, num_kv_heads=1, num_q_heads=4, head_dim=128, block_size=128,
                max_tokens=4096, kv_stride_b=4096 * 128, kv_stride_h=4096 * 128,
                kv_stride_t=128, kv_dtype=B.DTYPE_F16)
    base.update(kw)
    return B.KvLayout(**base)


FAKE = 1 << 20  # never dereferenced: every call below fails its argument checks


def _scan(lib, layout, cfg, q=FAKE):
    return lib.bsa_score_scan(ctypes.byref(layout), ctypes.byref(cfg), q, FAKE, FAKE, FAKE,
                              None, None, None, FAKE, FAKE, None)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=64), -2),
    (dict(block_size=64), -2),
    (dict(num_kv_heads=4, num_q_heads=6), -1),
    (dict(num_q_heads=12), -2),
    (dict(max_tokens=1000), -1),
    (dict(kv_stride_t=100), -1),
    (dict(kv_dtype=7), -2),
    (dict(value_dtype=7), -2),
])
def test_bad_layouts_are_rejected(lib, kw, code):
    cfg = B.select_cfg(B.BLOCK, 8)
    assert _scan(lib, _layout(**kw), cfg) == code
    assert lib.bsa_last_error().decode()


@pytest.mark.parametrize("cfg,code", [
    (B.SelectCfg(B.BLOCK, 0, 0, 0, 0.1), -1),
    (B.SelectCfg(B.BLOCK, 40, 0, 0, 0.1), -1),  # more blocks than the cache holds
    (B.SelectCfg(B.BLOCK, 1, 2, 0, 0.1), -1),   # budget below the forced pages
    (B.SelectCfg(B.BLOCK, 8, 3, 0, 0.1), -1),
    (B.SelectCfg(B.BLOCK, 8, 0, 0, 0.0), -1),
    (B.SelectCfg(B.TOKEN, 64, 0, 24, 0.1), -2),  # rank 24 unsupported
    (B.SelectCfg(B.TOKEN, 64, 1, 32, 0.1), -1),  # token mode has no tail pages
    (B.SelectCfg(5, 8, 0, 0, 0.1), -1),
])
def test_bad_configs_are_rejected(lib, cfg, code):
    assert _scan(lib, _layout(), cfg) == code


def test_null_and_misaligned_pointers_are_rejected(lib):
    L, cfg = _layout(), B.select_cfg(B.BLOCK, 8)
    assert _scan(lib, L, cfg, q=None) == -1
    assert _scan(lib, L, cfg, q=FAKE + 2) == -1
    rc = lib.bsa_sparse_decode_attn(ctypes.byref(L), ctypes.byref(cfg), FAKE, FAKE, FAKE, FAKE,
                                    FAKE, FAKE, None, None, 9, FAKE, FAKE, None)
    assert rc == -1 and "num_splits" in lib.bsa_last_error().decode()
    tail = B.select_cfg(B.BLOCK, 8, n_tail_pages=2)
    rc = lib.bsa_sparse_decode_attn(ctypes.byref(L), ctypes.byref(tail), FAKE, FAKE, FAKE, FAKE,
                                    FAKE, FAKE, None, None, 2, FAKE, FAKE, None)
    assert rc == -1 and "tail" in lib.bsa_last_error().decode()
    rc = lib.bsa_pack_kv_cache(ctypes.byref(L), ctypes.byref(cfg), FAKE, None, FAKE, None,
                               0, 33, FAKE, FAKE, None, None)
    assert rc == -1
    assert lib.bsa_combine(4, 2, 64, FAKE, FAKE, FAKE, None, None) == -2
    assert lib.bsa_combine(4, 0, 128, FAKE, FAKE, FAKE, None, None) == -1
    assert lib.bsa_combine(0, 1, 128, None, None, None, None, None) == 0  # nothing to do


def test_value_store_size_and_pack_checks(lib):
    L = _layout(batch=3, num_kv_heads=2, num_q_heads=8, value_dtype=B.VALUE_NVFP4)
    assert lib.bsa_value_store_size(ctypes.byref(L)) == 72 * 3 * 2 * 4096 + 4 * 2
    assert lib.bsa_value_store_size(ctypes.byref(_layout(batch=0))) == 0
    assert lib.bsa_value_store_size(None) == 0
    rc = lib.bsa_pack_values(ctypes.byref(L), FAKE, FAKE, 0, 33, FAKE, None)
    assert rc == -1 and "block range" in lib.bsa_last_error().decode()
    assert lib.bsa_pack_values(ctypes.byref(L), FAKE, FAKE, 0, 32, None, None) == -1
    assert lib.bsa_pack_values(ctypes.byref(L), FAKE, None, 0, 32, FAKE, None) == -1
    assert lib.bsa_pack_values(ctypes.byref(L), FAKE + 8, FAKE, 0, 32, FAKE, None) == -1
    assert lib.bsa_pack_values(None, FAKE, FAKE, 0, 32, FAKE, None) == -1
    assert lib.bsa_pack_values(ctypes.byref(_layout(head_dim=64)), FAKE, FAKE, 0, 1, FAKE,
                               None) == -2


def test_workspace_size(lib):
    L = _layout()
    assert lib.bsa_workspace_size(ctypes.byref(L), ctypes.byref(B.select_cfg(B.BLOCK, 8))) == 0
    bad = B.select_cfg(B.BLOCK, 8)
    bad.budget = -1
    assert lib.bsa_workspace_size(ctypes.byref(L), ctypes.byref(bad)) == 0
    # token mode: budgets up to 2048 (with or without top_p) select in one launch, which
    # adds a per-unit region (arrival counter, counts, an 8192-entry list per
    # 32768-token chunk)
    L2 = _layout(batch=2, num_kv_heads=3, num_q_heads=6)
    size = lambda budget, top_p=0.0: lib.bsa_workspace_size(
        ctypes.byref(L2), ctypes.byref(B.select_cfg(B.TOKEN, budget, 0, 32, top_p=top_p)))
    assert size(2048) - size(4096) == 6 * (64 + 2 * 8192) * 4
    assert size(300, top_p=0.5) == size(2048)


def test_combined_calls_check_their_arguments(lib):
    L, cfg = _layout(), B.select_cfg(B.BLOCK, 8)
    tok = B.select_cfg(B.TOKEN, 64, 0, 32)
    ws = lib.bsa_workspace_size(ctypes.byref(L), ctypes.byref(tok))
    assert ws > 0  # token selection needs its workspace
    # score_select: token mode without its workspace
    rc = lib.bsa_score_select(ctypes.byref(L), ctypes.byref(tok), FAKE, None, None, None, None,
                              FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, FAKE, None)
    assert rc == -4 and "workspace" in lib.bsa_last_error().decode()
    # attend_combine: the arrival counters are required
    rc = lib.bsa_attend_combine(ctypes.byref(L), ctypes.byref(cfg), FAKE, FAKE, FAKE, FAKE, FAKE,
                                FAKE, None, None, 2, FAKE, FAKE, None, FAKE, None, None)
    assert rc == -4
    # select_attend_combine (block mode: the selection, then the attention)
    args = lambda scores, splits, counters: (
        ctypes.byref(L), ctypes.byref(cfg), FAKE, FAKE, FAKE, FAKE, scores, None, 0, None, None,
        splits, FAKE, FAKE, FAKE, FAKE, counters, FAKE, None, None)
    assert lib.bsa_select_attend_combine(*args(None, 2, FAKE)) == -1
    assert "scores" in lib.bsa_last_error().decode()
    assert lib.bsa_select_attend_combine(*args(FAKE, 9, FAKE)) == -1  # more splits than budget
    assert lib.bsa_select_attend_combine(*args(FAKE, 2, None)) == -4
    # token mode goes through select_topk first: its workspace check comes first
    rc = lib.bsa_select_attend_combine(ctypes.byref(L), ctypes.byref(tok), FAKE, FAKE, FAKE, FAKE,
                                       FAKE, None, 0, None, None, 2, FAKE, FAKE, FAKE, FAKE, FAKE,
                                       FAKE, None, None)
    assert rc == -4
    # one merge arrival word per unit
    assert lib.bsa_counters_size(ctypes.byref(L)) == 4
    assert lib.bsa_counters_size(ctypes.byref(_layout(batch=3, num_kv_heads=2))) == 4 * 6


def test_decode_step_checks_every_stage_first(lib):
    L, cfg = _layout(), B.select_cfg(B.BLOCK, 8)
    tok = B.select_cfg(B.TOKEN, 64, 0, 32)

    def step(c, codes=FAKE, kproj=None, splits=2, scores=FAKE, ws_bytes=0, counters=FAKE,
             out=FAKE, k=FAKE, ws=None):
        return lib.bsa_decode_step(
            ctypes.byref(L), ctypes.byref(c), FAKE, codes, FAKE, FAKE, None, kproj, FAKE, k,
            FAKE, FAKE, None, None, splits, scores, ws, ws_bytes, FAKE, FAKE, FAKE, FAKE,
            counters, out, None, None)

    assert step(cfg, codes=None) == -1  # the scan's key copy
    assert "codes" in lib.bsa_last_error().decode()
    assert step(cfg, scores=None) == -1
    assert step(cfg, k=FAKE + 2) == -1  # attention operands
    assert step(cfg, splits=9) == -1 and "num_splits" in lib.bsa_last_error().decode()
    assert step(cfg, counters=None) == -4
    assert step(cfg, out=None) == -1
    assert step(tok, codes=None, kproj=FAKE) == -4  # token mode: the selection's workspace
    assert step(tok, codes=None, kproj=None) == -1


def test_projected_cache_format_is_checked(lib):
    L = _layout()
    fp8 = B.select_cfg(B.TOKEN, 64, 0, 32, proj_dtype=B.PROJ_FP8)
    assert lib.bsa_workspace_size(ctypes.byref(L), ctypes.byref(fp8)) > 0  # a valid cfg
    assert _scan(lib, L, B.select_cfg(B.TOKEN, 64, 0, 8, proj_dtype=B.PROJ_FP8)) == -2
    assert "FP8" in lib.bsa_last_error().decode()
    assert _scan(lib, L, B.select_cfg(B.TOKEN, 64, 0, 32, proj_dtype=7)) == -2
    assert _scan(lib, L, B.select_cfg(B.BLOCK, 8, proj_dtype=B.PROJ_FP8)) == -1



def test_append_checks_its_arguments(lib):
    L = _layout()
    blk = B.select_cfg(B.BLOCK, 8)
    tail = B.select_cfg(B.BLOCK, 8, n_tail_pages=2)
    tok = B.select_cfg(B.TOKEN, 64, 0, 32)

    def app(c, k_new=FAKE, codes=FAKE, proj=None, kproj=None, tail_k=None):
        return lib.bsa_append_token(ctypes.byref(L), ctypes.byref(c), k_new, FAKE, FAKE, FAKE,
                                    FAKE, None, FAKE, proj, codes, FAKE, kproj, tail_k, tail_k,
                                    None)

    assert app(blk, k_new=None) == -1
    assert app(blk, k_new=FAKE + 2) == -1  # 16-byte alignment
    assert app(blk, codes=None) == -1 and "codes" in lib.bsa_last_error().decode()
    assert app(tail) == -1 and "tail" in lib.bsa_last_error().decode()
    assert app(tail, tail_k=FAKE + 8) == -1
    assert app(tok, codes=None) == -1 and "proj" in lib.bsa_last_error().decode()
    assert app(tok, codes=None, proj=FAKE) == -1


def test_query_format_is_checked(lib):
    L = _layout()
    q4 = B.select_cfg(B.BLOCK, 8, query_dtype=B.QUERY_NVFP4)
    assert lib.bsa_workspace_size(ctypes.byref(L), ctypes.byref(q4)) == 0  # a valid cfg
    assert _scan(lib, L, B.select_cfg(B.BLOCK, 8, query_dtype=5)) == -2
    assert "query_dtype" in lib.bsa_last_error().decode()
    assert _scan(lib, L, B.select_cfg(B.TOKEN, 64, 0, 32, query_dtype=B.QUERY_NVFP4)) == -1
    assert "block mode only" in lib.bsa_last_error().decode()


def test_top_p_is_checked(lib):
    L = _layout()
    ok = B.select_cfg(B.TOKEN, 64, 0, 32, top_p=0.9)
    assert lib.bsa_workspace_size(ctypes.byref(L), ctypes.byref(ok)) > 0  # a valid cfg
    assert _scan(lib, L, B.select_cfg(B.BLOCK, 8, top_p=0.5)) == -1
    assert "token mode only" in lib.bsa_last_error().decode()
    for bad in (-0.1, 1.5, float("nan"), float("inf")):
        assert _scan(lib, L, B.select_cfg(B.TOKEN, 64, 0, 32, top_p=bad)) == -1, bad
        assert "top_p" in lib.bsa_last_error().decode()
    big = _layout(max_tokens=16384, kv_stride_b=16384 * 128, kv_stride_h=16384 * 128)
    assert _scan(lib, big, B.select_cfg(B.TOKEN, 8192, 0, 32, top_p=0.5)) == -2
    assert "4096" in lib.bsa_last_error().decode()
    fixed = B.select_cfg(B.TOKEN, 8192, 0, 32)  # the fixed budget has no such limit
    assert lib.bsa_workspace_size(ctypes.byref(big), ctypes.byref(fixed)) > 0


def test_noalloc_step_rejects_steps_beyond_its_scratch(lib):
    """The allocation-free step keeps its intermediates in a 64 MiB scratch per
    GPU: a token step whose scores alone need 128 MiB is refused before any
    device call."""
    big = _layout(batch=16, num_kv_heads=16, num_q_heads=64, max_tokens=131072,
                  kv_stride_b=16 * 131072 * 128, kv_stride_h=131072 * 128)
    tok = B.select_cfg(B.TOKEN, 2048, 0, 32)
    rc = lib.bsa_decode_step_noalloc(ctypes.byref(big), ctypes.byref(tok), FAKE, None, None,
                                     None, None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 8,
                                     FAKE, None, None)
    assert rc == -4
    msg = lib.bsa_last_error().decode()
    assert "scratch" in msg and str(64 << 20) in msg
    # a bad split count is an argument error
    blk = B.select_cfg(B.BLOCK, 8)
    rc = lib.bsa_decode_step_noalloc(ctypes.byref(_layout()), ctypes.byref(blk), FAKE, FAKE, FAKE,
                                     FAKE, None, None, None, FAKE, FAKE, FAKE, None, None, 9, FAKE,
                                     None, None)
    assert rc == -1 and "num_splits" in lib.bsa_last_error().decode()


def test_probe_checks_its_arguments(lib):
    fn = lib.bsa_probe_read
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                   ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                   ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    # (buf, buf_bytes, tile_off, n_tiles, tile_bytes, tiles_per_group, mode, depth, sink)
    assert fn(None, 1 << 20, None, 4, 256, 4, 0, 8, FAKE, None) == -1      # no buffer
    assert fn(FAKE, 1 << 20, None, 4, 250, 4, 0, 8, FAKE, None) == -1      # not 16-byte tiles
    assert fn(FAKE, 1 << 10, None, 8, 256, 4, 0, 8, FAKE, None) == -1      # past the buffer
    assert fn(FAKE, 1 << 20, None, 4, 4096 + 16, 4, 1, 8, FAKE, None) == -1  # LDS mode: KiB tiles
    assert fn(FAKE, 1 << 20, None, 4, 48, 4, 2, 8, FAKE, None) == -1       # rows: divides 4096
    assert fn(FAKE, 1 << 30, None, 4096, 256, 2048, 2, 8, FAKE, None) == -1  # rows: <= 1024 a group
    assert fn(FAKE, 1 << 20, None, 4, 256, 4, 3, 8, FAKE, None) == -2      # no such mode
    assert fn(FAKE, 1 << 20, None, 4, 256, 4, 0, 3, FAKE, None) == -2      # no such depth
