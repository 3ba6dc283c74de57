"""HBM read-rate probe: the ceiling the decode step's kernels are held against.

Runs ``bsa_probe_read`` (include/bsa_probe.h) over the two byte patterns of the
block-mode step and prints one JSON line per case:

* ``contiguous``: 604 MB read as 144 KiB contiguous runs, one per work-group
  (the block scan's 4-bit key records at 128K context, batch 16, 4 KV heads);
* ``tiles32k``: 8192 tiles of 32 KiB at seeded random tile-aligned offsets of a
  16 GiB region (the attention's selected key and value blocks: 64 units x 64
  blocks x K and V), 16 or 32 tiles per work-group;
* ``rows256``: the token-mode attention's rows at 128K context, batch 8, 8 KV
  heads, 2048 tokens per unit: for each of the 64 units 2048 distinct seeded
  random tokens (ascending, as the selection lists them), each a 256-byte key
  row and a 256-byte value row of a 2 GiB K and a 2 GiB V cache, 512 rows per
  work-group (the attention's 8 splits per unit), 16 threads per row.

Each launch reads a different quarter of its buffer, so no launch finds the
previous one's bytes in the 256 MB Infinity Cache. The rate is bytes read over
the mean HIP-event time of the timed launches.

Usage: python -m block_sparse_attention_pack_amd.probe [--reps N] [--quick] [--only PATTERN]
"""

from __future__ import annotations

import argparse
import ctypes
import json
import sys

from . import binding

SCAN_BYTES = 64 * 1024 * 9216         # 64 units x 1024 blocks x 9 KiB
ATTN_TILES = 64 * 64 * 2              # 64 units x 64 blocks, K and V
TILE = 32 * 1024
REGION = 4 << 30                      # one layer's K or V (4 GiB); 4 regions
TOK_UNITS, TOK_T, TOK_PICKS, ROW = 64, 131072, 2048, 256  # token mode's rows


def _fn():
    lib = binding.load()
    fn = lib.bsa_probe_read
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                   ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                   ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    return fn


def time_case(buf, nbytes_region, tile_offs, n_tiles, tile_bytes, per_group, mode, depth,
              reps, sink):
    """Mean seconds per launch; launch i reads region i % 4 (tile_offs: a list of
    4 device offset tensors, or None for contiguous runs)."""
    import torch

    fn = _fn()
    stream = torch.cuda.current_stream()
    base = buf.data_ptr()

    def launch(i):
        r = i % 4
        if tile_offs is None:
            rc = fn(base + r * nbytes_region, nbytes_region, None, n_tiles, tile_bytes,
                    per_group, mode, depth, sink.data_ptr(), stream.cuda_stream)
        else:
            rc = fn(base, buf.numel(), tile_offs[r].data_ptr(), n_tiles, tile_bytes, per_group,
                    mode, depth, sink.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"bsa_probe_read returned {rc}")

    for i in range(8):
        launch(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(reps):
        launch(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / reps


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--reps", type=int, default=40)
    ap.add_argument("--quick", action="store_true", help="one depth per mode")
    ap.add_argument("--only", choices=["contiguous", "tiles32k", "rows256"], default=None)
    a = ap.parse_args()
    import numpy as np
    import torch

    assert torch.cuda.is_available(), "the probe needs a GPU"
    binding.load()
    sink = torch.zeros(1 << 20, dtype=torch.int32, device="cuda")
    cases = []
    want = lambda p: a.only is None or a.only == p
    depths = {0: [8] if a.quick else [2, 4, 8], 1: [16] if a.quick else [8, 16, 32],
              2: [8] if a.quick else [2, 4, 8]}
    if want("contiguous"):
        contiguous(a, depths, sink, cases)
    if want("tiles32k"):
        tiles32k(a, depths, sink, cases)
    if want("rows256"):
        rows256(a, depths, sink, cases)
    pats = sorted({c["pattern"] for c in cases})
    best = {p: max(c["GBps"] for c in cases if c["pattern"] == p) for p in pats}
    print(json.dumps({"read_ceiling_GBps": best, "peak_GBps": 8000.0}), flush=True)
    return 0


def contiguous(a, depths, sink, cases):
    import torch

    # contiguous runs: 4 regions of SCAN_BYTES
    region = SCAN_BYTES
    buf = torch.empty(4 * region, dtype=torch.uint8, device="cuda")
    buf.random_(0, 256)
    run = 144 * 1024
    n = region // run
    for mode in (0, 1):
        for depth in depths[mode]:
            t = time_case(buf, region, None, n, run, 1, mode, depth, a.reps, sink)
            cases.append({"pattern": "contiguous", "bytes": n * run, "run_bytes": run,
                          "mode": ["vgpr", "lds"][mode], "depth": depth,
                          "us": round(t * 1e6, 2), "GBps": round(n * run / t / 1e9, 1)})
            print(json.dumps(cases[-1]), flush=True)
    del buf
    torch.cuda.synchronize()


def tiles32k(a, depths, sink, cases):
    import numpy as np
    import torch

    # random 32 KiB tiles from a 16 GiB region, offsets drawn per launch region
    total = 4 * REGION
    buf = torch.empty(total, dtype=torch.uint8, device="cuda")
    buf.random_(0, 256)
    rng = np.random.default_rng(5)
    offs = []
    for r in range(4):
        t = rng.choice(REGION // TILE, size=ATTN_TILES, replace=False).astype(np.int64)
        o = r * REGION + t * TILE
        assert o.min() >= 0 and o.max() + TILE <= total and np.all(o % 16 == 0)
        offs.append(torch.from_numpy(o).cuda())
    for per in (16, 32):
        for mode in (0, 1):
            for depth in depths[mode]:
                t = time_case(buf, REGION, offs, ATTN_TILES, TILE, per, mode, depth, a.reps,
                              sink)
                cases.append({"pattern": "tiles32k", "bytes": ATTN_TILES * TILE,
                              "tiles_per_group": per, "mode": ["vgpr", "lds"][mode],
                              "depth": depth, "us": round(t * 1e6, 2),
                              "GBps": round(ATTN_TILES * TILE / t / 1e9, 1)})
                print(json.dumps(cases[-1]), flush=True)
    del buf
    torch.cuda.synchronize()


def rows256(a, depths, sink, cases):
    """Launch r reads the rows of region r (a layer's 2 GiB K cache, then its
    2 GiB V cache): per unit, per run of 16 selected tokens, their 16 key rows
    then their 16 value rows."""
    import numpy as np
    import torch

    half = TOK_UNITS * TOK_T * ROW  # one layer's K (or V): 2 GiB
    total = 4 * 2 * half
    buf = torch.empty(total, dtype=torch.uint8, device="cuda")
    buf.random_(0, 256)
    rng = np.random.default_rng(6)
    n = TOK_UNITS * TOK_PICKS * 2
    offs = []
    for r in range(4):
        kbase = r * 2 * half
        rows = []
        for u in range(TOK_UNITS):
            tok = np.sort(rng.choice(TOK_T, size=TOK_PICKS, replace=False)).astype(np.int64)
            k = kbase + (u * TOK_T + tok) * ROW
            kv = np.stack([k.reshape(-1, 16), (k + half).reshape(-1, 16)], axis=1)
            rows.append(kv.reshape(-1))
        o = np.concatenate(rows)
        assert o.size == n and o.min() >= 0 and o.max() + ROW <= total and np.all(o % 16 == 0)
        offs.append(torch.from_numpy(o).cuda())
    per = 512  # rows of one split: 256 tokens, K and V
    for depth in depths[2]:
        t = time_case(buf, 2 * half, offs, n, ROW, per, 2, depth, a.reps, sink)
        cases.append({"pattern": "rows256", "bytes": n * ROW, "rows_per_group": per,
                      "mode": "rows", "depth": depth, "us": round(t * 1e6, 2),
                      "GBps": round(n * ROW / t / 1e9, 1)})
        print(json.dumps(cases[-1]), flush=True)
    del buf
    torch.cuda.synchronize()


if __name__ == "__main__":
    sys.exit(main())
