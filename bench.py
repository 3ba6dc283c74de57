"""Decode-step throughput of the sparse attention hot path on one MI355X.

A step is one pass of the whole path for one layer: score_scan (4-bit dense
scan or projected-key scan), select_topk, sparse_decode_attn and combine, over a batch of
synthetic inputs already resident in HBM. By default (--mode auto) a block-mode
step with at least 16384 scanned blocks and sequence lengths that differ is one
decode_step launch, every other step two calls, score_scan and
select_attend_combine. Consecutive steps rotate
over --layers distinct copies of the KV cache, as consecutive layers of a model
would, so no step finds the previous step's data in the 256 MB Infinity Cache.

Prints one JSON line. `value` is (batch x KV heads) decode steps per second;
`pct_hbm_peak` is the step's algorithmic bytes per second over 8 TB/s;
`dense_same_gpu` is dense FP16 attention (every block selected) on the same
cache and kernels, with the sparse step's speedup over it. `roofline` is the
dominant kernel (the one-launch step kernel, which is the whole step, or else the
scan) measured with HIP events on the
launch stream over the timed region (recorded on every --event-stride-th step,
since each event record costs the GPU a marker); `cpu_baseline` is the CPU oracle timed on
a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse decode-attention steps/sec (batch x KV heads) at 128K; % HBM peak"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
# rocprofv3 counter summaries of a kernel's HBM traffic (FETCH_SIZE + WRITE_SIZE,
# calibrated on a copy of known size) in profiles/<kernel>.<workload>.traffic.md,
# valid while the kernel's sources (listed here) are unchanged
TRAFFIC_SOURCES = {  # kernel: (file name stem, sources)
    "scan_block_kernel": ("scan_block_kernel", ["scan.hip", "scan_core.hpp", "common.hpp"]),
    "scan_token_kernel<32>": ("scan_token_kernel_r32", ["scan.hip", "common.hpp"]),
    "scan_token_kernel<32, fp8>": ("scan_token_kernel_r32_fp8", ["scan.hip", "common.hpp"]),
    "step_kernel": ("step_kernel", ["step.hip", "scan_core.hpp", "attn_core.hpp",
                                    "select_core.hpp", "combine_core.hpp", "common.hpp"]),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    from block_sparse_attention_pack_amd.workloads import ORDER

    ap.add_argument("--workload", default="jetqsparse", choices=ORDER)
    ap.add_argument("--layers", type=int, default=4, help="distinct KV-cache copies rotated per step")
    ap.add_argument("--splits", type=int, default=None)
    ap.add_argument("--no-dense", dest="dense", action="store_false",
                    help="skip the dense-attention reference on the same GPU")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of the CPU oracle sample (0 disables it)")
    ap.add_argument("--no-stage-events", action="store_true",
                    help="time only the whole step, without per-kernel events")
    ap.add_argument("--event-stride", type=int, default=25,
                    help="record the per-kernel events on every n-th timed step (each event "
                         "record costs the GPU a marker packet)")
    ap.add_argument("--mode", default="auto",
                    choices=["auto", "step", "fused", "scoresel", "three", "split"],
                    help="auto: step where the one-launch step pays off (block mode, "
                         ">= 16384 scanned blocks, ragged lengths), else fused; "
                         "step: decode_step (one launch in block mode); "
                         "fused: score_scan, select_attend_combine; "
                         "scoresel: score_select, attend_combine; "
                         "three: score_scan, select_topk, attend_combine; "
                         "split: score_scan, select_topk, sparse_decode_attn, combine")
    return ap.parse_args()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, or None when it
    covers another kernel or workload, or the kernel's sources changed since."""
    if kernel not in TRAFFIC_SOURCES:
        return None
    stem, sources = TRAFFIC_SOURCES[kernel]
    try:
        with open(os.path.join(ROOT, "profiles", f"{stem}.{workload}.traffic.md")) as f:
            fields = dict(re.findall(r"^(\w+): (.+)$", f.read(), re.M))
        h = hashlib.sha256()
        for name in sources:
            with open(os.path.join(ROOT, "block_sparse_attention_pack_amd", "csrc", name), "rb") as f:
                h.update(f.read())
    except OSError:
        return None
    if fields.get("kernel") != kernel or fields.get("workload") != workload:
        return None
    if fields.get("source_sha256") != h.hexdigest():
        return None
    return int(float(fields["traffic_bytes_per_launch"]))


def dense_same_gpu(d0, sparse_ms: float, steps: int = 10):
    """Dense FP16 attention on the same GPU and cache: the same kernels with the
    budget set to every block (every token in token mode), timed per step."""
    import torch

    s = d0.w.spec
    full = s.max_blocks if d0.block_mode else s.max_tokens
    dd = d0.with_budget(full)
    stream = torch.cuda.current_stream()
    for _ in range(2):
        dd.select_attend_combine()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        dd.select_attend_combine()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    dense_bytes = s.kv_heads * 512 * int(d0.w.seq_lens.astype("int64").sum())  # every K, V row
    del dd
    return {"ms_per_step": round(ms, 4), "steps": steps, "budget": full,
            "bytes_per_step": dense_bytes,
            "pct_hbm_peak": round(100.0 * dense_bytes / (ms * 1e-3) / (PEAK_HBM_GBS * 1e9), 2),
            "sparse_speedup": round(ms / sparse_ms, 3)}


def cpu_baseline(w, budget_s: float):
    """The oracle (float64 NumPy) timed on a bounded sample of the workload's units.

    Units are packed (untimed: the pack is not part of the step) until half the
    budget is spent, then the step (scan, select, attention, combine) is run over
    them, round after round, for the other half; the rate is units stepped per
    second of step time.
    """
    import numpy as np

    from oracle import decode as O

    try:
        from threadpoolctl import threadpool_info

        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    s = w.spec
    G, sigma = s.group, w.softmax_scale
    order = [(b, h) for b in range(s.batch) for h in range(s.kv_heads)]
    rng = np.random.default_rng(0)
    order = [order[i] for i in rng.permutation(len(order))]
    t_start = time.perf_counter()
    packed = []
    for b, h in order:
        if packed and time.perf_counter() - t_start >= budget_s / 2:
            break
        if s.granularity == "block":
            rec = O.pack_unit_blocks(w.k[b, h], w.key_center[h], w.global_scale[h], 0,
                                     s.max_blocks)
        else:
            rec = O.project_keys(w.k[b, h], w.proj[h], s.proj_fmt)
        packed.append((b, h, rec))
    log(f"[cpu] {len(packed)} units packed in {time.perf_counter() - t_start:.1f} s")

    def step(b, h, rec):
        L = int(w.seq_lens[b])
        qg = w.q[b, h * G:(h + 1) * G]
        if s.granularity == "block":
            rc, rs = rec
            tk = w.tail_k[b, h] if s.n_tail else None
            tv = w.tail_v[b, h] if s.n_tail else None
            sc = O.scan_block_unit(O.scan_query(qg, s.query_fmt), rc, rs, w.global_scale[h],
                                   w.key_center[h], L, s.n_tail, sigma, s.max_blocks)
            idx, _ = O.select_blocks_unit(sc, L, s.n_tail, s.budget)
            rows = lambda sel: O.gather_rows_block(w.k[b, h], w.v[b, h], sel, L, s.n_tail, tk, tv)
        else:
            sc = O.scan_token_unit(qg, rec, w.proj[h], L, sigma, s.proj_fmt)
            if s.top_p > 0:
                idx, _ = O.select_tokens_top_p(sc, L, s.budget, s.top_p)
            else:
                idx, _ = O.select_tokens_unit(sc, L, s.budget)
            rows = lambda sel: O.gather_rows_token(w.k[b, h], w.v[b, h], [t for t in sel if t < L])
        po, pl = O.attend_splits(qg, idx, 1, rows, sigma)
        O.combine(po, pl)

    done, spent = 0, 0.0
    while spent < budget_s / 2 or done == 0:
        for b, h, rec in packed:
            t0 = time.perf_counter()
            step(b, h, rec)
            spent += time.perf_counter() - t0
            done += 1
    log(f"[cpu] {done} unit steps in {spent:.1f} s")
    return {"value": done / spent, "unit": "steps/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{len(packed)} of {len(order)} (sequence, KV head) units of the same "
                      f"workload, packed once (pack not timed), then stepped {done} times "
                      f"(scan, select, attention, combine; NumPy float64) in {spent:.1f} s"}


def main() -> int:
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {a.gpus} is not supported "
              "(the path shards by (sequence, KV head) with no exchange; run one process per GPU)",
              file=sys.stderr)
        return 2
    import numpy as np
    import torch

    from block_sparse_attention_pack_amd import binding, workloads as W
    from block_sparse_attention_pack_amd.step import one_launch_pays, upload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    binding.load()
    spec = W.SPECS[a.workload]
    log(f"[bench] generating {spec.name} ...")
    t0 = time.time()
    w = W.generate(spec, threads=16)
    log(f"[bench] generated in {time.time() - t0:.1f} s; uploading")
    if a.mode == "auto":
        ragged = len(set(int(x) for x in w.seq_lens)) > 1
        a.mode = "step" if one_launch_pays(spec.units, spec.max_blocks, spec.granularity,
                                           ragged) else "fused"
    d0 = upload(w, splits=a.splits, one_launch=a.mode == "step")
    d0.pack()
    torch.cuda.synchronize()
    layers = [d0]
    for i in range(1, a.layers):
        if d0.block_mode:
            layers.append(dataclasses.replace(d0, k=d0.k.clone(), v=d0.v.clone(),
                                              codes=d0.codes.clone(), scales=d0.scales.clone()))
        else:
            layers.append(dataclasses.replace(d0, k=d0.k.clone(), v=d0.v.clone(),
                                              kproj=d0.kproj.clone()))
    torch.cuda.synchronize()
    log(f"[bench] {a.layers} layer copies resident; warmup {a.warmup}")
    nbytes = W.algorithmic_bytes(w)
    stream = torch.cuda.current_stream()

    if a.mode == "step":
        stages = ["decode_step"]
        calls = lambda d: [d.decode_step]
    elif a.mode == "fused":
        stages = ["scan", "select_attend_combine"]
        calls = lambda d: [d.scan, d.select_attend_combine]
    elif a.mode == "scoresel":
        stages = ["score_select", "attend_combine"]
        calls = lambda d: [d.score_select, d.attend_combine]
    elif a.mode == "three":
        stages = ["scan", "select", "attend_combine"]
        calls = lambda d: [d.scan, d.select, d.attend_combine]
    else:
        stages = ["scan", "select", "attend", "combine"]
        calls = lambda d: [d.scan, d.select, d.attend, d.combine]
    for i in range(a.warmup):
        for c in calls(layers[i % len(layers)]):
            c()
    torch.cuda.synchronize()
    kept = None
    if spec.top_p > 0:  # the adaptive budget: the attention reads the tokens kept
        if a.warmup == 0:
            for c in calls(d0):
                c()
            torch.cuda.synchronize()
        kept = int(layers[max(a.warmup - 1, 0) % len(layers)].count.sum())
        nbytes = W.algorithmic_bytes(w, kept_tokens=kept)

    ns = len(stages)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(ns + 1)] for _ in range(a.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    stride = max(1, a.event_stride)
    for i in range(a.steps):
        cs = calls(layers[i % len(layers)])
        if a.no_stage_events or i % stride:
            for c in cs:
                c()
            continue
        e = ev[i]
        e[0].record(stream)
        for j, c in enumerate(cs):
            c()
            e[j + 1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = elapsed * 1e3 / a.steps
    units = spec.batch * spec.kv_heads
    value = units * a.steps / elapsed
    stage_us = {}
    if not a.no_stage_events:
        sampled = range(0, a.steps, stride)
        for j, name in enumerate(stages):
            ts = [ev[i][j].elapsed_time(ev[i][j + 1]) * 1e3 for i in sampled]
            stage_us[name] = float(np.mean(ts))
        step_us = [ev[i][0].elapsed_time(ev[i][ns]) * 1e3 for i in sampled]
        stage_us["step_events_p50"] = float(np.median(step_us))
    log(f"[bench] {a.steps} steps in {elapsed * 1e3:.2f} ms; stages (us): {stage_us}")

    # the dominant kernel: the whole step when it is one launch, else the scan
    one_launch = a.mode == "step" and d0.block_mode
    kern_us = stage_us.get("decode_step" if one_launch else "scan")
    kbytes = nbytes["total" if one_launch else "scan"]
    roofline = None
    if kern_us:
        achieved = kbytes / (kern_us * 1e-6) / 1e9
        if one_launch:
            kname = "step_kernel"
        else:
            kname = ("scan_block_kernel" if d0.block_mode else "scan_token_kernel<%d%s>"
                     % (spec.rank, ", fp8" if spec.proj_fmt == "fp8" else ""))
        roofline = {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1),
                    "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                    "traffic": measured_traffic(kname, spec.name),
                    "bytes_per_launch": kbytes}
    step_gbs = nbytes["total"] / (ms_per_step * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": spec.name, "batch": spec.batch, "kv_heads": spec.kv_heads,
                   "q_heads": spec.q_heads, "context": spec.max_tokens,
                   "granularity": spec.granularity, "budget": spec.budget,
                   "tail_pages": spec.n_tail, "splits": d0.splits, "layers_rotated": a.layers,
                   "calls": a.mode,
                   **({"top_p": spec.top_p, "kept_tokens_per_step": kept} if kept is not None
                      else {}),
                   "scan": ("%s query, e2m1*e4m3 keys -> f16 MFMA, f32 acc" % spec.query_fmt)
                   if d0.block_mode
                   else "%s rank-%d keys, f32" % (spec.proj_fmt, spec.rank)},
        "pct_hbm_peak": round(100.0 * step_gbs / PEAK_HBM_GBS, 2),
        "algorithmic_bytes_per_step": nbytes["total"],
        "stages_us": {k: round(v, 2) for k, v in stage_us.items()},
        "stage_events": None if a.no_stage_events else f"every {stride}th timed step",
        "roofline": roofline,
    }
    if a.dense:
        log("[bench] timing dense attention on the same GPU")
        out["dense_same_gpu"] = dense_same_gpu(d0, ms_per_step)
    if a.cpu_seconds > 0:
        log("[bench] timing the CPU oracle on a sample")
        out["cpu_baseline"] = cpu_baseline(w, a.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
