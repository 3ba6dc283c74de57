"""Decode-step throughput of the sparse attention hot path on one MI355X.

A step is one pass of the whole path for one layer: score_scan (4-bit dense
scan or projected-key scan), select_topk, sparse_decode_attn and combine, over a
batch of synthetic inputs already resident in HBM. By default (--mode auto) a
step is two calls, score_scan and select_attend_combine (the selection, then
the attention with its merge). Consecutive steps rotate over --layers
distinct copies of the KV cache, as consecutive layers of a model would, so no
step finds the previous step's data in the 256 MB Infinity Cache.

Prints one JSON line. `value` is (batch x KV heads) decode steps per second;
`pct_hbm_peak` is the step's algorithmic bytes per second over 8 TB/s;
`dense_same_gpu` is dense FP16 attention (every block selected) on the same
cache and kernels, with the sparse step's speedup over it. `roofline` is the
dominant kernel, the scan, measured with HIP events on the launch stream over
the timed region (recorded on about 8 sampled steps, since each event record
costs the GPU a marker); `components_us` splits a step into scoring, top-B
selection and sparse attention, from an untimed pass of the step as separate
calls; `cpu_baseline` is the CPU oracle timed on a bounded sample of the same
workload.
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
    "scan_block_kernel": ("scan_block_kernel", ["scan.hip", "scan_core.hpp", "select_core.hpp",
                                                "common.hpp"]),
    "scan_token_kernel<32>": ("scan_token_kernel_r32", ["scan.hip", "common.hpp"]),
    "scan_token_kernel<32, fp8>": ("scan_token_kernel_r32_fp8", ["scan.hip", "common.hpp"]),
    "attn_kernel<4, false, false, 0, 1>": ("attn_kernel_g4_token",
                                        ["attn.hip", "attn_core.hpp", "combine_core.hpp",
                                         "select_core.hpp", "common.hpp"]),
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
    ap.add_argument("--event-stride", type=int, default=0,
                    help="record the per-kernel events on every n-th timed step (each event "
                         "record costs the GPU a marker packet); 0: about 8 samples (4 below "
                         "100 steps), with a stride coprime with --layers")
    ap.add_argument("--warmup-ms", type=float, default=1500.0,
                    help="after the --warmup steps, keep warming up (untimed) until this much "
                         "wall time has passed, so clocks and address translations settle")
    ap.add_argument("--mode", default="auto",
                    choices=["auto", "scoresel", "fused", "three", "split", "step"],
                    help="auto: fused; "
                         "scoresel: score_select, attend_combine; "
                         "fused: score_scan, select_attend_combine; "
                         "three: score_scan, select_topk, attend_combine; "
                         "split: score_scan, select_topk, sparse_decode_attn, combine; "
                         "step: decode_step")
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
    if d0.cluster_mode:  # every block fits: the choice, then the attention
        dense_call = lambda: (dd.score_select_clusters(), dd.attend_combine())
    else:
        dense_call = dd.select_attend_combine
    for _ in range(2):
        dense_call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        dense_call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    row = 256 + (72 if s.value_fmt == "nvfp4" else 256)  # a K row and a V row
    dense_bytes = s.kv_heads * row * int(d0.w.seq_lens.astype("int64").sum())
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

    # threads it can use: the BLAS pool (NumPy's matrix products) within the
    # process's CPU affinity; every other NumPy step runs on one core
    try:
        affinity = len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        affinity = os.cpu_count() or 1
    try:
        from threadpoolctl import threadpool_info

        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = 1
    cores = max(1, min(blas, affinity))
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
        elif s.granularity == "cluster":
            rec = O.cluster_index(w.k[b, h], w.assign[b, h], s.n_clusters, int(w.seq_lens[b]))
        else:
            rec = O.project_keys(w.k[b, h], w.proj[h], s.proj_fmt)
        vst = None
        if s.value_fmt == "nvfp4":
            s_v = np.float32(w.value_scale[h])
            vst = (*O.pack_values(w.v[b, h], s_v), s_v)
        packed.append((b, h, rec, vst))
    log(f"[cpu] {len(packed)} units packed in {time.perf_counter() - t_start:.1f} s")

    def step(b, h, rec, vst):
        L = int(w.seq_lens[b])
        qg = w.q[b, h * G:(h + 1) * G]
        if s.granularity == "block":
            rc, rs = rec
            tk = w.tail_k[b, h] if s.n_tail else None
            tv = w.tail_v[b, h] if s.n_tail else None
            sc = O.scan_block_unit(O.scan_query(qg, s.query_fmt), rc, rs, w.global_scale[h],
                                   w.key_center[h], L, s.n_tail, sigma, s.max_blocks)
            idx, _ = O.select_blocks_unit(sc, L, s.n_tail, s.budget)
            rows = lambda sel: O.gather_rows_block(w.k[b, h], w.v[b, h], sel, L, s.n_tail, tk, tv,
                                                   v_store=vst)
        elif s.granularity == "cluster":
            cent, off, mem = rec
            sc = O.cluster_scores(qg, cent, np.diff(off), sigma)
            ch, _ = O.select_clusters(sc, np.diff(off), s.budget)
            idx, _ = O.cluster_tokens(ch, off, mem, s.budget)
            rows = lambda sel: O.gather_rows_token(w.k[b, h], w.v[b, h], [t for t in sel if t < L],
                                                   v_store=vst)
        else:
            sc = O.scan_token_unit(qg, rec, w.proj[h], L, sigma, s.proj_fmt)
            if s.top_p > 0:
                idx, _ = O.select_tokens_top_p(sc, L, s.budget, s.top_p)
            else:
                idx, _ = O.select_tokens_unit(sc, L, s.budget)
            rows = lambda sel: O.gather_rows_token(w.k[b, h], w.v[b, h], [t for t in sel if t < L],
                                                   v_store=vst)
        po, pl = O.attend_splits(qg, idx, 1, rows, sigma)
        O.combine(po, pl)

    done, spent = 0, 0.0
    while spent < budget_s / 2 or done == 0:
        for b, h, rec, vst in packed:
            t0 = time.perf_counter()
            step(b, h, rec, vst)
            spent += time.perf_counter() - t0
            done += 1
    log(f"[cpu] {done} unit steps in {spent:.1f} s")
    return {"value": done / spent, "unit": "steps/s", "cores": int(cores), "kind": "oracle",
            "threads": f"BLAS pool {blas} within an affinity of {affinity} cores; "
                       "the non-BLAS steps run on one core",
            "sample": f"{len(packed)} of {len(order)} (sequence, KV head) units of the same "
                      f"workload, packed once (pack not timed), then stepped {done} times "
                      f"(scan, select, attention, combine; NumPy float64) in {spent:.1f} s"}


def event_stride(steps: int, layers: int, requested: int) -> int:
    """Stride of the sampled steps: the requested one, else about 8 samples (4
    below 100 steps: a sampled step's three event markers cost the GPU about
    10 us, measured at 128K context, batch 16, 4 KV heads: 20 steps ran at
    72.5% of peak with 7 sampled and at 74.2% with none), coprime with the
    layer rotation so that every layer copy is sampled."""
    if requested > 0:
        return requested
    s = max(1, steps // (4 if steps < 100 else 8))
    while math.gcd(s, layers) != 1:
        s += 1
    return s


def component_split(layers, cluster: bool, steps: int = 24):
    """JSSA Figure 9's split of a decode step (candidate scoring, top-B
    selection, sparse attention) from an untimed pass of the step as separate
    calls (score_scan, select_topk, attend_combine; in cluster mode
    score_clusters, select_clusters, attend and combine), every call bracketed
    by HIP events on the launch stream. The scoring prep (the group's mean query
    and its projection, or the block scan's query stage) runs inside the scoring
    kernel's first microseconds."""
    import numpy as np
    import torch

    from block_sparse_attention_pack_amd.step import step_calls

    form = "split" if cluster else "three"
    parts = (["scoring", "top_selection", "sparse_attention", "sparse_attention"] if cluster
             else ["scoring", "top_selection", "sparse_attention"])
    stream = torch.cuda.current_stream()
    for i in range(4):  # settle: one step per layer copy
        for c in step_calls(layers[i % len(layers)], form):
            c()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(parts) + 1)]
          for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        e = ev[i]
        e[0].record(stream)
        for j, c in enumerate(step_calls(layers[i % len(layers)], form)):
            c()
            e[j + 1].record(stream)
    torch.cuda.synchronize()
    out = {}
    for name in dict.fromkeys(parts):
        js = [j for j, p in enumerate(parts) if p == name]
        ts = [sum(ev[i][j].elapsed_time(ev[i][j + 1]) for j in js) * 1e3 for i in range(1, steps)]
        out[name] = round(float(np.median(ts)), 2)
    out["calls"] = form
    out["steps"] = steps - 1
    out["statistic"] = "median of the per-step event times (the first step, after an idle queue, left out)"
    return out


def percentiles(xs):
    import numpy as np

    return [round(float(np.percentile(xs, q)), 2) for q in (10, 50, 90)]


def check_after_timing(layers, calls, steps: int) -> None:
    """The timed steps completed as they should: every counter word is back at
    zero (a bounded wait that gave up leaves the fault word set), and one
    layer's output is reproduced bit for bit by an untimed step."""
    import torch

    for d in layers:
        bad = int(torch.count_nonzero(d.counters))
        assert bad == 0, f"{bad} counter words are not zero after the timed steps"
    d = layers[(steps - 1) % len(layers)]
    out, lse = d.out.clone(), d.out_lse.clone()
    for c in calls(d):
        c()
    torch.cuda.synchronize()
    assert torch.equal(out, d.out) and torch.equal(torch.nan_to_num(lse), torch.nan_to_num(d.out_lse)), \
        "an untimed step did not reproduce the timed step's output"


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
    from block_sparse_attention_pack_amd.step import default_form, forms_of, step_calls, upload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    binding.load()
    spec = W.SPECS[a.workload]
    log(f"[bench] generating {spec.name} ...")
    t0 = time.time()
    w = W.generate(spec, threads=16)
    log(f"[bench] generated in {time.time() - t0:.1f} s; uploading")
    if a.mode == "auto":
        a.mode = default_form(spec.granularity)
    d0 = upload(w, splits=a.splits)
    d0.pack()
    torch.cuda.synchronize()
    layers = [d0]
    for i in range(1, a.layers):
        if d0.block_mode:
            layers.append(dataclasses.replace(d0, k=d0.k.clone(), v=d0.v.clone(),
                                              codes=d0.codes.clone(), scales=d0.scales.clone()))
        elif d0.cluster_mode:
            layers.append(dataclasses.replace(d0, k=d0.k.clone(), v=d0.v.clone(),
                                              centroids=d0.centroids.clone(),
                                              offsets=d0.offsets.clone(),
                                              members=d0.members.clone()))
        else:
            layers.append(dataclasses.replace(d0, k=d0.k.clone(), v=d0.v.clone(),
                                              kproj=d0.kproj.clone()))
    torch.cuda.synchronize()
    log(f"[bench] {a.layers} layer copies resident; warmup {a.warmup}")
    nbytes = W.algorithmic_bytes(w)
    stream = torch.cuda.current_stream()

    stages = forms_of(spec.granularity)[a.mode]
    calls = lambda d: step_calls(d, a.mode)
    # untimed warm-up: the --warmup steps, then more in batches of 16 until
    # --warmup-ms of wall time has passed (short runs of a few steps otherwise
    # time a GPU whose clocks have not settled)
    t_warm = time.perf_counter()
    warm_steps = 0
    while True:
        n_batch = max(a.warmup - warm_steps, 0) if warm_steps < a.warmup else 16
        for _ in range(n_batch):
            for c in calls(layers[warm_steps % len(layers)]):
                c()
            warm_steps += 1
        torch.cuda.synchronize()
        if warm_steps >= a.warmup and (time.perf_counter() - t_warm) * 1e3 >= a.warmup_ms:
            break
    warm_ms = (time.perf_counter() - t_warm) * 1e3
    kept = None
    if spec.top_p > 0 or d0.cluster_mode:  # the attention reads the tokens kept
        if a.warmup == 0:
            for c in calls(d0):
                c()
            torch.cuda.synchronize()
        kept = int(layers[max(a.warmup - 1, 0) % len(layers)].count.sum())
        nbytes = W.algorithmic_bytes(w, kept_tokens=kept)

    ns = len(stages)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(ns + 1)] for _ in range(a.steps)]
    stride = event_stride(a.steps, a.layers, a.event_stride)
    # sampled steps start at the second one: the first follows a synchronize
    # with an empty queue, so its events would also time the launch latency
    sample0 = 1 if a.steps > 1 else 0
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(a.steps):
        cs = calls(layers[i % len(layers)])
        if a.no_stage_events or i < sample0 or (i - sample0) % stride:
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
    stage_us, stage_pct = {}, {}
    sampled = [] if a.no_stage_events else list(range(sample0, a.steps, stride))
    if sampled:
        for j, name in enumerate(stages):
            ts = [ev[i][j].elapsed_time(ev[i][j + 1]) * 1e3 for i in sampled]
            stage_us[name] = float(np.mean(ts))
            stage_pct[name] = percentiles(ts)
        step_us = [ev[i][0].elapsed_time(ev[i][ns]) * 1e3 for i in sampled]
        stage_pct["step"] = percentiles(step_us)
    log(f"[bench] {a.steps} steps in {elapsed * 1e3:.2f} ms after {warm_steps} warm-up steps "
        f"({warm_ms:.0f} ms); stages (us): {stage_pct}")
    check_after_timing(layers, calls, a.steps)

    # the dominant kernel: the scan (timed where it is a call of its own); in
    # cluster mode the attention (the centroids are the smaller read)
    if d0.cluster_mode:
        scan_stage, kbytes = "attend_combine", nbytes["attn"]
        kname = "attn_kernel<%d, false, false, %d, 1>" % (spec.group, int(d0.value_store))
    else:
        scan_stage, kbytes = "scan", nbytes["scan"]
        kname = ("scan_block_kernel" if d0.block_mode else "scan_token_kernel<%d%s>"
                 % (spec.rank, ", fp8" if spec.proj_fmt == "fp8" else ""))
    kern_us = stage_us.get(scan_stage)
    roofline = None
    if kern_us:
        achieved = kbytes / (kern_us * 1e-6) / 1e9
        roofline = {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1),
                    "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                    "traffic": measured_traffic(kname, spec.name),
                    "bytes_per_launch": kbytes,
                    "events": f"{scan_stage} stage, {len(sampled)} sampled steps, mean"}
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
                   else ("f32 centroids of %d coarse blocks" % spec.n_clusters
                         if d0.cluster_mode
                         else "%s rank-%d keys, f32" % (spec.proj_fmt, spec.rank)),
                   "values": ("nvfp4 store (e2m1 * e4m3 * s_v), f32 acc"
                              if spec.value_fmt == "nvfp4" else "f16 cache, f32 acc")},
        "pct_hbm_peak": round(100.0 * step_gbs / PEAK_HBM_GBS, 2),
        "algorithmic_bytes_per_step": nbytes["total"],
        "stages_us": {k: round(v, 2) for k, v in stage_us.items()},
        "stages_us_p10_p50_p90": stage_pct,
        "stage_events": None if not sampled else
        f"{len(sampled)} of {a.steps} timed steps (every {stride}th from step {sample0})",
        "warmup_run": {"steps": warm_steps, "ms": round(warm_ms, 1)},
        "roofline": roofline,
        "components_us": component_split(layers, d0.cluster_mode),
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
