#!/usr/bin/env python3
"""Throughput of one DP rank's sharded Adam step on one MI355X.

A step is one sharded_adam_step call on the rank's shard: reduce the D
replica contributions (scaled, fixed rank order), Adam on the fp32
master/m/v shard, bf16 write-back into the owned range; one fused kernel.
Default workload: GPT-2-small-shaped parameter list (124,439,808 elements,
buckets of 40,000,000, D = 8), rank 1's shard (15,554,976 elements), 8 full
bf16 replica buffers in HBM.

Prints one JSON line: elements/s of the step (wall clock over the timed
steps), the HBM roofline of the step kernel (algorithmic bytes (2D+26) per
owned element over its average duration, from HIP events on the launch
stream: one event pair around the timed steps, so that the average is the
region over K), and the CPU oracle timed on a bounded sample beside it.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--rank R]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sharded Adam step: elements/s and HBM GB/s (% of peak) at 1 MI355X"
PEAK_HBM_GBPS = 8000.0
KERNEL_SOURCES = [os.path.join(ROOT, "zero_distributed_optimizer_amd", "csrc", f)
                  for f in ("kernels.hip", "kernels.h", "zdo_internal.h")]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """sha256[:16] over the kernel source and the headers that shape it."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str) -> float | None:
    """HBM bytes per launch of the step kernel from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, calibrated against a plain copy), or
    None if there is none or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"sharded_adam_step_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    src = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not src or not val or src.group(1) != kernel_source_hash():
        return None
    return float(val.group(1))


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="gpt2_small")
    ap.add_argument("--rank", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--stagger", type=int, default=0,
                    help="extra bytes (a multiple of 16) placed between consecutive input buffers")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only: the D ranks' contributions are D "
                          "replica buffers in one GPU's HBM; run with --gpus 1"}), flush=True)
        return 2

    import numpy as np
    import torch

    import workloads as W
    import zero_distributed_optimizer_amd as zdo

    zdo.require_library()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    w = W.get(args.workload)
    rank = w.time_ranks[0] if args.rank is None else args.rank
    D = w.dp_size
    plan = zdo.build_range_map(w.param_numel, w.bucket_numel, D, rank)
    N, Ln, E = plan.buffer_numel, plan.shard_numel, plan.owned_numel
    coords = zdo.WORLD if w.grad_mode == "world" else zdo.LOCAL
    n_rep = N if coords == zdo.WORLD else Ln
    stride = (n_rep + 63) // 64 * 64      # 128-byte-aligned replica buffers
    log(f"workload {w.name}: N={N} D={D} rank={rank} E={E} L={Ln} grads={w.grad_mode}")

    # inputs, resident in HBM before the timed region: the D replicas in one
    # allocation, then the three state arrays in another, each buffer starting
    # on a 128-byte line (plus `stagger` bytes further from the previous one)
    if args.stagger % 16:
        raise SystemExit("--stagger must be a multiple of 16")
    t0 = time.perf_counter()
    gap2, gap4 = args.stagger // 2, args.stagger // 4
    rep_buf = torch.empty(D * (stride + gap2), dtype=torch.bfloat16, device=dev)
    reps = []
    for j in range(D):
        s = rep_buf[j * (stride + gap2): j * (stride + gap2) + n_rep]
        W.normal_bf16(n_rep, w.grad_sigma, W.seed(w.cfg, 0, "grad", j), out=s,
                      probe_fraction=w.probe_fraction, probe_seed=W.seed(w.cfg, 0, "probe", j))
        reps.append(s.view(torch.int16))
    sstride = (Ln + 31) // 32 * 32 + gap4
    state_buf = torch.empty(3 * sstride, dtype=torch.float32, device=dev)
    master, exp_avg, exp_avg_sq = (state_buf[i * sstride: i * sstride + Ln] for i in range(3))
    W.normal_f32(Ln, w.master_sigma, W.seed(w.cfg, 0, "master"), out=master)
    W.normal_f32(Ln, w.m_sigma, W.seed(w.cfg, 0, "m"), out=exp_avg)
    W.square_normal_f32(Ln, w.v_sigma, W.seed(w.cfg, 0, "v"), out=exp_avg_sq)
    params = torch.zeros(n_rep, dtype=torch.int16, device=dev)
    torch.cuda.synchronize(dev)
    log(f"inputs generated in {time.perf_counter() - t0:.1f}s")

    stream = torch.cuda.current_stream(dev)
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay)

    def step(t: int) -> None:
        zdo.sharded_adam_step(plan, reps, coords, w.scale, master, exp_avg, exp_avg_sq, params, coords,
                              step=t, stream=stream, **hp)

    t = 0
    for _ in range(args.warmup):
        t += 1
        step(t)
    torch.cuda.synchronize(dev)

    # timed region: K back-to-back steps between one HIP event pair on the
    # launch stream; the average launch duration is the region over K. An
    # event pair around every launch would drain the queue before and after
    # each step and slow the steps it measures (GPT-2 shape: 96.8 us per step
    # back to back, 98.7-99.6 us per step between per-launch pairs)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    w0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        t += 1
        step(t)
    ev1.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - w0
    ms_per_step = wall * 1e3 / args.steps
    kern_avg_s = ev0.elapsed_time(ev1) / 1e3 / args.steps
    bytes_per_elem = 2 * D + 26
    alg_bytes = E * bytes_per_elem
    achieved = alg_bytes / kern_avg_s / 1e9
    log(f"step: wall {ms_per_step * 1e3:.1f} us/step, kernel avg {kern_avg_s * 1e6:.1f} us, "
        f"{achieved:.0f} GB/s algorithmic")

    # after the timed region: single launches between their own event pairs,
    # for the spread of one launch's duration
    n_iso = min(args.steps, 50)
    iev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_iso)]
    for a, b in iev:
        t += 1
        a.record(stream)
        step(t)
        b.record(stream)
    torch.cuda.synchronize(dev)
    iso_ms = [a.elapsed_time(b) for a, b in iev]
    isolated = {"steps": n_iso, "avg_us": float(np.mean(iso_ms)) * 1e3,
                "p10_us": float(np.percentile(iso_ms, 10)) * 1e3, "p90_us": float(np.percentile(iso_ms, 90)) * 1e3,
                "how": "each launch between its own event pair, after the timed region"}
    log(f"single launches: avg {isolated['avg_us']:.1f} us (p10 {isolated['p10_us']:.1f}, "
        f"p90 {isolated['p90_us']:.1f})")

    # plain-copy reference on the same stream (1 GiB read + 1 GiB write)
    nb = 1 << 30
    src = torch.empty(nb // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        zdo.device_copy(dst, src, stream)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        zdo.device_copy(dst, src, stream)
    c1.record(stream)
    torch.cuda.synchronize(dev)
    copy_gbps = 2 * nb / (c0.elapsed_time(c1) / 1e3 / 10) / 1e9
    log(f"copy reference: {copy_gbps:.0f} GB/s")

    # cold caches: the same step after 1 GiB of ordinary (temporal) reads,
    # which evict the 256 MB Infinity Cache and the L2s as the forward/backward
    # passes of a training step would. Reads, so that no dirty line of the
    # flush is written back during the step; the copy above uses non-temporal
    # accesses, which do not displace cached lines. HIP events around the step
    # kernel only
    n_cold = min(args.steps, 50)
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_cold)]
    for a, b in kev:
        src.sum()
        t += 1
        a.record(stream)
        step(t)
        b.record(stream)
    torch.cuda.synchronize(dev)
    cold_s = float(np.mean([a.elapsed_time(b) for a, b in kev])) / 1e3
    cold = {"kernel_avg_us": cold_s * 1e6, "achieved_gbps": alg_bytes / cold_s / 1e9,
            "frac": alg_bytes / cold_s / 1e9 / PEAK_HBM_GBPS, "elements_per_s": E / cold_s, "steps": n_cold,
            "flush": "torch sum over a 1 GiB buffer (temporal loads) before every step, outside the kernel's "
                     "events"}
    log(f"cold caches: kernel avg {cold_s * 1e6:.1f} us, {cold['achieved_gbps']:.0f} GB/s algorithmic")
    del src, dst

    variants = measure_variants(zdo, torch, np, plan, w, reps, coords, stream, min(args.steps, 50))

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(plan, w, reps, coords, master, exp_avg, exp_avg_sq, args.cpu_seconds)

    traffic = traffic_from_profiles(w.name)
    out = {
        "metric": METRIC,
        "value": E / (ms_per_step / 1e3),
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "params": len(w.param_numel),
            "buffer_elements": N,
            "bucket_elements": w.bucket_numel,
            "buckets": int(plan.buckets().size),
            "dp_size": D,
            "rank": rank,
            "owned_elements": E,
            "grad_replicas": f"{D} x bf16 {'whole buffers' if coords == zdo.WORLD else 'shard slices'}",
            "state": "fp32 master/exp_avg/exp_avg_sq shard",
            "bytes_per_element": bytes_per_elem,
            "buffer_stagger_bytes": args.stagger,
        },
        "hbm_gbps": alg_bytes / (ms_per_step / 1e3) / 1e9,
        "hbm_frac_of_peak": alg_bytes / (ms_per_step / 1e3) / 1e9 / PEAK_HBM_GBPS,
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBPS,
            "traffic": traffic,
        },
        "kernel": {"name": "step_kernel", "avg_us": kern_avg_s * 1e6,
                   "how": "one HIP event pair around the timed steps on the launch stream, divided by the steps",
                   "single_launches": isolated,
                   "source_sha256_16": kernel_source_hash()},
        "cold_cache": cold,
        "variants": variants,
        "copy_reference_gbps": copy_gbps,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


def measure_variants(zdo, torch, np, plan, w, reps, coords, stream, n: int) -> dict:
    """The other device calls on the same inputs: reduce_scatter_local over
    the rank's whole ranges (2D + 2 bytes per element of the ranges), the step
    bucket by bucket, the clipped path, two instances (composed from a
    reduce-scatter within each and the step on both results, and in one
    pass), the parameter all-gather in place (4 bytes per element of the
    other ranks' ranges) and, when the replicas are whole buffers,
    force_all_reduce over the padded buffer (2D + 2 bytes per buffer
    element). Each call timed as n back-to-back calls between one HIP event
    pair."""
    import workloads as W

    D = plan.dp_size
    out = {}

    def timed(fn) -> float:
        """Average seconds per call of n back-to-back calls between one event pair."""
        for _ in range(3):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / 1e3 / n

    ranges = int(sum(b["shard_numel"] for b in plan.buckets()))
    red = torch.empty(plan.shard_numel, dtype=torch.int16, device=reps[0].device)
    t = timed(lambda: zdo.reduce_scatter_local(plan, reps, coords, w.scale, red, zdo.LOCAL, stream))
    gbps = ranges * (2 * D + 2) / t / 1e9
    out["reduce_scatter_local"] = {"elements": ranges, "bytes_per_element": 2 * D + 2, "kernel_avg_us": t * 1e6,
                                   "achieved_gbps": gbps, "frac": gbps / PEAK_HBM_GBPS}
    log(f"reduce_scatter_local: {t * 1e6:.1f} us, {gbps:.0f} GB/s algorithmic")
    del red
    # bucket by bucket: the same step launched once per bucket, last bucket
    # first (the order a backward pass makes them ready), in one timed region
    nb = int(plan.buckets().size)
    st_b = [torch.zeros(plan.shard_numel, dtype=torch.float32, device=reps[0].device) for _ in range(3)]
    par_b = torch.empty(plan.extent(coords), dtype=torch.int16, device=reps[0].device)
    hp_b = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, step=1)

    reps_b = zdo.Buffers(reps, "replicas")   # checked once for the nb launches

    def per_bucket(st=stream):
        for b in reversed(range(nb)):
            zdo.sharded_adam_step(plan, reps_b, coords, w.scale, *st_b, par_b, coords, stream=st,
                                  buckets=(b, b + 1), **hp_b)
    t_b = timed(per_bucket)
    # the same launches replayed from a HIP graph, so that the host's
    # per-launch cost (Python here) does not leave the GPU idle between
    # short launches
    side = torch.cuda.Stream(device=reps[0].device)
    side.wait_stream(torch.cuda.current_stream(reps[0].device))
    with torch.cuda.stream(side):
        per_bucket(None)
    torch.cuda.current_stream(reps[0].device).wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        per_bucket(None)
    t_g = timed(graph.replay)
    gbps = plan.owned_numel * (2 * D + 26) / t_b / 1e9
    out["bucket_by_bucket"] = {"buckets": nb, "total_us": t_b * 1e6, "achieved_gbps": gbps,
                               "frac": gbps / PEAK_HBM_GBPS,
                               "graph_total_us": t_g * 1e6,
                               "graph_achieved_gbps": plan.owned_numel * (2 * D + 26) / t_g / 1e9,
                               "launches": "sharded_adam_step_buckets, one per bucket, last bucket first; "
                                           "graph_*: the same launches replayed from a captured HIP graph"}
    log(f"bucket by bucket ({nb} launches): {t_b * 1e6:.1f} us, {gbps:.0f} GB/s algorithmic; "
        f"from a HIP graph {t_g * 1e6:.1f} us")
    del graph, st_b, par_b, reps_b

    # global-norm clipping: the rank's squared norm (writing the reduced
    # gradient), the coefficient, the clipped step from the reduced gradient
    E = plan.owned_numel
    dev = reps[0].device
    ws = torch.empty(plan.norm_workspace_bytes, dtype=torch.uint8, device=dev)
    parts = torch.zeros(D, dtype=torch.float64, device=dev)
    coeff = torch.empty(1, dtype=torch.float32, device=dev)
    red = torch.empty(plan.shard_numel, dtype=torch.int16, device=dev)
    st = [torch.zeros(plan.shard_numel, dtype=torch.float32, device=dev) for _ in range(3)]
    par = torch.empty(plan.extent(coords), dtype=torch.int16, device=dev)
    hp = dict(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, step=1)
    r = plan.rank
    t_norm = timed(lambda: zdo.grad_norm_sq(plan, reps, coords, w.scale, ws, parts[r:r + 1], red, zdo.LOCAL,
                                            stream=stream))
    t_clip = timed(lambda: zdo.clip_coefficient(parts, 1.0, coeff, stream=stream))
    t_step = timed(lambda: zdo.sharded_adam_step_clipped(plan, [red], zdo.LOCAL, 1.0, *st, par, coords,
                                                         grad_coeff=coeff, stream=stream, **hp))
    t_all = t_norm + t_clip + t_step
    # the step on one pre-reduced gradient, as after a collective
    # reduce-scatter across devices: 2 + 26 bytes per owned element
    t_pre = timed(lambda: zdo.sharded_adam_step(plan, [red], zdo.LOCAL, 1.0, *st, par, coords, stream=stream, **hp))
    out["pre_reduced_step"] = {
        "path": "sharded_adam_step on one reduced gradient (n_grads = 1, scale 1)", "bytes_per_element": 28,
        "elements": E, "kernel_avg_us": t_pre * 1e6, "achieved_gbps": E * 28 / t_pre / 1e9,
        "frac": E * 28 / t_pre / 1e9 / PEAK_HBM_GBPS, "elements_per_s": E / t_pre}
    log(f"pre-reduced step (n_grads = 1): {t_pre * 1e6:.1f} us, {E * 28 / t_pre / 1e9:.0f} GB/s algorithmic")
    # the write-back alone (bf16(master) into the owned elements): 4 + 2
    # bytes per owned element
    t_wb = timed(lambda: zdo.writeback_params(plan, st[0], par, coords, stream=stream))
    out["writeback_params"] = {"bytes_per_element": 6, "elements": E, "kernel_avg_us": t_wb * 1e6,
                               "achieved_gbps": E * 6 / t_wb / 1e9, "frac": E * 6 / t_wb / 1e9 / PEAK_HBM_GBPS}
    log(f"writeback_params: {t_wb * 1e6:.1f} us, {E * 6 / t_wb / 1e9:.0f} GB/s algorithmic")
    out["clipped_step"] = {
        "path": "grad_norm_sq (writes the reduced gradient) + clip_coefficient + sharded_adam_step_clipped "
                "(n_grads = 1)",
        "bytes_per_element": 2 * D + 30, "elements": E,
        "norm_us": t_norm * 1e6, "clip_us": t_clip * 1e6, "step_us": t_step * 1e6, "total_us": t_all * 1e6,
        "norm_gbps": E * (2 * D + 2) / t_norm / 1e9, "step_gbps": E * 28 / t_step / 1e9,
        "achieved_gbps": E * (2 * D + 30) / t_all / 1e9, "frac": E * (2 * D + 30) / t_all / 1e9 / PEAK_HBM_GBPS,
        "elements_per_s": E / t_all}
    log(f"clipped step: norm {t_norm * 1e6:.1f} us + clip {t_clip * 1e6:.1f} us + step {t_step * 1e6:.1f} us, "
        f"{out['clipped_step']['achieved_gbps']:.0f} GB/s algorithmic")
    del ws, red, st, par

    # two instances of D ranks: the bench's replicas and D more in the same
    # coordinates. Composed: a reduce-scatter within each instance, then the
    # step on the two results with scale 1 (which sums them as the all-reduce
    # across instances does). One pass: sharded_adam_step_instances.
    n_inst = 2
    Ln = plan.shard_numel
    n_rep = plan.extent(coords)
    stride = (n_rep + 63) // 64 * 64
    need = 2 * D * stride + 2 * n_inst * Ln + 12 * Ln + 2 * n_rep + (1 << 30)
    if torch.cuda.mem_get_info(dev)[0] < need:
        out["two_level_instances"] = {"skipped": "not enough free device memory for a second instance"}
        log("two-level instances: skipped (device memory)")
    else:
        extra = torch.empty(D * stride, dtype=torch.bfloat16, device=dev)
        inst1 = []
        for j in range(D):
            s = extra[j * stride: j * stride + n_rep]
            W.normal_bf16(n_rep, w.grad_sigma, W.seed(w.cfg, 1, "grad", j), out=s)
            inst1.append(s.view(torch.int16))
        rs = [torch.empty(Ln, dtype=torch.int16, device=dev) for _ in range(n_inst)]
        st = [torch.zeros(Ln, dtype=torch.float32, device=dev) for _ in range(3)]
        par = torch.empty(n_rep, dtype=torch.int16, device=dev)
        s_i = w.scale / n_inst
        t_rs0 = timed(lambda: zdo.reduce_scatter_local(plan, reps, coords, s_i, rs[0], zdo.LOCAL, stream))
        t_rs1 = timed(lambda: zdo.reduce_scatter_local(plan, inst1, coords, s_i, rs[1], zdo.LOCAL, stream))
        t_st = timed(lambda: zdo.sharded_adam_step(plan, rs, zdo.LOCAL, 1.0, *st, par, coords, stream=stream, **hp))
        t_one = timed(lambda: zdo.sharded_adam_step_instances(plan, [reps, inst1], coords, s_i, *st, par, coords,
                                                              stream=stream, **hp))
        t_all = t_rs0 + t_rs1 + t_st
        bytes_all = n_inst * ranges * (2 * D + 2) + E * (2 * n_inst + 26)
        bytes_one = E * (2 * n_inst * D + 26)
        out["two_level_instances"] = {
            "instances": n_inst,
            "composed": {"path": f"reduce_scatter_local within each of {n_inst} instances of D ranks, then "
                                 f"sharded_adam_step on the {n_inst} results (scale 1)",
                         "rs_us": [t_rs0 * 1e6, t_rs1 * 1e6], "step_us": t_st * 1e6, "total_us": t_all * 1e6,
                         "algorithmic_bytes": bytes_all, "achieved_gbps": bytes_all / t_all / 1e9,
                         "frac": bytes_all / t_all / 1e9 / PEAK_HBM_GBPS},
            "one_pass": {"path": "sharded_adam_step_instances", "bytes_per_element": 2 * n_inst * D + 26,
                         "kernel_avg_us": t_one * 1e6, "achieved_gbps": bytes_one / t_one / 1e9,
                         "frac": bytes_one / t_one / 1e9 / PEAK_HBM_GBPS, "elements_per_s": E / t_one}}
        log(f"two-level, {n_inst} instances: composed rs {t_rs0 * 1e6:.1f} + {t_rs1 * 1e6:.1f} us + step "
            f"{t_st * 1e6:.1f} us ({bytes_all / t_all / 1e9:.0f} GB/s); one pass {t_one * 1e6:.1f} us "
            f"({bytes_one / t_one / 1e9:.0f} GB/s)")
        del extra, inst1, rs, st, par

    # parameter all-gather, in place into this rank's buffer: the other ranks'
    # ranges of every padded bucket copied from their buffers. Sources: the
    # bench's whole-buffer replicas, else D uninitialised buffers of N if they
    # fit (the copy's timing does not depend on the values)
    N = plan.buffer_numel
    ranges = int(sum(b["shard_numel"] for b in plan.buckets()))
    srcs = None
    if coords == zdo.WORLD:
        srcs = list(reps)
    elif torch.cuda.mem_get_info(dev)[0] >= D * N * 2 + (1 << 30):
        srcs = [torch.zeros(N, dtype=torch.int16, device=dev) for _ in range(D)]
    if srcs is None:
        out["all_gather_params"] = {"skipped": "D whole parameter buffers do not fit beside the inputs"}
        log("all_gather_params: skipped (device memory)")
    else:
        mine = srcs[plan.rank].clone()
        srcs[plan.rank] = mine
        t = timed(lambda: zdo.all_gather_params(plan, srcs, mine, stream))
        nbytes = (N - ranges) * 4
        out["all_gather_params"] = {"path": "in place into the rank's buffer", "elements_copied": N - ranges,
                                    "bytes_per_element": 4, "kernel_avg_us": t * 1e6,
                                    "achieved_gbps": nbytes / t / 1e9, "frac": nbytes / t / 1e9 / PEAK_HBM_GBPS}
        log(f"all_gather_params: {t * 1e6:.1f} us, {nbytes / t / 1e9:.0f} GB/s algorithmic")
        del mine
    del srcs

    if coords == zdo.WORLD:
        N = plan.buffer_numel
        full = torch.empty(N, dtype=torch.int16, device=reps[0].device)
        t = timed(lambda: zdo.force_all_reduce(plan, reps, w.scale, full, stream))
        gbps = N * (2 * D + 2) / t / 1e9
        out["force_all_reduce"] = {"elements": N, "bytes_per_element": 2 * D + 2, "kernel_avg_us": t * 1e6,
                                   "achieved_gbps": gbps, "frac": gbps / PEAK_HBM_GBPS}
        log(f"force_all_reduce: {t * 1e6:.1f} us, {gbps:.0f} GB/s algorithmic")
        del full
    return out


def cpu_baseline(plan, w, reps, coords, master, exp_avg, exp_avg_sq, seconds: float) -> dict:
    """The oracle (oracle/step.c through oracle.step.rank_step) on the host
    cores, over the same rank's whole shard, repeated for about `seconds`;
    only the step compute is timed."""
    import numpy as np

    import oracle.layout as OL
    import oracle.numerics as ON
    import oracle.step as OS

    t0 = time.perf_counter()
    lay = OL.build_layout(w.param_numel, w.bucket_numel, w.dp_size)
    r = plan.rank
    reps_h = [x.cpu().numpy().view(np.uint16) for x in reps]
    st = [x.cpu().numpy().copy() for x in (master, exp_avg, exp_avg_sq)]
    par = np.zeros(reps_h[0].size, np.uint16)
    log(f"cpu baseline: host copies in {time.perf_counter() - t0:.1f}s, {ON.threads()} threads")
    passes, spent, t = 0, 0.0, 0
    while spent < seconds or passes < 1:
        t += 1
        hp = ON.hp_array(w.hp, t)
        a = time.perf_counter()
        OS.rank_step(lay, r, reps_h, coords, w.scale, *st, hp, par, coords)
        spent += time.perf_counter() - a
        passes += 1
    E = plan.owned_numel
    log(f"cpu baseline: {passes} passes in {spent:.1f}s")
    return {"value": E * passes / spent, "unit": "elements/s", "cores": ON.threads(), "kind": "oracle",
            "sample": f"rank {r}'s whole shard of {w.name} ({E} elements, D={w.dp_size}), {passes} passes, "
                      f"{spent:.1f} s of step compute (host copies excluded)",
            "gbps": E * (2 * w.dp_size + 26) * passes / spent / 1e9}


if __name__ == "__main__":
    sys.exit(main())
