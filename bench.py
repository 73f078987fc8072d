#!/usr/bin/env python3
"""Throughput of one DP rank's sharded Adam step on one MI355X.

A step is one sharded_adam_step call on the rank's shard: reduce the D
replica contributions (scaled, fixed rank order), Adam on the fp32
master/m/v shard, bf16 write-back into the owned range; one fused kernel.

Headline (default): the Llama-3-70B-shaped parameter list (723 tensors,
70,553,706,496 elements, buckets of 200,000,000, D = 32), rank 1's shard of
2,204,803,328 owned elements, its 32 bf16 contribution slices, fp32
master/m/v and bf16 parameter slice resident in HBM (172 GB).

Prints one JSON line:
  * value: elements/s of the timed steps (wall clock), ms_per_step;
  * roofline: the step kernel's algorithmic bytes, (2D + 26) per owned
    element, over its average duration: one HIP event pair on the launch
    stream around the K timed steps, divided by K; traffic: HBM bytes per
    launch from the committed counter summary of the same kernel source;
  * cold_cache: the step after 1 GiB of reads evicted the caches;
  * variants: the library's other calls on the same shard;
  * configs: every workload the step is measured on, rank by rank (Tiny
    ranks 1..3, GPT-2 rank 1, Llama-3-8B rank 1, fragmentation ranks 0..15
    and its force_all_reduce path). Where the fp32 state fits the 256 MB
    Infinity Cache, back-to-back steps find part of it there; their HBM
    figure is the cold-cache one, and the back-to-back one is labelled;
  * cpu_baseline: the oracle on the host cores, streamed over the shard in
    chunks of 2^26 slots (a bounded sample of them), and on one core.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--rank R]
                    [--configs all|none] [--cpu-seconds S] [--no-cpu]
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
STATE_CACHE_BYTES = 1 << 30      # below this, a back-to-back step finds state in the Infinity Cache
CPU_CHUNK = 1 << 26
KERNEL_SOURCES = [os.path.join(ROOT, "zero_distributed_optimizer_amd", "csrc", f)
                  for f in ("kernels.hip", "kernels.h", "zdo_internal.h")]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """sha256[:16] over the kernel source and the headers that shape it, with
    comments and blank lines dropped: a change of wording leaves the code,
    and so the counters taken on it, as they were."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES:
        with open(path, encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        lines = [ln.rstrip() for ln in text.splitlines() if ln.strip()]
        h.update("\n".join(lines).encode())
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


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---- inputs --------------------------------------------------------------------------------------

class Shard:
    """A rank's inputs resident in HBM: the D contributions (whole buffers
    or shard slices, each on a 128-byte line), master/exp_avg/exp_avg_sq
    and a parameter buffer."""

    def __init__(self, zdo, torch, W, w, rank: int, dev, stagger: int = 0, reps=None):
        self.w, self.rank = w, rank
        self.plan = zdo.build_range_map(w.param_numel, w.bucket_numel, w.dp_size, rank)
        p = self.plan
        self.coords = zdo.WORLD if w.grad_mode == "world" else zdo.LOCAL
        self.n_rep = p.buffer_numel if self.coords == zdo.WORLD else p.shard_numel
        D, Ln = w.dp_size, p.shard_numel
        if reps is None:
            stride = (self.n_rep + 63) // 64 * 64
            gap2 = stagger // 2
            self.rep_buf = torch.empty(D * (stride + gap2), dtype=torch.bfloat16, device=dev)
            reps = []
            for j in range(D):
                s = self.rep_buf[j * (stride + gap2): j * (stride + gap2) + self.n_rep]
                W.normal_bf16(self.n_rep, w.grad_sigma, W.seed(w.cfg, 0, "grad", j), out=s,
                              probe_fraction=w.probe_fraction, probe_seed=W.seed(w.cfg, 0, "probe", j))
                reps.append(s.view(torch.int16))
        self.reps = reps
        sstride = (Ln + 31) // 32 * 32 + stagger // 4
        self.state_buf = torch.empty(3 * sstride, dtype=torch.float32, device=dev)
        self.state = [self.state_buf[i * sstride: i * sstride + Ln] for i in range(3)]
        W.normal_f32(Ln, w.master_sigma, W.seed(w.cfg, 0, "master", rank), out=self.state[0])
        W.normal_f32(Ln, w.m_sigma, W.seed(w.cfg, 0, "m", rank), out=self.state[1])
        W.square_normal_f32(Ln, w.v_sigma, W.seed(w.cfg, 0, "v", rank), out=self.state[2])
        self.params = torch.zeros(self.n_rep, dtype=torch.int16, device=dev)
        self.t = 0
        self.E = p.owned_numel
        self.D = D
        self.bytes_per_elem = 2 * D + 26
        self.alg_bytes = self.E * self.bytes_per_elem
        self.state_bytes = 12 * Ln

    def step(self, zdo, stream) -> None:
        self.t += 1
        w = self.w
        zdo.sharded_adam_step(self.plan, self.reps, self.coords, w.scale, *self.state, self.params, self.coords,
                              step=self.t, stream=stream, **w.hp)


def back_to_back(torch, fn, stream, n: int, warmup: int = 3) -> tuple:
    """(seconds per call from one HIP event pair around n back-to-back calls
    on the launch stream, seconds per call by wall clock)."""
    for _ in range(warmup):
        fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    a.record(stream)
    for _ in range(n):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / 1e3 / n, (time.perf_counter() - w0) / n


COLD_SPREAD = {}


def cold(torch, np, fn, stream, flush_src, n: int) -> float:
    """Seconds per call (mean over n) of calls each after 1 GiB of ordinary
    (temporal) reads, which evict the 256 MB Infinity Cache and the L2s as a
    training step's forward and backward passes would; the event pair
    brackets the call only. The median, p10 and p90 of the n calls (us) are
    left in COLD_SPREAD."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        flush_src.sum()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    COLD_SPREAD.clear()
    COLD_SPREAD.update(median_us=float(np.median(ms)) * 1e3, p10_us=float(np.percentile(ms, 10)) * 1e3,
                       p90_us=float(np.percentile(ms, 90)) * 1e3, calls=n)
    return float(np.mean(ms)) / 1e3


def rate(alg_bytes: float, seconds: float, spread: dict | None = None) -> dict:
    gbps = alg_bytes / seconds / 1e9
    out = {"us": seconds * 1e6, "gbps": gbps, "frac": gbps / PEAK_HBM_GBPS}
    if spread:
        out["spread"] = dict(spread)
    return out


# ---- main ------------------------------------------------------------------------------------

def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama3_70b")
    ap.add_argument("--rank", type=int, default=None)
    ap.add_argument("--configs", choices=("all", "none"), default="all",
                    help="also time every other workload, rank by rank")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--stagger", type=int, default=0,
                    help="extra bytes (a multiple of 16) placed between consecutive input buffers")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU only: the D ranks' contributions are D "
                          "replica buffers in one GPU's HBM; run with --gpus 1"}), flush=True)
        return 2
    if args.stagger % 16:
        raise SystemExit("--stagger must be a multiple of 16")

    import numpy as np
    import torch

    import workloads as W
    import zero_distributed_optimizer_amd as zdo

    zdo.require_library()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    w = W.get(args.workload)
    rank = w.time_ranks[0] if args.rank is None else args.rank

    t0 = time.perf_counter()
    sh = Shard(zdo, torch, W, w, rank, dev, args.stagger)
    plan, E, D = sh.plan, sh.E, sh.D
    torch.cuda.synchronize(dev)
    log(f"workload {w.name}: N={plan.buffer_numel} D={D} rank={rank} E={E} L={plan.shard_numel} "
        f"grads={w.grad_mode}; inputs generated in {time.perf_counter() - t0:.1f}s")

    # timed region: K back-to-back steps between one HIP event pair on the
    # launch stream (bracketed by synchronisations); the average launch
    # duration is the region over K. An event pair around every launch would
    # drain the queue before and after each step and slow the steps it
    # measures.
    for _ in range(args.warmup):
        sh.step(zdo, stream)
    kern_s, wall_s = back_to_back(torch, lambda: sh.step(zdo, stream), stream, args.steps, warmup=0)
    ms_per_step = wall_s * 1e3
    achieved = sh.alg_bytes / kern_s / 1e9
    log(f"step: wall {wall_s * 1e6:.1f} us/step, kernel avg {kern_s * 1e6:.1f} us, {achieved:.0f} GB/s "
        f"algorithmic ({achieved / PEAK_HBM_GBPS:.1%} of 8 TB/s)")

    # single launches between their own event pairs: the spread of one launch
    n_iso = min(args.steps, 20)
    iev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_iso)]
    for a, b in iev:
        a.record(stream)
        sh.step(zdo, stream)
        b.record(stream)
    torch.cuda.synchronize(dev)
    iso_ms = [a.elapsed_time(b) for a, b in iev]
    isolated = {"steps": n_iso, "avg_us": float(np.mean(iso_ms)) * 1e3,
                "p10_us": float(np.percentile(iso_ms, 10)) * 1e3, "p90_us": float(np.percentile(iso_ms, 90)) * 1e3,
                "how": "each launch between its own event pair, after the timed region"}

    # plain-copy reference on the same stream (1 GiB read + 1 GiB write)
    nb = 1 << 30
    flush_src = torch.empty(nb // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(flush_src)
    copy_s, _ = back_to_back(torch, lambda: zdo.device_copy(dst, flush_src, stream), stream, 10)
    copy_gbps = 2 * nb / copy_s / 1e9
    del dst
    log(f"copy reference: {copy_gbps:.0f} GB/s")

    cold_s = cold(torch, np, lambda: sh.step(zdo, stream), stream, flush_src, min(args.steps, 20))
    cold_r = rate(sh.alg_bytes, cold_s, COLD_SPREAD)
    log(f"cold caches: kernel avg {cold_s * 1e6:.1f} us, {cold_r['gbps']:.0f} GB/s algorithmic")

    variants = None
    if not args.no_variants:
        variants = measure_variants(zdo, torch, np, plan, w, sh.reps, sh.coords, stream, min(args.steps, 20))

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(torch, np, sh, args.cpu_seconds)

    # the ceiling of the step's stream shape: the same traffic with trivial
    # arithmetic on the same buffers (overwrites their values; last)
    probe = stream_probe(zdo, torch, sh, stream, min(args.steps, 10), achieved)

    del sh
    torch.cuda.synchronize(dev)
    torch.cuda.empty_cache()
    configs = {}
    if args.configs == "all":
        for name in ("tiny", "gpt2_small", "llama3_8b", "llama3_70b", "frag"):
            if name == w.name:
                continue
            configs[name] = measure_config(zdo, torch, np, W, W.get(name), dev, stream, flush_src,
                                           variants=not args.no_variants)
            torch.cuda.synchronize(dev)
            torch.cuda.empty_cache()

    traffic = traffic_from_profiles(w.name)
    in_cache = 12 * plan.shard_numel <= STATE_CACHE_BYTES
    out = {
        "metric": METRIC,
        "value": E / wall_s,
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
            "buffer_elements": plan.buffer_numel,
            "bucket_elements": w.bucket_numel,
            "buckets": int(plan.buckets().size),
            "dp_size": D,
            "rank": rank,
            "owned_elements": E,
            "grad_replicas": f"{D} x bf16 {'whole buffers' if sh_coords_world(w) else 'shard slices'}",
            "state": "fp32 master/exp_avg/exp_avg_sq shard",
            "bytes_per_element": 2 * D + 26,
            "buffer_stagger_bytes": args.stagger,
        },
        "hbm_gbps": E * (2 * D + 26) / wall_s / 1e9,
        "hbm_frac_of_peak": E * (2 * D + 26) / wall_s / 1e9 / PEAK_HBM_GBPS,
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBPS,
            "traffic": traffic,
        },
        "kernel": {"name": "step_kernel", "avg_us": kern_s * 1e6,
                   "how": "one HIP event pair around the timed steps on the launch stream, divided by the steps",
                   "single_launches": isolated,
                   "source_sha256_16": kernel_source_hash(),
                   "state_in_infinity_cache": in_cache},
        "cold_cache": {"kernel_avg_us": cold_s * 1e6, "achieved_gbps": cold_r["gbps"], "frac": cold_r["frac"],
                       "elements_per_s": E / cold_s, "spread": cold_r["spread"],
                       "flush": "torch sum over a 1 GiB buffer (temporal loads) before every step, outside the "
                                "kernel's events"},
        "copy_reference_gbps": copy_gbps,
        "frac_of_copy_reference": achieved / copy_gbps,
        "stream_probe": probe,
        "variants": variants,
        "configs": configs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


def sh_coords_world(w) -> bool:
    return w.grad_mode == "world"


def stream_probe(zdo, torch, sh, stream, n: int, step_gbps: float) -> dict | None:
    """zdo_stream_probe on the shard's own buffers: the step's reads and
    writes (2D + 26 bytes per slot, the same tile and lane layout) with
    trivial arithmetic, at several occupancy caps; the best is the ceiling
    of this stream shape on this part. At the best cap, the same loads with
    only the parameter stream stored (2D + 14 bytes per slot) and with no
    stores (2D + 12) take the shape apart: what the loads alone reach, and
    what the state's stores cost."""
    D = sh.D
    if D not in (8, 16, 32):
        return None
    m = min(sh.plan.shard_numel, sh.n_rep) // 512 * 512
    out = {"elements": m, "bytes_per_element": 2 * D + 26, "caps": {}}
    for cap in (4, 5, 6, 8, 10):
        t, _ = back_to_back(torch, lambda: zdo.stream_probe(sh.reps, sh.state, sh.params, m, cap, stream), stream, n)
        out["caps"][str(cap)] = rate(m * (2 * D + 26), t)
    best = max(out["caps"].items(), key=lambda kv: kv[1]["gbps"])
    out["best"] = {"waves_per_cu": int(best[0]), **best[1]}
    out["step_vs_best"] = step_gbps / best[1]["gbps"]
    cap = int(best[0])
    parts = {}
    for name, stores, bpe in (("param_stores_only", zdo.PROBE_STORE_OUT, 2 * D + 14),
                              ("loads_only", zdo.PROBE_STORE_NONE, 2 * D + 12)):
        t, _ = back_to_back(torch, lambda: zdo.stream_probe(sh.reps, sh.state, sh.params, m, cap, stream,
                                                            stores=stores), stream, n)
        parts[name] = {"bytes_per_element": bpe, **rate(m * bpe, t)}
    out["parts_at_best_cap"] = parts
    log(f"stream-shape probe: " + ", ".join(f"{k} waves/CU {v['gbps']:.0f} GB/s" for k, v in out["caps"].items()) +
        f"; the step runs at {out['step_vs_best']:.1%} of the best; at {cap} waves/CU the loads with the "
        f"parameter stores only reach {parts['param_stores_only']['frac']:.1%} of 8 TB/s, the loads alone "
        f"{parts['loads_only']['frac']:.1%}")
    return out


# ---- every workload, rank by rank -----------------------------------------------------------------

def measure_config(zdo, torch, np, W, w, dev, stream, flush_src, variants: bool = True) -> dict:
    """Every rank the workload times: the step back to back and with cold
    caches. HBM figure: cold caches where the rank's fp32 state fits in 1 GiB
    (back-to-back steps there read part of it from the Infinity Cache),
    back to back otherwise (the state streams from HBM either way). On the
    Llama-3-8B shape also the library's other calls (measure_variants): two
    instances and the all-gather fit beside it, which they do not beside the
    Llama-3-70B shard."""
    t0 = time.perf_counter()
    ranks = []
    reps = None
    big = None
    for r in w.time_ranks:
        sh = Shard(zdo, torch, W, w, r, dev, reps=reps)
        if sh.coords == zdo.WORLD:
            reps = sh.reps          # whole buffers: shared by every rank
        small = sh.state_bytes <= STATE_CACHE_BYTES
        n = 200 if small else 20
        b2b, _ = back_to_back(torch, lambda: sh.step(zdo, stream), stream, n)
        entry = {"rank": r, "owned_elements": sh.E, "bytes_per_element": sh.bytes_per_elem,
                 "back_to_back": rate(sh.alg_bytes, b2b)}
        if small:
            c = cold(torch, np, lambda: sh.step(zdo, stream), stream, flush_src, 200)
            entry["cold_cache"] = rate(sh.alg_bytes, c, COLD_SPREAD)
            hbm = entry["cold_cache"]
            entry["hbm_figure"] = "cold_cache"
        else:
            hbm = entry["back_to_back"]
            entry["hbm_figure"] = "back_to_back (the state exceeds the Infinity Cache)"
        entry["elements_per_s"] = sh.E / (hbm["us"] * 1e-6)
        entry["frac"] = hbm["frac"]
        ranks.append(entry)
        big = sh
        del sh
    out = {"dp_size": w.dp_size, "grad_replicas": w.grad_mode, "ranks": ranks,
           "hbm_frac_min": min(e["frac"] for e in ranks), "hbm_frac_max": max(e["frac"] for e in ranks)}
    if w.name == "frag":
        out["bucket_groups"] = bucket_groups(zdo, torch, big, stream, 100)
        out["fixed_cost_fit"] = fixed_cost_fit(zdo, torch, np, W, w, dev, stream, flush_src)
        # the force_all_reduce path: the whole reduced buffer (2D + 2 bytes
        # per buffer element)
        Nn = big.plan.buffer_numel
        full = torch.empty(Nn, dtype=torch.int16, device=dev)
        fn = lambda: zdo.force_all_reduce(big.plan, reps, w.scale, full, stream)   # noqa: E731
        b2b, _ = back_to_back(torch, fn, stream, 50)
        c = cold(torch, np, fn, stream, flush_src, 20)
        out["force_all_reduce"] = {"elements": Nn, "bytes_per_element": 2 * w.dp_size + 2,
                                   "back_to_back": rate(Nn * (2 * w.dp_size + 2), b2b),
                                   "cold_cache": rate(Nn * (2 * w.dp_size + 2), c, COLD_SPREAD)}
        del full
    if w.name == "llama3_8b" and variants:
        out["variants"] = measure_variants(zdo, torch, np, big.plan, w, big.reps, big.coords, stream, 10)
    del big, reps
    log(f"config {w.name}: " + ", ".join(f"r{e['rank']} {e['frac']:.1%}" for e in ranks) +
        f" ({time.perf_counter() - t0:.1f}s)")
    return out


def fixed_cost_fit(zdo, torch, np, W, w, dev, stream, flush_src) -> dict:
    """Where a short step's time goes: rank 0's cold-cache step on the
    parameter list repeated 1, 2 and 4 times (same bucket size and D), fitted
    as time = fixed + bytes / rate. The fixed part is what one launch costs
    whatever its size (dispatch, the first loads' latency, the last wave);
    the rate is the step's streaming rate at this shape."""
    import dataclasses
    pts = []
    for k in (1, 2, 4):
        wk = dataclasses.replace(w, param_numel=tuple(w.param_numel) * k)
        sh = Shard(zdo, torch, W, wk, 0, dev)
        c = cold(torch, np, lambda: sh.step(zdo, stream), stream, flush_src, 40)
        pts.append((k, sh.alg_bytes, c))
        del sh
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    x = np.array([p[1] for p in pts], dtype=np.float64)
    y = np.array([p[2] for p in pts], dtype=np.float64)
    slope, icpt = np.polyfit(x, y, 1)
    out = {"repeats": [p[0] for p in pts], "bytes": [p[1] for p in pts], "cold_us": [p[2] * 1e6 for p in pts],
           "fixed_us": icpt * 1e6, "steady_gbps": 1 / slope / 1e9, "steady_frac": 1 / slope / 1e9 / PEAK_HBM_GBPS}
    log(f"frag fixed-cost fit: fixed {out['fixed_us']:.1f} us, steady {out['steady_gbps']:.0f} GB/s "
        f"({out['steady_frac']:.1%})")
    return out


def bucket_groups(zdo, torch, sh, stream, n: int) -> dict:
    """The step bucket by bucket, in bucket groups and in one launch, back to
    back (n rounds each): one launch per bucket; three groups of adjacent
    buckets (one launch each); three groups of scattered buckets (every third
    bucket, one bucket-list launch each); the whole step."""
    nb = int(sh.plan.buckets().size)
    reps = zdo.Buffers(sh.reps, "replicas")
    w = sh.w

    def calls(groups):
        def fn():
            sh.t += 1
            for g in groups:
                zdo.sharded_adam_step(sh.plan, reps, sh.coords, w.scale, *sh.state, sh.params, sh.coords,
                                      step=sh.t, stream=stream, buckets=g, **w.hp)
        return fn
    third = -(-nb // 3)
    forms = {
        "one_launch": [(0, nb)],
        "per_bucket": [(b, b + 1) for b in reversed(range(nb))],
        "three_adjacent_groups": [(k, min(nb, k + third)) for k in reversed(range(0, nb, third))],
        "three_scattered_groups": [[(b, b + 1) for b in range(k, nb, 3)] for k in range(3)],
    }
    out = {"buckets": nb}
    for name, groups in forms.items():
        t, _ = back_to_back(torch, calls(groups), stream, n)
        out[name] = {"launches": len(groups), "us": t * 1e6, "gbps": sh.alg_bytes / t / 1e9}
    base = out["one_launch"]["us"]
    for name in forms:
        out[name]["vs_one_launch"] = out[name]["us"] / base
    log("bucket groups: " + ", ".join(f"{k} {v['us']:.1f} us ({v['vs_one_launch']:.2f}x)"
                                      for k, v in out.items() if isinstance(v, dict)))
    return out


# ---- the other calls on the headline shard --------------------------------------------------------

def measure_variants(zdo, torch, np, plan, w, reps, coords, stream, n: int) -> dict:
    """The other device calls on the same inputs: reduce_scatter_local over
    the rank's whole ranges (2D + 2 bytes per element of the ranges), the step
    bucket by bucket, the clipped path, two instances (composed and in one
    pass), the parameter all-gather in place (4 bytes per element of the
    other ranks' ranges) and, when the replicas are whole buffers,
    force_all_reduce over the padded buffer (2D + 2 bytes per buffer
    element). Each call timed as n back-to-back calls between one HIP event
    pair."""
    import workloads as W

    D = plan.dp_size
    out = {}

    def timed(fn) -> float:
        return back_to_back(torch, fn, stream, n)[0]

    ranges = int(sum(b["shard_numel"] for b in plan.buckets()))
    red = torch.empty(plan.shard_numel, dtype=torch.int16, device=reps[0].device)
    t = timed(lambda: zdo.reduce_scatter_local(plan, reps, coords, w.scale, red, zdo.LOCAL, stream))
    gbps = ranges * (2 * D + 2) / t / 1e9
    out["reduce_scatter_local"] = {"elements": ranges, "bytes_per_element": 2 * D + 2, "kernel_avg_us": t * 1e6,
                                   "achieved_gbps": gbps, "frac": gbps / PEAK_HBM_GBPS}
    log(f"reduce_scatter_local: {t * 1e6:.1f} us, {gbps:.0f} GB/s algorithmic")
    del red
    # bucket by bucket: the same step launched once per bucket, last bucket
    # first (the order a backward pass makes them ready)
    nb = int(plan.buckets().size)
    st_b = [torch.zeros(plan.shard_numel, dtype=torch.float32, device=reps[0].device) for _ in range(3)]
    par_b = torch.empty(plan.extent(coords), dtype=torch.int16, device=reps[0].device)
    hp_b = dict(w.hp, step=1)
    reps_b = zdo.Buffers(reps, "replicas")   # checked once for the nb launches

    def per_bucket(st=stream):
        for b in reversed(range(nb)):
            zdo.sharded_adam_step(plan, reps_b, coords, w.scale, *st_b, par_b, coords, stream=st,
                                  buckets=(b, b + 1), **hp_b)
    t_b = timed(per_bucket)
    # the same launches replayed from a HIP graph
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
    hp = dict(w.hp, step=1)
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
    # step on the two results with scale 1. One pass: sharded_adam_step_instances.
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
        log(f"two-level, {n_inst} instances: composed {t_all * 1e6:.1f} us ({bytes_all / t_all / 1e9:.0f} GB/s); "
            f"one pass {t_one * 1e6:.1f} us ({bytes_one / t_one / 1e9:.0f} GB/s)")
        del extra, inst1, rs, st, par

    # parameter all-gather, in place into this rank's buffer
    N = plan.buffer_numel
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
        full = torch.empty(N, dtype=torch.int16, device=reps[0].device)
        t = timed(lambda: zdo.force_all_reduce(plan, reps, w.scale, full, stream))
        gbps = N * (2 * D + 2) / t / 1e9
        out["force_all_reduce"] = {"elements": N, "bytes_per_element": 2 * D + 2, "kernel_avg_us": t * 1e6,
                                   "achieved_gbps": gbps, "frac": gbps / PEAK_HBM_GBPS}
        log(f"force_all_reduce: {t * 1e6:.1f} us, {gbps:.0f} GB/s algorithmic")
        del full
    return out


# ---- the oracle on the host -------------------------------------------------------------------------

def cpu_baseline(torch, np, sh, seconds: float) -> dict:
    """The oracle's element arithmetic (oracle/step.c) on the host cores,
    streamed over the rank's owned elements in chunks of at most 2^26 slots
    as the oracle's range map gives them (one run per bucket): each chunk's D
    contribution slices and state are copied to pinned host memory, then one
    timed oracle step runs on them. Chunks spread evenly over the shard are
    taken until about `seconds` of oracle compute (a bounded sample unless
    the whole shard fits in that time); only the oracle's compute is timed.
    The same on one core over one chunk of at most 2^22 slots."""
    import oracle.layout as OL
    import oracle.numerics as ON

    w, r, D = sh.w, sh.rank, sh.D
    lay = OL.build_layout(w.param_numel, w.bucket_numel, D)
    runs = []
    for pc in OL.rank_pieces(lay, r):
        if runs and runs[-1][0] + runs[-1][2] == pc.shard_offset and \
                runs[-1][1] + runs[-1][2] == pc.gbuf_world.start:
            runs[-1][2] += pc.gbuf_world.size
        else:
            runs.append([pc.shard_offset, pc.gbuf_world.start, pc.gbuf_world.size])
    world = sh.coords == 0
    chunks = [(k + off, (wb if world else k) + off, min(CPU_CHUNK, n - off))
              for k, wb, n in runs for off in range(0, n, CPU_CHUNK)]
    cmax = max(c[2] for c in chunks)
    stage_g = torch.empty((D, cmax), dtype=torch.int16, pin_memory=True)
    stage_s = torch.empty((3, cmax), dtype=torch.float32, pin_memory=True)
    hp = ON.hp_array(w.hp, 1)
    cores = ON.threads()

    def load(k0, gi, n):
        for j in range(D):
            stage_g[j, :n].copy_(sh.reps[j][gi:gi + n], non_blocking=True)
        for i in range(3):
            stage_s[i, :n].copy_(sh.state[i][k0:k0 + n], non_blocking=True)
        torch.cuda.synchronize()
        return [stage_g[j, :n].numpy().view(np.uint16) for j in range(D)], [stage_s[i, :n].numpy() for i in range(3)]

    # chunks in an order that spreads any prefix of them over the shard
    order = sorted(range(len(chunks)), key=lambda i: (bin(i)[2:].zfill(32)[::-1], i))
    done = spent = 0.0
    taken = 0
    par = np.empty(cmax, np.uint16)
    t_all = time.perf_counter()
    for i in order:
        k0, gi, n = chunks[i]
        grads, st = load(k0, gi, n)
        a = time.perf_counter()
        ON.step(grads, w.scale, *st, hp, par[:n])
        spent += time.perf_counter() - a
        done += n
        taken += 1
        if spent >= seconds:
            break
    # one core, one chunk of at most 2^22 slots
    k0, gi, n = chunks[order[0]]
    n1 = min(n, 1 << 22)
    grads, st = load(k0, gi, n1)
    ON.set_threads(1)
    a = time.perf_counter()
    ON.step(grads, w.scale, *st, hp, par[:n1])
    one = time.perf_counter() - a
    ON.set_threads(cores)
    E = sh.E
    bpe = 2 * D + 26
    log(f"cpu baseline: {int(done)} of {E} elements in {spent:.1f}s of oracle compute on {cores} threads "
        f"({done / spent / 1e9:.3f} G elem/s); 1 core {n1 / one / 1e9:.4f} G elem/s; "
        f"{time.perf_counter() - t_all:.1f}s with the host copies")
    return {"value": done / spent, "unit": "elements/s", "cores": cores, "kind": "oracle",
            "sample": f"rank {r}'s shard of {w.name} (D={D}): {taken} of {len(chunks)} chunks of at most 2^26 "
                      f"slots, spread over the shard ({int(done)} of {E} owned elements, {done / E:.0%}), "
                      f"{spent:.1f} s of oracle compute (host copies excluded)",
            "gbps": done * bpe / spent / 1e9,
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
            "one_core": {"value": n1 / one, "unit": "elements/s", "elements": n1, "seconds": one}}


if __name__ == "__main__":
    sys.exit(main())
