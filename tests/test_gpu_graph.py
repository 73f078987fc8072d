"""The launch calls inside a HIP graph: the clipping pipeline (squared norms of
every rank, the coefficient, every rank's clipped step), the plain fused
step, the ZeRO-1 loop (every rank's step, then every rank's all-gather) and
the one-pass two-instance step are captured once and replayed several times,
with eager work between replays; every replay must equal the same calls run
eagerly. The calls
allocate nothing and never synchronise the host, and no memset is recorded
(the norm's workspace needs no clearing)."""

import numpy as np
import pytest
import torch

import oracle.layout as OL
import workloads as W
from test_gpu_parity import DEV, SENTINEL, _gen_state, _gen_world, free, hp_kwargs

pytestmark = pytest.mark.gpu


def _pipeline(gpu, w, plans, reps, states, parts, coeff, wss, reds, params, hpk, max_norm, fused, fused_params):
    D = w.dp_size
    gpu.sharded_adam_step(plans[1], reps, gpu.WORLD, w.scale, *fused, fused_params, gpu.WORLD, **hpk)
    for r in range(D):
        gpu.grad_norm_sq(plans[r], reps, gpu.WORLD, w.scale, wss[r], parts[r:r + 1], reds[r], gpu.LOCAL)
    gpu.clip_coefficient(parts, max_norm, coeff)
    for r in range(D):
        gpu.sharded_adam_step_clipped(plans[r], [reds[r]], gpu.LOCAL, 1.0, *states[r], params, gpu.WORLD,
                                      grad_coeff=coeff, **hpk)


@pytest.mark.parametrize("max_norm", [0.01, 1e6])
def test_graph_replays_equal_eager(gpu, max_norm):
    w = W.get("tiny")
    D = w.dp_size
    lay = OL.build_layout(w.param_numel, w.bucket_numel, D)
    N = lay.buffer_numel
    plans = [gpu.build_range_map(w.param_numel, w.bucket_numel, D, r) for r in range(D)]
    reps = _gen_world(w, N)
    hpk = hp_kwargs(w.hp, 3)

    def fresh():
        return dict(states=[_gen_state(w, p.shard_numel) for p in plans],
                    parts=torch.zeros(D, dtype=torch.float64, device=DEV),
                    coeff=torch.zeros(1, dtype=torch.float32, device=DEV),
                    wss=[torch.empty(p.norm_workspace_bytes, dtype=torch.uint8, device=DEV) for p in plans],
                    reds=[torch.empty(p.shard_numel, dtype=torch.int16, device=DEV) for p in plans],
                    params=torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV),
                    fused=_gen_state(w, plans[1].shard_numel),
                    fused_params=torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV))

    eager, graphed = fresh(), fresh()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            _pipeline(gpu, w, plans, reps, graphed["states"], graphed["parts"], graphed["coeff"], graphed["wss"],
                      graphed["reds"], graphed["params"], hpk, max_norm, graphed["fused"], graphed["fused_params"])
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for replay in range(4):
        g.replay()
        _pipeline(gpu, w, plans, reps, eager["states"], eager["parts"], eager["coeff"], eager["wss"], eager["reds"],
                  eager["params"], hpk, max_norm, eager["fused"], eager["fused_params"])
        torch.cuda.synchronize()
        # eager work between replays on the same buffers' neighbours
        scratch = torch.randn(1 << 20, device=DEV)
        scratch.mul_(2.0)
        for a, b in zip(graphed["states"], eager["states"]):
            for x, y in zip(a, b):
                assert torch.equal(x.view(torch.int32), y.view(torch.int32)), f"replay {replay}"
        assert torch.equal(graphed["params"], eager["params"]), f"replay {replay}"
        for x, y in zip(graphed["fused"], eager["fused"]):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32)), f"replay {replay} fused"
        assert torch.equal(graphed["fused_params"], eager["fused_params"]), f"replay {replay} fused"
        assert torch.equal(graphed["parts"], eager["parts"]) and torch.equal(graphed["coeff"], eager["coeff"])
    del g
    free()


def _loop(gpu, w, plans, reps, reps2, states, bufs, inst_state, inst_params, hpk):
    """Every rank's step into its own parameter buffer, then every rank's
    all-gather in place; and one two-instance step in one pass."""
    D = w.dp_size
    for r in range(D):
        gpu.sharded_adam_step(plans[r], reps, gpu.WORLD, w.scale, *states[r], bufs[r], gpu.WORLD, **hpk)
    for r in range(D):
        gpu.all_gather_params(plans[r], bufs, bufs[r])
    gpu.sharded_adam_step_instances(plans[2], [reps, reps2], gpu.WORLD, w.scale / 2, *inst_state, inst_params,
                                    gpu.WORLD, **hpk)


def test_graph_zero1_loop_and_instances(gpu):
    w = W.get("tiny")
    D = w.dp_size
    N = OL.build_layout(w.param_numel, w.bucket_numel, D).buffer_numel
    plans = [gpu.build_range_map(w.param_numel, w.bucket_numel, D, r) for r in range(D)]
    reps = _gen_world(w, N)
    reps2 = _gen_world(w, N, step=1)
    hpk = hp_kwargs(w.hp, 2)
    base = torch.randn(N, device=DEV).mul_(0.02).to(torch.bfloat16).view(torch.int16)

    def fresh():
        return dict(states=[_gen_state(w, p.shard_numel) for p in plans],
                    bufs=[base.clone() for _ in range(D)],
                    inst_state=_gen_state(w, plans[2].shard_numel),
                    inst_params=torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV))

    eager, graphed = fresh(), fresh()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            _loop(gpu, w, plans, reps, reps2, graphed["states"], graphed["bufs"], graphed["inst_state"],
                  graphed["inst_params"], hpk)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for replay in range(4):
        g.replay()
        _loop(gpu, w, plans, reps, reps2, eager["states"], eager["bufs"], eager["inst_state"], eager["inst_params"],
              hpk)
        torch.cuda.synchronize()
        scratch = torch.randn(1 << 20, device=DEV)
        scratch.mul_(2.0)
        for a, b in zip(graphed["states"], eager["states"]):
            for x, y in zip(a, b):
                assert torch.equal(x.view(torch.int32), y.view(torch.int32)), f"replay {replay}"
        for r in range(D):
            assert torch.equal(graphed["bufs"][r], eager["bufs"][r]), f"replay {replay} rank {r}"
            assert torch.equal(eager["bufs"][r], eager["bufs"][0]), "every rank holds the same parameters"
        for x, y in zip(graphed["inst_state"], eager["inst_state"]):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32)), f"replay {replay} instances"
        assert torch.equal(graphed["inst_params"], eager["inst_params"]), f"replay {replay} instances"
    del g
    free()


def _groups(gpu, plan, reps, w, st, par, red, ns, groups, hpk):
    """Bucket-list launches (their run table read from the kernel
    arguments), and the squared norm on the library's static scratch."""
    for g in groups:
        gpu.sharded_adam_step(plan, reps, gpu.WORLD, w.scale, *st, par, gpu.WORLD, buckets=g, **hpk)
        gpu.reduce_scatter_local(plan, reps, gpu.WORLD, w.scale, red, gpu.WORLD, buckets=g)
    gpu.grad_norm_sq_no_alloc(plan, reps, gpu.WORLD, w.scale, ns)


def test_graph_bucket_lists_and_no_alloc_norm(gpu):
    """Launches over lists of scattered bucket ranges and the allocation-free
    squared norm, captured once and replayed four times with eager work in
    between: every replay equals the eager calls."""
    w = W.get("frag")
    D = w.dp_size
    N = OL.build_layout(w.param_numel, w.bucket_numel, D).buffer_numel
    plan = gpu.build_range_map(w.param_numel, w.bucket_numel, D, 3)
    nb = plan.buckets().size
    groups = [[(b, b + 1) for b in range(k, nb, 3)] for k in (2, 0, 1)]
    reps = _gen_world(w, N)
    hpk = hp_kwargs(w.hp, 4)

    def fresh():
        return dict(st=_gen_state(w, plan.shard_numel), par=torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV),
                    red=torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV),
                    ns=torch.zeros(1, dtype=torch.float64, device=DEV))

    eager, graphed = fresh(), fresh()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            _groups(gpu, plan, reps, w, graphed["st"], graphed["par"], graphed["red"], graphed["ns"], groups, hpk)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for replay in range(4):
        g.replay()
        _groups(gpu, plan, reps, w, eager["st"], eager["par"], eager["red"], eager["ns"], groups, hpk)
        torch.cuda.synchronize()
        scratch = torch.randn(1 << 20, device=DEV)
        scratch.mul_(2.0)
        for x, y in zip(graphed["st"], eager["st"]):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32)), f"replay {replay}"
        assert torch.equal(graphed["par"], eager["par"]), f"replay {replay} params"
        assert torch.equal(graphed["red"], eager["red"]), f"replay {replay} reduce-scatter"
        assert torch.equal(graphed["ns"], eager["ns"]), f"replay {replay} squared norm"
    del g
    free()
