"""Every kernel's tile loop beyond the first grid, against the oracle.

The launches cap their grid (2^24 workgroups in the library) and walk the
remaining tiles with a stride of the grid size. Real shards reach that only
beyond 2^24 tiles (8.6 G elements); this module runs the same parity checks
through a build of the library whose grid cap is 64 workgroups
(libzdo_gridloop.so, -DZDO_MAX_GRID=64), so that every launch here takes the
continuation many times over: the fused step (WORLD and LOCAL, several
contributions, bucket ranges, the instances form), the reduce-scatter, the
all-reduce's flat walk, the squared norm, the write-back and the all-gather.
Bars as in test_gpu_parity and test_gpu_clip.
"""

import random

import numpy as np
import pytest
import torch

import oracle.layout as OL
import oracle.numerics as ON
import oracle.step as OS
import workloads as W
import zero_distributed_optimizer_amd as Z
from zero_distributed_optimizer_amd import build as ZB
from test_gpu_clip import _norm_case
from test_gpu_parity import (DEV, SENTINEL, assert_bf16, assert_f32, bf16_host, free, host_f32, host_u16,
                             hp_kwargs, run_rank_step, to_dev)

pytestmark = pytest.mark.gpu

GRID = 64
TILE = 512


@pytest.fixture(scope="module")
def loop_gpu(gpu):
    """The binding, with every call going to the 64-workgroup build."""
    with Z.use_library(ZB.GRID_LOOP_LIB):
        yield gpu
        free()


def _layout(seed, D):
    """A mix of tiny, small and large parameters, about 100,000 elements per
    rank (200 tiles: the 64-workgroup grid walks each launch 3 times over),
    in 2 to 8 buckets."""
    pr = random.Random(7000 + seed)
    sizes = []
    while sum(sizes) < D * 100_000:
        sizes.append(pr.choice([pr.randint(1, 9), pr.randint(1, 5000), pr.randint(20000, 300000)]))
    bucket = pr.randint(max(2, sum(sizes) // 8), max(3, sum(sizes) // 2))
    return pr, sizes, bucket, D


@pytest.mark.parametrize("seed,D", [(0, 2), (1, 4), (2, 8), (3, 16), (4, 32), (5, 33)])
def test_fused_step_beyond_the_grid(loop_gpu, seed, D):
    pr, sizes, bucket, D = _layout(seed, D)
    rng = np.random.default_rng(7000 + seed)
    lay = OL.build_layout(sizes, bucket, D)
    reps_h = [bf16_host(rng, lay.buffer_numel, pr.choice([1e-3, 1.0])) for _ in range(D)]
    hp = W.get("tiny").hp
    for r in sorted({0, D - 1, pr.randrange(D)}):
        Ln = OL.shard_numel(lay, r)
        assert OL.owned_numel(lay, r) > 2 * GRID * TILE
        state = [(rng.standard_normal(Ln) * 0.02).astype(np.float32),
                 (rng.standard_normal(Ln) * 1e-3).astype(np.float32),
                 ((rng.standard_normal(Ln) * 1e-3) ** 2).astype(np.float32)]
        run_rank_step(loop_gpu, sizes, bucket, D, r, reps_h, state, 1.0 / D, hp, pr.choice([1, 7]),
                      pr.choice([loop_gpu.WORLD, loop_gpu.LOCAL]), pr.choice([loop_gpu.WORLD, loop_gpu.LOCAL]))
    free()


@pytest.mark.parametrize("seed,D", [(100, 3), (101, 16), (102, 33)])
def test_reduce_scatter_all_reduce_norm_writeback_beyond_the_grid(loop_gpu, seed, D):
    pr, sizes, bucket, D = _layout(seed, D)
    rng = np.random.default_rng(7100 + seed)
    lay = OL.build_layout(sizes, bucket, D)
    N = lay.buffer_numel
    assert N > 8 * GRID * TILE
    reps_h = [bf16_host(rng, N) for _ in range(D)]
    reps_d = [to_dev(x) for x in reps_h]
    scale = 1.0 / D
    out = torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV)
    plan = loop_gpu.build_range_map(sizes, bucket, D, 0)
    loop_gpu.force_all_reduce(plan, reps_d, scale, out)
    assert_bf16(host_u16(out), OS.all_reduce(reps_h, scale), "force_all_reduce")
    for r in sorted({0, D - 1, pr.randrange(D)}):
        plan = loop_gpu.build_range_map(sizes, bucket, D, r)
        Ln = plan.shard_numel
        for out_c in (loop_gpu.WORLD, loop_gpu.LOCAL):
            n_out = plan.extent(out_c)
            o = torch.full((max(n_out, 8),), SENTINEL, dtype=torch.int16, device=DEV)
            loop_gpu.reduce_scatter_local(plan, reps_d, loop_gpu.WORLD, scale, o, out_c)
            want = np.full(max(n_out, 8), SENTINEL, np.uint16)
            OS.reduce_scatter(lay, r, reps_h, OS.WORLD, scale, want, out_c)
            assert_bf16(host_u16(o), want, f"reduce-scatter r={r} out={out_c}")
        _norm_case(loop_gpu, sizes, bucket, D, r, reps_h, scale, pr.choice([loop_gpu.WORLD, loop_gpu.LOCAL]),
                   pr.choice([loop_gpu.WORLD, loop_gpu.LOCAL]))
        master = (rng.standard_normal(Ln) * 0.02).astype(np.float32)
        for c in (loop_gpu.WORLD, loop_gpu.LOCAL):
            n_par = plan.extent(c)
            par = torch.full((max(n_par, 8),), SENTINEL, dtype=torch.int16, device=DEV)
            loop_gpu.writeback_params(plan, to_dev(master), par, c)
            want = np.full(max(n_par, 8), SENTINEL, np.uint16)
            OS.writeback(lay, r, master, want, c)
            assert_bf16(host_u16(par), want, f"writeback r={r} coords={c}")
    free()


def test_bucket_ranges_and_instances_beyond_the_grid(loop_gpu):
    """Per-bucket launches start past tile 0 and loop; the instances form
    loops over the same tiles with two levels of reduction."""
    rng = np.random.default_rng(7200)
    sizes, bucket, D, r = [300000, 1, 90000, 17, 250000, 2, 70000, 3000, 110000], 80000, 4, 1
    lay = OL.build_layout(sizes, bucket, D)
    nb = len(lay.buckets)
    assert nb >= 4
    N = lay.buffer_numel
    reps_h = [bf16_host(rng, N) for _ in range(2 * D)]
    reps_d = [to_dev(x) for x in reps_h]
    plan = loop_gpu.build_range_map(sizes, bucket, D, r)
    Ln = plan.shard_numel
    st0 = [(rng.standard_normal(Ln) * 0.02).astype(np.float32), (rng.standard_normal(Ln) * 1e-3).astype(np.float32),
           ((rng.standard_normal(Ln) * 1e-3) ** 2).astype(np.float32)]
    hp = W.get("tiny").hp
    scale = 1.0 / (2 * D)
    # bucket by bucket, last bucket first
    st = [to_dev(x) for x in st0]
    par = torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV)
    for b in reversed(range(nb)):
        loop_gpu.sharded_adam_step(plan, reps_d[:D], loop_gpu.WORLD, scale, *st, par, loop_gpu.WORLD,
                                   buckets=(b, b + 1), **hp_kwargs(hp, 3))
    want = [x.copy() for x in st0]
    want_par = np.full(N, SENTINEL, np.uint16)
    OS.rank_step(lay, r, reps_h[:D], OS.WORLD, scale, *want, ON.hp_array(hp, 3), want_par, OS.WORLD)
    for g, wv, nm in zip(st, want, ("master", "exp_avg", "exp_avg_sq")):
        assert_f32(host_f32(g), wv, f"per bucket {nm}")
    assert_bf16(host_u16(par), want_par, "per bucket params")
    # bucket lists: separate runs of tiles in one launch, each walked
    # through the grid-stride continuation
    st = [to_dev(x) for x in st0]
    par = torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV)
    red = torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV)
    for g in ([(3, 4), (0, 1)], [(1, 3)]):
        loop_gpu.sharded_adam_step(plan, reps_d[:D], loop_gpu.WORLD, scale, *st, par, loop_gpu.WORLD, buckets=g,
                                   **hp_kwargs(hp, 3))
        loop_gpu.reduce_scatter_local(plan, reps_d[:D], loop_gpu.WORLD, scale, red, loop_gpu.WORLD, buckets=g)
    for g, wv, nm in zip(st, want, ("master", "exp_avg", "exp_avg_sq")):
        assert_f32(host_f32(g), wv, f"bucket lists {nm}")
    assert_bf16(host_u16(par), want_par, "bucket lists params")
    want_rs = np.full(N, SENTINEL, np.uint16)
    OS.reduce_scatter(lay, r, reps_h[:D], OS.WORLD, scale, want_rs, OS.WORLD)
    assert_bf16(host_u16(red), want_rs, "bucket lists reduce-scatter")
    # two instances in one pass = reduce-scatter per instance, then the step
    # on the instance results
    st = [to_dev(x) for x in st0]
    par = torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV)
    loop_gpu.sharded_adam_step_instances(plan, [reps_d[:D], reps_d[D:]], loop_gpu.WORLD, scale, *st, par,
                                         loop_gpu.WORLD, **hp_kwargs(hp, 3))
    inst = []
    for i in range(2):
        o = np.zeros(Ln, np.uint16)
        OS.reduce_scatter(lay, r, reps_h[i * D:(i + 1) * D], OS.WORLD, scale, o, OS.LOCAL)
        inst.append(o)
    want = [x.copy() for x in st0]
    want_par = np.full(N, SENTINEL, np.uint16)
    OS.rank_step(lay, r, inst, OS.LOCAL, 1.0, *want, ON.hp_array(hp, 3), want_par, OS.WORLD)
    for g, wv, nm in zip(st, want, ("master", "exp_avg", "exp_avg_sq")):
        assert_f32(host_f32(g), wv, f"instances {nm}")
    assert_bf16(host_u16(par), want_par, "instances params")
    free()


def test_all_gather_and_copy_beyond_the_grid(loop_gpu):
    rng = np.random.default_rng(7300)
    sizes, bucket, D = [500000, 3, 260000, 77777, 1, 400000], 300000, 5
    lay = OL.build_layout(sizes, bucket, D)
    N = lay.buffer_numel
    params_h = [bf16_host(rng, N, 1.0) for _ in range(D)]
    params_d = [to_dev(x) for x in params_h]
    plan = loop_gpu.build_range_map(sizes, bucket, D, 2)
    out = torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV)
    loop_gpu.all_gather_params(plan, params_d, out)
    want = np.full(N, SENTINEL, np.uint16)
    OS.all_gather(lay, params_h, want)
    assert_bf16(host_u16(out), want, "all-gather out of place")
    bufs = [to_dev(x) for x in params_h]
    loop_gpu.all_gather_params(plan, bufs, bufs[2])
    w = params_h[2].copy()
    OS.all_gather(lay, params_h, w)
    assert_bf16(host_u16(bufs[2]), w, "all-gather in place")
    src = torch.from_numpy(rng.integers(-2**31, 2**31, size=1 << 20, dtype=np.int64).astype(np.int32)).to(DEV)
    dst = torch.zeros_like(src)
    loop_gpu.device_copy(dst, src)
    assert torch.equal(dst, src)
    free()
