"""Seeded random layouts through the fused step and the bucket lists,
against the oracle element by element.

Page "04 · 分布式优化器", §2-§5: whatever the parameter sizes, bucket size,
DP size and rank, the rank's step over its ranges (split parameters
included) equals the oracle's, and launching the buckets in any grouping and
order equals one launch. Each case draws D from 1 to 64 (the runtime-D path
included), 1-300 parameters of 1 to 70,000 elements, a bucket size from one
element up, a rank, WORLD or LOCAL coordinates for the contributions and
the parameters, and a step t <= 50. Then it compares:
  * the fused step, with its main-grad output, against the oracle;
  * random groups of buckets in random order, through
    sharded_adam_step_bucket_list and reduce_scatter_local_bucket_list,
    against the oracle's full step and reduce-scatter.
"""

import random

import numpy as np
import pytest
import torch

import oracle.layout as OL
import oracle.numerics as ON
import oracle.step as OS
import workloads as W
from test_gpu_parity import DEV, SENTINEL, assert_bf16, assert_f32, bf16_host, free, host_f32, host_u16, hp_kwargs, \
    run_rank_step, to_dev

pytestmark = pytest.mark.gpu

CASES_PER_SEED = 12


def _case(gpu, seed):
    pr = random.Random(seed)
    rng = np.random.default_rng(seed)
    D = pr.choice([1, 2, 3, 4, 5, 7, 8, 12, 16, 17, 24, 31, 32, 33, 48, 64])
    sizes = [pr.choice([1, pr.randint(1, 80), pr.randint(100, 3000), pr.randint(3000, 70000)])
             for _ in range(pr.randint(1, 300))]
    bucket = pr.randint(1, max(2, sum(sizes) // pr.choice([1, 2, 5, 20, 60])))
    r = pr.randrange(D)
    lay = OL.build_layout(sizes, bucket, D)
    N = lay.buffer_numel
    if N * D > 40_000_000:
        return False
    hp = W.get("tiny").hp
    reps_h = [bf16_host(rng, N, pr.choice([1e-3, 1.0])) for _ in range(D)]
    Ln = OL.shard_numel(lay, r)
    state = [(rng.standard_normal(Ln) * 0.02).astype(np.float32), (rng.standard_normal(Ln) * 1e-3).astype(np.float32),
             ((rng.standard_normal(Ln) * 1e-3) ** 2).astype(np.float32)]
    gc, pc = pr.choice([gpu.WORLD, gpu.LOCAL]), pr.choice([gpu.WORLD, gpu.LOCAL])
    t = pr.randint(1, 50)
    what = f"seed {seed}: D={D}, {len(sizes)} params, N={N}, {len(lay.buckets)} buckets, rank {r}"
    run_rank_step(gpu, sizes, bucket, D, r, reps_h, state, pr.choice([1.0 / D, 0.5, 1.0]), hp, t, gc, pc)
    nb = len(lay.buckets)
    if nb >= 2:
        plan = gpu.build_range_map(sizes, bucket, D, r)
        reps_d = [to_dev(x) for x in reps_h]
        order = list(range(nb))
        pr.shuffle(order)
        k = pr.randint(1, min(nb, 5))
        groups = [[(b, b + 1) for b in order[i::k]] for i in range(k)]
        st = [to_dev(x) for x in state]
        par = torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV)
        out = torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV)
        scale = 1.0 / D
        for g in groups:
            gpu.sharded_adam_step(plan, reps_d, gpu.WORLD, scale, *st, par, gpu.WORLD, buckets=g, **hp_kwargs(hp, t))
            gpu.reduce_scatter_local(plan, reps_d, gpu.WORLD, scale, out, gpu.WORLD, buckets=g)
        want = [x.copy() for x in state]
        want_par = np.full(N, SENTINEL, np.uint16)
        OS.rank_step(lay, r, reps_h, OS.WORLD, scale, *want, ON.hp_array(hp, t), want_par, OS.WORLD)
        want_rs = np.full(N, SENTINEL, np.uint16)
        OS.reduce_scatter(lay, r, reps_h, OS.WORLD, scale, want_rs, OS.WORLD)
        for x, wv, nm in zip(st, want, ("master", "exp_avg", "exp_avg_sq")):
            assert_f32(host_f32(x), wv, f"{what}, {k} bucket groups, {nm}")
        assert_bf16(host_u16(par), want_par, f"{what}, {k} bucket groups, params")
        assert_bf16(host_u16(out), want_rs, f"{what}, {k} bucket groups, reduce-scatter")
    free()
    return True


@pytest.mark.parametrize("block", range(6))
def test_random_layouts(gpu, block):
    ran = sum(_case(gpu, 20000 + block * CASES_PER_SEED + i) for i in range(CASES_PER_SEED))
    assert ran >= CASES_PER_SEED // 2
