"""grad_norm_sq_no_alloc: the squared norm with the library's static scratch
array instead of a caller's workspace (for callers that cannot allocate).

Two calls in a row, the second on a smaller input, each compared with
grad_norm_sq on the same inputs with a fresh workspace: the squared norm and
the reduced gradient must be equal bit for bit (the same kernels and the
same fixed summation order), and the norm within the fp64 summation bound
of the oracle's sequential sum.
"""

import numpy as np
import pytest
import torch

import oracle.layout as OL
import oracle.step as OS
import workloads as W
from test_gpu_clip import assert_norm
from test_gpu_parity import DEV, SENTINEL, _gen_world, assert_bf16, bf16_host, free, host_u16, to_dev

pytestmark = pytest.mark.gpu


def _both(gpu, w_sizes, bucket, D, r, reps_h, reps_d, scale, coords, out_coords):
    lay = OL.build_layout(w_sizes, bucket, D)
    plan = gpu.build_range_map(w_sizes, bucket, D, r)
    assert plan.norm_workspace_bytes <= gpu.NO_ALLOC_SCRATCH_BYTES
    n_out = plan.extent(out_coords)
    outs = []
    for no_alloc in (True, False):
        red = torch.full((max(n_out, 8),), SENTINEL, dtype=torch.int16, device=DEV)
        ns = torch.full((1,), -1.0, dtype=torch.float64, device=DEV)
        if no_alloc:
            gpu.grad_norm_sq_no_alloc(plan, reps_d, coords, scale, ns, red, out_coords)
        else:
            ws = torch.empty(plan.norm_workspace_bytes, dtype=torch.uint8, device=DEV)
            gpu.grad_norm_sq(plan, reps_d, coords, scale, ws, ns, red, out_coords)
            del ws
        torch.cuda.synchronize()
        outs.append((float(ns.item()), host_u16(red)))
    (n_static, red_static), (n_ws, red_ws) = outs
    assert np.float64(n_static).view(np.uint64) == np.float64(n_ws).view(np.uint64), (n_static, n_ws)
    assert_bf16(red_static, red_ws, "reduced gradient, static scratch vs workspace")
    want = OS.rank_norm_sq(lay, r, reps_h, coords, scale)
    assert_norm(n_static, want, plan.owned_numel, "squared norm vs oracle")
    return plan.norm_workspace_bytes


def test_no_alloc_norm_equals_the_workspace_call_twice_in_a_row(gpu):
    # first call: the fragmentation workload, rank 3 (16 contributions,
    # 4.8e6 owned elements, about 9,400 tiles)
    w = W.get("frag")
    lay = OL.build_layout(w.param_numel, w.bucket_numel, w.dp_size)
    reps_d = _gen_world(w, lay.buffer_numel)
    reps_h = [host_u16(x) for x in reps_d]
    big = _both(gpu, w.param_numel, w.bucket_numel, w.dp_size, 3, reps_h, reps_d, w.scale, gpu.WORLD, gpu.LOCAL)
    del reps_d, reps_h
    free()
    # second call, smaller: a ragged layout of 40,000-odd elements, D = 4,
    # LOCAL contributions, WORLD output
    rng = np.random.default_rng(99)
    sizes, bucket, D, r = [7000, 3, 12000, 1, 999, 20000, 5], 15000, 4, 2
    lay = OL.build_layout(sizes, bucket, D)
    full_h = [bf16_host(rng, lay.buffer_numel, 1.0) for _ in range(D)]
    loc_h = [OS.local_slices(lay, r, x) for x in full_h]
    small = _both(gpu, sizes, bucket, D, r, loc_h, [to_dev(x) for x in loc_h], 0.25, gpu.LOCAL, gpu.WORLD)
    assert small < big
    free()
