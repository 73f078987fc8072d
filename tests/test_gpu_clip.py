"""Global-norm clipping on the GPU (through the C-ABI) against the oracle.

Reading of the distributed-training notes, section 8.3: every rank's squared
gradient sum, summed across ranks, gives the global norm; the gradients are
clipped before the update. Bars:
  * clip coefficient and global norm from given squared norms: bit-exact;
  * a rank's squared norm: within the fp64 summation bound of a sequential
    sum (the two sides add in different orders), and bit-identical run to run;
  * the reduced gradient it writes: bit-exact, and nothing outside the owned
    elements is touched;
  * the clipped step at a given coefficient: bit-exact (coefficient 1: equal
    to the unclipped step; NaN: nothing changes);
  * end to end (norms -> coefficient -> clipped step, every rank): the
    coefficients agree, then every output bit-exact.
"""

import random

import numpy as np
import pytest
import torch

import oracle.layout as OL
import oracle.numerics as ON
import oracle.step as OS
import workloads as W
from test_gpu_parity import (DEV, SENTINEL, _gen_state, _gen_world, assert_bf16, assert_f32, bf16_host, free,
                             host_f32, host_u16, hp_kwargs, to_dev)

pytestmark = pytest.mark.gpu


def norm_bound(n: int, total: float) -> float:
    """|two fp64 sums of n non-negative terms| <= 2 n u total (u = 2^-53), each
    side's error being at most (n - 1) u total."""
    return 2.0 * max(n, 1) * 2.0**-53 * total + 1e-300


def assert_norm(got: float, want: float, n: int, what: str):
    if not np.isfinite(want):
        assert (np.isnan(want) and np.isnan(got)) or got == want, (what, got, want)
        return
    assert abs(got - want) <= norm_bound(n, want), (what, got, want)


def f64_dev(x):
    return torch.tensor(np.asarray(x, dtype=np.float64), device=DEV)


def test_clip_coefficient_bit_exact(gpu):
    rng = np.random.default_rng(41)
    cases = [([4.0], 1.0), ([0.25, 0.0], 1.0), ([16.0, 9.0], 1.0), ([0.0], 0.5), ([1e-30], 1e-20),
             ([1.0, np.inf], 1.0), ([np.nan, 1.0], 1.0), ([2.0**60, 1.0, -2.0**60], 1.0), ([1e300, 1e300], 1.0)]
    for _ in range(40):
        n = int(rng.integers(1, 65))
        cases.append((list(rng.random(n) * 10.0 ** rng.integers(-8, 8)), float(np.float32(rng.random() * 3))))
    coeff = torch.empty(1, dtype=torch.float32, device=DEV)
    norm = torch.empty(1, dtype=torch.float64, device=DEV)
    for parts, max_norm in cases:
        gpu.clip_coefficient(f64_dev(parts), max_norm, coeff, norm)
        want_c, want_n = ON.clip_coefficient(parts, max_norm)
        got_c, got_n = float(coeff.item()), float(norm.item())
        if np.isnan(want_c):
            assert np.isnan(got_c), (parts, max_norm)
        else:
            assert np.float32(got_c).view(np.uint32) == np.float32(want_c).view(np.uint32), (parts, max_norm)
        assert (np.isnan(want_n) and np.isnan(got_n)) or got_n == want_n, (parts, got_n, want_n)
    free()


def _norm_case(gpu, sizes, bucket, D, r, reps_h, scale, coords, out_coords):
    lay = OL.build_layout(sizes, bucket, D)
    plan = gpu.build_range_map(sizes, bucket, D, r)
    src_h = reps_h if coords == gpu.WORLD else [OS.local_slices(lay, r, x) for x in reps_h]
    src_d = [to_dev(x) for x in src_h]
    ws = torch.empty(plan.norm_workspace_bytes, dtype=torch.uint8, device=DEV)
    out = torch.empty(2, dtype=torch.float64, device=DEV)
    n_out = plan.extent(out_coords)
    red = torch.full((max(n_out, 8),), SENTINEL, dtype=torch.int16, device=DEV)
    gpu.grad_norm_sq(plan, src_d, coords, scale, ws, out[0:1], red, out_coords)
    gpu.grad_norm_sq(plan, src_d, coords, scale, ws, out[1:2])
    got = out.cpu().numpy()
    want = OS.rank_norm_sq(lay, r, src_h, coords, scale)
    assert got[0] == got[1], "run to run"
    assert_norm(got[0], want, plan.owned_numel, "squared norm")
    # the reduced gradient at the owned elements, nothing else
    want_red = np.full(max(n_out, 8), SENTINEL, np.uint16)
    for pc in OL.rank_pieces(lay, r):
        k0 = pc.shard_offset
        g0, g1 = OS._span(coords, pc.gbuf_world, k0)
        o0, o1 = OS._span(out_coords, pc.gbuf_world, k0)
        ON.reduce([x[g0:g1] for x in src_h], scale, out=want_red[o0:o1])
    assert_bf16(host_u16(red), want_red, "reduced_out")
    return got[0], want


@pytest.mark.parametrize("seed", range(8))
def test_norm_sq_random_layouts(gpu, seed):
    pr = random.Random(500 + seed)
    rng = np.random.default_rng(500 + seed)
    sizes = [pr.choice([pr.randint(1, 9), pr.randint(1, 3000), pr.randint(1, 70000)]) for _ in range(pr.randint(1, 20))]
    D = pr.choice([1, 2, 3, 4, 8, 16, 32])
    bucket = pr.randint(1, max(2, sum(sizes) // pr.choice([1, 3])))
    lay = OL.build_layout(sizes, bucket, D)
    reps_h = [bf16_host(rng, lay.buffer_numel, pr.choice([1e-3, 1.0])) for _ in range(D)]
    scale = pr.choice([1.0, 1.0 / D, 0.3])
    for r in sorted({0, D - 1, pr.randrange(D)}):
        _norm_case(gpu, sizes, bucket, D, r, reps_h, scale, pr.choice([gpu.WORLD, gpu.LOCAL]),
                   pr.choice([gpu.WORLD, gpu.LOCAL]))
    free()


def test_norm_sq_padding_only_rank_is_zero(gpu):
    plan = gpu.build_range_map([3, 2], 100, 4, 3)
    reps = [to_dev(np.full(8, 0x3F80, np.uint16)) for _ in range(4)]
    ws = torch.empty(plan.norm_workspace_bytes, dtype=torch.uint8, device=DEV)
    out = torch.full((1,), 7.0, dtype=torch.float64, device=DEV)
    gpu.grad_norm_sq(plan, reps, gpu.WORLD, 1.0, ws, out)
    assert out.item() == 0.0
    free()


def test_clipped_step_given_coefficient(gpu):
    rng = np.random.default_rng(43)
    sizes, bucket, D = [5000, 17, 1, 30000, 2049, 999], 12000, 8
    lay = OL.build_layout(sizes, bucket, D)
    N = lay.buffer_numel
    reps_h = [bf16_host(rng, N) for _ in range(D)]
    reps_d = [to_dev(x) for x in reps_h]
    hp = W.get("tiny").hp
    for r in (0, 3, 7):
        plan = gpu.build_range_map(sizes, bucket, D, r)
        Ln = plan.shard_numel
        st0 = [(rng.standard_normal(Ln) * 0.02).astype(np.float32), (rng.standard_normal(Ln) * 1e-3).astype(np.float32),
               ((rng.standard_normal(Ln) * 1e-3) ** 2).astype(np.float32)]
        for c in (1.0, float(np.float32(0.3721)), 1e-3, float("nan")):
            st = [to_dev(x) for x in st0]
            par = torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV)
            mg = torch.full((Ln,), -7.0, dtype=torch.float32, device=DEV)
            cd = torch.tensor([c], dtype=torch.float32, device=DEV)
            gpu.sharded_adam_step_clipped(plan, reps_d, gpu.WORLD, 0.125, *st, par, gpu.WORLD, grad_coeff=cd,
                                          main_grad_out=mg, **hp_kwargs(hp, 3))
            want = [x.copy() for x in st0]
            want_par = np.full(N, SENTINEL, np.uint16)
            want_mg = np.full(Ln, -7.0, np.float32)
            OS.rank_step(lay, r, reps_h, OS.WORLD, 0.125, *want, ON.hp_array(hp, 3), want_par, OS.WORLD, want_mg,
                         grad_coeff=c)
            for got, w, nm in zip(st, want, ("master", "exp_avg", "exp_avg_sq")):
                assert_f32(host_f32(got), w, f"r={r} c={c} {nm}")
            assert_bf16(host_u16(par), want_par, f"r={r} c={c} params")
            assert_f32(host_f32(mg), want_mg, f"r={r} c={c} main grad")
            if c == 1.0:
                st2 = [to_dev(x) for x in st0]
                par2 = torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV)
                gpu.sharded_adam_step(plan, reps_d, gpu.WORLD, 0.125, *st2, par2, gpu.WORLD, **hp_kwargs(hp, 3))
                for a, b in zip(st, st2):
                    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
                assert torch.equal(par, par2)
            if np.isnan(c):
                assert all(np.array_equal(host_f32(a), b) for a, b in zip(st, st0))
                assert (host_u16(par) == SENTINEL).all()
    free()


def _end_to_end(gpu, w, reps_d, reps_h, max_norm, ranks=None):
    """Every rank's squared norm, the coefficient, every rank's clipped step
    (fused, and from the reduced gradient with n_grads = 1), against the oracle."""
    D = w.dp_size
    lay = OL.build_layout(w.param_numel, w.bucket_numel, D)
    N = lay.buffer_numel
    plans = [gpu.build_range_map(w.param_numel, w.bucket_numel, D, r) for r in range(D)]
    parts = torch.empty(D, dtype=torch.float64, device=DEV)
    reds = []
    for r, plan in enumerate(plans):
        ws = torch.empty(plan.norm_workspace_bytes, dtype=torch.uint8, device=DEV)
        red = torch.empty(plan.shard_numel, dtype=torch.int16, device=DEV)
        gpu.grad_norm_sq(plan, reps_d, gpu.WORLD, w.scale, ws, parts[r:r + 1], red, gpu.LOCAL)
        reds.append(red)
    coeff = torch.empty(1, dtype=torch.float32, device=DEV)
    gnorm = torch.empty(1, dtype=torch.float64, device=DEV)
    gpu.clip_coefficient(parts, max_norm, coeff, gnorm)
    want_parts = [OS.rank_norm_sq(lay, r, reps_h, OS.WORLD, w.scale) for r in range(D)]
    got_parts = parts.cpu().numpy()
    for r in range(D):
        assert_norm(got_parts[r], want_parts[r], plans[r].owned_numel, f"rank {r} squared norm")
    want_c, want_n = ON.clip_coefficient(want_parts, max_norm)
    got_c = float(coeff.item())
    assert_norm(float(gnorm.item()), want_n, N, "global norm")
    if np.isnan(want_c):
        assert np.isnan(got_c)
    else:
        # the norms differ only by fp64 rounding; the fp32 coefficients agree
        assert np.float32(got_c) == np.float32(want_c), (got_c, want_c)
    hpk, hpa = hp_kwargs(w.hp, 1), ON.hp_array(w.hp, 1)
    par_f = torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV)
    par_r = torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV)
    want_par = np.full(N, SENTINEL, np.uint16)
    for r in (range(D) if ranks is None else ranks):
        plan = plans[r]
        st_f = _gen_state(w, plan.shard_numel)
        st_h = [host_f32(x) for x in st_f]
        st_r = [x.clone() for x in st_f]
        gpu.sharded_adam_step_clipped(plan, reps_d, gpu.WORLD, w.scale, *st_f, par_f, gpu.WORLD, grad_coeff=coeff,
                                      **hpk)
        gpu.sharded_adam_step_clipped(plan, [reds[r]], gpu.LOCAL, 1.0, *st_r, par_r, gpu.WORLD, grad_coeff=coeff,
                                      **hpk)
        OS.rank_step(lay, r, reps_h, OS.WORLD, w.scale, *st_h, hpa, want_par, OS.WORLD, grad_coeff=want_c)
        for a, b, want, nm in zip(st_f, st_r, st_h, ("master", "exp_avg", "exp_avg_sq")):
            assert_f32(host_f32(a), want, f"{w.name} r={r} {nm} fused")
            assert_f32(host_f32(b), want, f"{w.name} r={r} {nm} from reduced")
    assert_bf16(host_u16(par_f), want_par, f"{w.name} params fused")
    assert_bf16(host_u16(par_r), want_par, f"{w.name} params from reduced")
    return want_n, want_c


@pytest.mark.parametrize("name,max_norm", [("tiny", 0.01), ("tiny", 1e6), ("gpt2_small", 0.5), ("frag", 1e5)])
def test_clipping_end_to_end(gpu, name, max_norm):
    w = W.get(name)
    lay = OL.build_layout(w.param_numel, w.bucket_numel, w.dp_size)
    reps_d = _gen_world(w, lay.buffer_numel)
    reps_h = [host_u16(x) for x in reps_d]
    norm, c = _end_to_end(gpu, w, reps_d, reps_h, max_norm)
    if max_norm < norm:
        assert c < 1.0
    else:
        assert c == 1.0
    del reps_d
    free()


def test_found_inf_skips_every_rank(gpu):
    w = W.get("tiny")
    lay = OL.build_layout(w.param_numel, w.bucket_numel, w.dp_size)
    reps_d = _gen_world(w, lay.buffer_numel)
    reps_d[2][777] = 0x7F80          # +Inf in one rank's contribution to element 777
    reps_h = [host_u16(x) for x in reps_d]
    norm, c = _end_to_end(gpu, w, reps_d, reps_h, 1.0)
    assert not np.isfinite(norm) and np.isnan(c)
    free()


def test_clipped_step_state_beyond_the_infinity_cache(gpu):
    """The clipped step on a shard whose fp32 state exceeds 1 GiB (the
    non-temporal state path): GPT-2 small's parameters twice over plus three
    ragged ones at D = 2, rank 1 (about 124 M slots), coefficient 0.3721
    against the oracle element by element; a NaN coefficient changes
    nothing."""
    sizes = W.gpt2_small_params() * 2 + [4093, 1, 77777]
    bucket, D, r = 40_000_000, 2, 1
    lay = OL.build_layout(sizes, bucket, D)
    N = lay.buffer_numel
    reps_d = [W.normal_bf16(N, 1e-3, W.seed(2, 6, "grad", j), DEV).view(torch.int16) for j in range(D)]
    reps_h = [host_u16(x) for x in reps_d]
    hp = W.get("gpt2_small").hp
    plan = gpu.build_range_map(sizes, bucket, D, r)
    Ln = plan.shard_numel
    assert 12 * Ln > 1 << 30
    st0 = [W.normal_f32(Ln, 0.02, W.seed(2, 6, "master"), DEV), W.normal_f32(Ln, 1e-3, W.seed(2, 6, "m"), DEV),
           W.square_normal_f32(Ln, 1e-3, W.seed(2, 6, "v"), DEV)]
    st0_h = [host_f32(x) for x in st0]
    c = float(np.float32(0.3721))
    st = [x.clone() for x in st0]
    par = torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV)
    gpu.sharded_adam_step_clipped(plan, reps_d, gpu.WORLD, 1.0 / D, *st, par, gpu.WORLD,
                                  grad_coeff=torch.tensor([c], dtype=torch.float32, device=DEV), **hp_kwargs(hp, 2))
    want = [x.copy() for x in st0_h]
    want_par = np.full(N, SENTINEL, np.uint16)
    OS.rank_step(lay, r, reps_h, OS.WORLD, 1.0 / D, *want, ON.hp_array(hp, 2), want_par, OS.WORLD, grad_coeff=c)
    for got, w, nm in zip(st, want, ("master", "exp_avg", "exp_avg_sq")):
        assert_f32(host_f32(got), w, f"c={c} {nm}")
    assert_bf16(host_u16(par), want_par, f"c={c} params")
    st = [x.clone() for x in st0]
    par = torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV)
    gpu.sharded_adam_step_clipped(plan, reps_d, gpu.WORLD, 1.0 / D, *st, par, gpu.WORLD,
                                  grad_coeff=torch.tensor([float("nan")], dtype=torch.float32, device=DEV),
                                  **hp_kwargs(hp, 2))
    for a, b in zip(st, st0):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert bool((par == SENTINEL).all())
    del reps_d, st, st0, par
    free()
