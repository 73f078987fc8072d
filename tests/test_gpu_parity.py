"""Parity of the HIP path (through the C-ABI) with the CPU oracle.

Bar: range maps and every bf16 output bit-exact; fp32 master / exp_avg /
exp_avg_sq within a relative 1e-6 (absolute 1e-9 near zero) and, by design,
bit-exact too; NaN compared by NaN-ness only. Every input is seeded
(workloads.py); the oracle always runs on the bytes the device received.
"""

import random

import numpy as np
import pytest
import torch

import oracle.layout as OL
import oracle.numerics as ON
import oracle.step as OS
import workloads as W

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FBF
DEV = "cuda"


# ---- helpers ----------------------------------------------------------------------------

def to_dev(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).to(DEV)
    return torch.from_numpy(a.copy()).to(DEV)


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def host_f32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def assert_bf16(got: np.ndarray, want: np.ndarray, what: str):
    gn = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)
    wn = ((want & 0x7F80) == 0x7F80) & ((want & 0x7F) != 0)
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ"
    bad = np.flatnonzero(got[~gn] != want[~gn])
    assert bad.size == 0, f"{what}: {bad.size} bf16 mismatches, first at {bad[:5]}"


def assert_f32(got: np.ndarray, want: np.ndarray, what: str):
    gn, wn = np.isnan(got), np.isnan(want)
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ"
    g, w = got[~gn], want[~gn]
    with np.errstate(invalid="ignore"):
        close = (g == w) | (np.abs(g.astype(np.float64) - w) <= np.maximum(1e-6 * np.abs(w.astype(np.float64)), 1e-9))
    assert close.all(), f"{what}: {np.count_nonzero(~close)} outside rel 1e-6 / abs 1e-9"
    bad = np.flatnonzero(g.view(np.uint32) != w.view(np.uint32))
    assert bad.size == 0, f"{what}: {bad.size} fp32 values not bit-identical (within tolerance)"


def hp_kwargs(hp: dict, t: int) -> dict:
    return dict(lr=hp["lr"], beta1=hp["beta1"], beta2=hp["beta2"], eps=hp["eps"],
                weight_decay=hp["weight_decay"], step=t)


def bf16_host(rng, n, sigma=1e-2):
    x = (rng.standard_normal(n) * sigma).astype(np.float32)
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def local_stride(L: int) -> int:
    return max(8, (L + 7) // 8 * 8)


def free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# ---- rounding and reduction -----------------------------------------------------------------

def test_bf16_rounding_through_reduce(gpu):
    """D = 1: out = bf16(bf16(x) * scale); scales that produce ties, subnormals,
    overflow to Inf, signed zeros and NaN, compared with the oracle."""
    rng = np.random.default_rng(1)
    n = 1 << 16
    h = np.arange(n, dtype=np.uint32).astype(np.uint16)     # every bf16 pattern
    plan = gpu.build_range_map([n], n, 1, 0)
    rep = to_dev(h)
    out = torch.empty(n, dtype=torch.int16, device=DEV)
    scales = [1.0, 0.5, 2.0 ** -20, 2.0 ** -126, 3.0, 1.0 + 2.0 ** -8, 1.0 + 2.0 ** -23, 1.0 / 3.0,
              2.0 ** 100, -1.0, 0.0, float(np.float32(rng.random())), 1e-38, 2.0 ** 127]
    for s in scales:
        s = float(np.float32(s))
        gpu.reduce_scatter_local(plan, [rep], gpu.WORLD, s, out, gpu.WORLD)
        want = ON.reduce([h], s)
        assert_bf16(host_u16(out), want, f"scale {s!r}")
    free()


def test_allreduce_worked_example(gpu):
    # distributed-training notes, section "AllReduce": [1,2],[2,3],[3,3] -> [6,8]
    plan = gpu.build_range_map([2], 10, 3, 0)
    assert plan.buffer_numel == 3
    vals = [[1.0, 2.0, 0.0], [2.0, 3.0, 0.0], [3.0, 3.0, 0.0]]
    reps = [torch.tensor(v, dtype=torch.bfloat16, device=DEV).view(torch.int16) for v in vals]
    out = torch.full((8,), SENTINEL, dtype=torch.int16, device=DEV)
    gpu.force_all_reduce(plan, reps, 1.0, out)
    assert out.view(torch.bfloat16)[:3].float().tolist() == [6.0, 8.0, 0.0]
    assert (host_u16(out)[3:] == SENTINEL).all()
    free()


def _random_layout(pr):
    kind = pr.random()
    if kind < 0.3:
        sizes = [pr.randint(1, 20) for _ in range(pr.randint(1, 40))]
    elif kind < 0.7:
        sizes = [pr.randint(1, 9000) for _ in range(pr.randint(1, 30))]
    else:
        sizes = [pr.choice([1, 7, 8, 9, 2047, 2048, 2049, 60000]) for _ in range(pr.randint(1, 12))]
    D = pr.choice([1, 2, 3, 4, 5, 7, 8, 16, 32, 33])
    bucket = pr.randint(1, max(2, sum(sizes) // pr.choice([1, 2, 5])))
    return sizes, bucket, D


@pytest.mark.parametrize("seed", range(10))
def test_reduce_scatter_random_layouts(gpu, seed):
    pr = random.Random(seed)
    rng = np.random.default_rng(seed)
    sizes, bucket, D = _random_layout(pr)
    lay = OL.build_layout(sizes, bucket, D)
    N = lay.buffer_numel
    reps_h = [bf16_host(rng, N) for _ in range(D)]
    reps_d = [to_dev(r) for r in reps_h]
    scale = pr.choice([1.0, 1.0 / D, 0.3, 2.0])
    full = OS.all_reduce(reps_h, scale)
    for r in sorted({0, D - 1, pr.randrange(D)}):
        plan = gpu.build_range_map(sizes, bucket, D, r)
        Ln = plan.shard_numel
        for in_c in (gpu.WORLD, gpu.LOCAL):
            src_h = reps_h if in_c == gpu.WORLD else [OS.local_slices(lay, r, x) for x in reps_h]
            src_d = reps_d if in_c == gpu.WORLD else [to_dev(x) for x in src_h]
            for out_c in (gpu.WORLD, gpu.LOCAL):
                n_out = N if out_c == gpu.WORLD else Ln
                out = torch.full((max(n_out, 8),), SENTINEL, dtype=torch.int16, device=DEV)
                gpu.reduce_scatter_local(plan, src_d, in_c, scale, out, out_c)
                want = np.full(max(n_out, 8), SENTINEL, np.uint16)
                OS.reduce_scatter(lay, r, src_h, in_c, scale, want, out_c)
                assert_bf16(host_u16(out), want, f"rs r={r} in={in_c} out={out_c}")
        # restricted all-reduce == reduce-scatter
        out = torch.empty(max(N, 8), dtype=torch.int16, device=DEV)
        gpu.force_all_reduce(plan, reps_d, scale, out)
        assert_bf16(host_u16(out)[:N], full, "force_all_reduce")
    free()


def test_reduce_scatter_in_place(gpu):
    rng = np.random.default_rng(5)
    sizes, bucket, D = [1000, 3, 4097, 20000, 5], 9000, 4
    lay = OL.build_layout(sizes, bucket, D)
    N = lay.buffer_numel
    reps_h = [bf16_host(rng, N) for _ in range(D)]
    for r in range(D):
        plan = gpu.build_range_map(sizes, bucket, D, r)
        reps_d = [to_dev(x) for x in reps_h]
        gpu.reduce_scatter_local(plan, reps_d, gpu.WORLD, 0.25, reps_d[r], gpu.WORLD)
        want = reps_h[r].copy()
        OS.reduce_scatter(lay, r, reps_h, gpu.WORLD, 0.25, want, gpu.WORLD)
        assert_bf16(host_u16(reps_d[r]), want, f"in-place r={r}")
    # force_all_reduce in place into replica 0
    plan = gpu.build_range_map(sizes, bucket, D, 0)
    reps_d = [to_dev(x) for x in reps_h]
    gpu.force_all_reduce(plan, reps_d, 0.25, reps_d[0])
    assert_bf16(host_u16(reps_d[0]), OS.all_reduce(reps_h, 0.25), "far in place")
    free()


# ---- the fused step ----------------------------------------------------------------------------

def run_rank_step(gpu, sizes, bucket, D, r, reps_h, state_h, scale, hp, t, grad_c, param_c, reps_d=None,
                  with_main_grad=True):
    """One step on the GPU and in the oracle; compare everything."""
    lay = OL.build_layout(sizes, bucket, D)
    plan = gpu.build_range_map(sizes, bucket, D, r)
    N, Ln = plan.buffer_numel, plan.shard_numel
    if grad_c == gpu.WORLD:
        src_h = reps_h
    else:
        src_h = [OS.local_slices(lay, r, x) for x in reps_h]
    if reps_d is None or grad_c == gpu.LOCAL:
        reps_d = [to_dev(x) for x in src_h]
    master, m, v = (to_dev(x) for x in state_h)
    n_par = N if param_c == gpu.WORLD else Ln
    par = torch.full((max(n_par, 8),), SENTINEL, dtype=torch.int16, device=DEV)
    mg = torch.full((max(Ln, 8),), -7.0, dtype=torch.float32, device=DEV) if with_main_grad else None
    gpu.sharded_adam_step(plan, reps_d, grad_c, scale, master, m, v, par, param_c, main_grad_out=mg,
                          **hp_kwargs(hp, t))
    want = [x.copy() for x in state_h]
    want_par = np.full(max(n_par, 8), SENTINEL, np.uint16)
    want_mg = np.full(max(Ln, 8), -7.0, np.float32) if with_main_grad else None
    OS.rank_step(lay, r, src_h, grad_c, scale, *want, ON.hp_array(hp, t), want_par, param_c,
                 None if want_mg is None else want_mg[:Ln])
    for got, w, name in zip((master, m, v), want, ("master", "exp_avg", "exp_avg_sq")):
        assert_f32(host_f32(got), w, f"{name} r={r}")
    assert_bf16(host_u16(par), want_par, f"params r={r}")
    if with_main_grad:
        assert_f32(host_f32(mg), want_mg, f"main grad r={r}")
    return [host_f32(x) for x in (master, m, v)], host_u16(par)


def test_tiny_all_ranks_ten_steps(gpu):
    """The Tiny workload: 1000 elements, D = 4, every rank, ten steps with
    fresh grads each step; the one parameter the rank edge cuts (120 / 300)
    and ranks whose shard starts off the 8-element phase."""
    w = W.get("tiny")
    lay = OL.build_layout(w.param_numel, w.bucket_numel, w.dp_size)
    master0 = W.normal_f32(lay.buffer_numel, w.master_sigma, W.seed(1, 0, "master")).numpy()
    for r in w.verify_ranks:
        Ln = OL.shard_numel(lay, r)
        state = [OS.gather_shard(lay, r, master0), np.zeros(Ln, np.float32), np.zeros(Ln, np.float32)]
        for t in range(1, w.steps + 1):
            reps = [W.bf16_bits(W.normal_bf16(1000, w.grad_sigma, W.seed(1, t, "grad", j)))
                    for j in range(w.dp_size)]
            state, par = run_rank_step(gpu, w.param_numel, w.bucket_numel, w.dp_size, r, reps, state, w.scale,
                                       w.hp, t, gpu.WORLD, gpu.WORLD)
    free()


@pytest.mark.parametrize("seed", range(16))
def test_fused_step_random_layouts(gpu, seed):
    pr = random.Random(1000 + seed)
    rng = np.random.default_rng(1000 + seed)
    sizes, bucket, D = _random_layout(pr)
    lay = OL.build_layout(sizes, bucket, D)
    N = lay.buffer_numel
    reps_h = [bf16_host(rng, N, pr.choice([1e-3, 1e-2, 1.0])) for _ in range(D)]
    scale = pr.choice([1.0, 1.0 / D, 1.0 / 3.0, 0.5])
    hp = dict(lr=pr.choice([1e-3, 3e-4]), beta1=0.9, beta2=pr.choice([0.999, 0.95]), eps=1e-8,
              weight_decay=pr.choice([0.0, 0.01, 0.1]))
    t = pr.choice([1, 2, 10, 1000])
    for r in sorted({0, D - 1, pr.randrange(D)}):
        Ln = OL.shard_numel(lay, r)
        state = [(rng.standard_normal(Ln) * 0.02).astype(np.float32),
                 (rng.standard_normal(Ln) * 1e-3).astype(np.float32),
                 ((rng.standard_normal(Ln) * 1e-3) ** 2).astype(np.float32)]
        run_rank_step(gpu, sizes, bucket, D, r, reps_h, state, scale, hp, t,
                      pr.choice([gpu.WORLD, gpu.LOCAL]), pr.choice([gpu.WORLD, gpu.LOCAL]))
    free()


def test_rank_with_only_padding(gpu):
    # 5 elements at D = 4: padded to 8, rank 3's range is all padding
    rng = np.random.default_rng(3)
    sizes, bucket, D = [3, 2], 100, 4
    plan = gpu.build_range_map(sizes, bucket, D, 3)
    assert plan.owned_numel == 0
    reps = [to_dev(bf16_host(rng, 8)) for _ in range(D)]
    st = [torch.full((8,), 1.5, dtype=torch.float32, device=DEV) for _ in range(3)]
    par = torch.full((8,), SENTINEL, dtype=torch.int16, device=DEV)
    gpu.sharded_adam_step(plan, reps, gpu.WORLD, 0.25, *st, par, gpu.WORLD, **hp_kwargs(W.get("tiny").hp, 1))
    gpu.writeback_params(plan, st[0], par, gpu.WORLD)
    torch.cuda.synchronize()
    assert (host_u16(par) == SENTINEL).all()
    assert all((host_f32(x) == 1.5).all() for x in st)
    # its reduce-scatter still covers the padding of its range
    out = torch.full((8,), SENTINEL, dtype=torch.int16, device=DEV)
    gpu.reduce_scatter_local(plan, reps, gpu.WORLD, 1.0, out, gpu.WORLD)
    want = np.full(8, SENTINEL, np.uint16)
    OS.reduce_scatter(OL.build_layout(sizes, bucket, D), 3, [host_u16(x) for x in reps], 0, 1.0, want, 0)
    assert_bf16(host_u16(out), want, "padding-only rs")
    free()


def test_prereduced_and_writeback_equal_fused(gpu):
    """reduce_scatter_local (or force_all_reduce) then the step with the one
    reduced buffer and scale 1, and the step without write-back followed by
    writeback_params, give the fused step's bytes."""
    rng = np.random.default_rng(9)
    sizes, bucket, D = [5000, 17, 1, 30000, 2049, 999], 12000, 8
    lay = OL.build_layout(sizes, bucket, D)
    N = lay.buffer_numel
    reps_h = [bf16_host(rng, N) for _ in range(D)]
    reps_d = [to_dev(x) for x in reps_h]
    hp = W.get("tiny").hp
    for r in range(D):
        plan = gpu.build_range_map(sizes, bucket, D, r)
        Ln = plan.shard_numel
        st0 = [(rng.standard_normal(Ln) * 0.02).astype(np.float32), np.zeros(Ln, np.float32),
               np.zeros(Ln, np.float32)]
        outs = []
        for variant in ("fused", "rs", "far", "split"):
            st = [to_dev(x) for x in st0]
            par = torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV)
            if variant == "fused":
                gpu.sharded_adam_step(plan, reps_d, gpu.WORLD, 0.125, *st, par, gpu.WORLD, **hp_kwargs(hp, 1))
            elif variant == "rs":
                red = torch.empty(Ln, dtype=torch.int16, device=DEV)
                gpu.reduce_scatter_local(plan, reps_d, gpu.WORLD, 0.125, red, gpu.LOCAL)
                gpu.sharded_adam_step(plan, [red], gpu.LOCAL, 1.0, *st, par, gpu.WORLD, **hp_kwargs(hp, 1))
            elif variant == "far":
                red = torch.empty(N, dtype=torch.int16, device=DEV)
                gpu.force_all_reduce(plan, reps_d, 0.125, red)
                gpu.sharded_adam_step(plan, [red], gpu.WORLD, 1.0, *st, par, gpu.WORLD, **hp_kwargs(hp, 1))
            else:
                gpu.sharded_adam_step(plan, reps_d, gpu.WORLD, 0.125, *st, None, gpu.WORLD, **hp_kwargs(hp, 1))
                gpu.writeback_params(plan, st[0], par, gpu.WORLD)
            outs.append(([host_f32(x) for x in st], host_u16(par)))
        for (st, par), name in zip(outs[1:], ("rs", "far", "split")):
            for a, b in zip(st, outs[0][0]):
                assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), name
            assert np.array_equal(par, outs[0][1]), name
    free()


def test_nan_inf_propagate(gpu):
    rng = np.random.default_rng(10)
    sizes, bucket, D = [300, 4000], 5000, 4
    lay = OL.build_layout(sizes, bucket, D)
    N = lay.buffer_numel
    reps_h = [bf16_host(rng, N) for _ in range(D)]
    nan, inf, ninf = 0x7FC1, 0x7F80, 0xFF80
    for k, pos in enumerate(rng.choice(N, 60, replace=False)):
        reps_h[k % D][pos] = (nan, inf, ninf)[k % 3]
    for r in range(D):
        Ln = OL.shard_numel(lay, r)
        st = [(rng.standard_normal(Ln) * 0.02).astype(np.float32), np.zeros(Ln, np.float32),
              np.zeros(Ln, np.float32)]
        run_rank_step(gpu, sizes, bucket, D, r, reps_h, st, 0.25, W.get("tiny").hp, 1, gpu.WORLD, gpu.WORLD)
    free()


def test_error_paths(gpu):
    Z = gpu
    plan = Z.build_range_map([100, 28], 64, 2, 1)
    x = torch.zeros(256, dtype=torch.int16, device=DEV)
    f = torch.zeros(256, dtype=torch.float32, device=DEV)
    g = torch.zeros(256, dtype=torch.float32, device=DEV)
    h = torch.zeros(256, dtype=torch.float32, device=DEV)
    hp = hp_kwargs(W.get("tiny").hp, 1)
    with pytest.raises(Z.ZdoError) as e:
        Z.reduce_scatter_local(plan, [x] * 65, Z.WORLD, 1.0, x, Z.WORLD)      # more than 64 contributions
    assert e.value.code == Z.EINVAL
    with pytest.raises(Z.ZdoError) as e:
        Z.reduce_scatter_local(plan, [x, x], Z.WORLD, 1.0, x[8:], Z.WORLD)    # partial overlap
    assert e.value.code == Z.EALIAS
    with pytest.raises(Z.ZdoError) as e:
        Z.reduce_scatter_local(plan, [x, x], 7, 1.0, x, Z.WORLD)
    assert e.value.code == Z.EINVAL
    with pytest.raises(Z.ZdoError) as e:
        Z.sharded_adam_step(plan, [x, x], Z.WORLD, 1.0, f, f, h, None, **hp)   # master == exp_avg
    assert e.value.code == Z.EALIAS
    with pytest.raises(Z.ZdoError) as e:
        Z.sharded_adam_step(plan, [x, x], Z.WORLD, 1.0, f[1:], g, h, None, **hp)   # misaligned
    assert e.value.code == Z.EALIGN
    with pytest.raises(Z.ZdoError) as e:
        Z.sharded_adam_step(plan, [], Z.WORLD, 1.0, f, g, h, None, **hp)           # no contribution
    assert e.value.code == Z.EINVAL
    with pytest.raises(Z.ZdoError) as e:
        Z.sharded_adam_step(plan, [x, x], Z.WORLD, 1.0, f, g, h, x, Z.WORLD, **dict(hp, step=0))
    assert e.value.code == Z.EINVAL
    with pytest.raises(Z.ZdoError) as e:
        Z.sharded_adam_step(plan, [x, x], Z.WORLD, 1.0, f, g, h, x, Z.WORLD, **dict(hp, beta2=1.0))
    assert e.value.code == Z.EINVAL
    with pytest.raises(Z.ZdoError) as e:
        Z.writeback_params(plan, f, f.view(torch.int16)[:256], Z.WORLD)
    assert e.value.code == Z.EALIAS
    with pytest.raises(ValueError):
        Z.sharded_adam_step(plan, [x, x], Z.WORLD, 1.0, f[:10], g, h, None, **hp)   # too small
    torch.cuda.synchronize()
    free()


# ---- the five workloads at full size ---------------------------------------------------------

def _gen_world(w, N, step=0):
    reps = []
    for j in range(w.dp_size):
        t = torch.empty(N, dtype=torch.bfloat16, device=DEV)
        W.normal_bf16(N, w.grad_sigma, W.seed(w.cfg, step, "grad", j), out=t,
                      probe_fraction=w.probe_fraction, probe_seed=W.seed(w.cfg, step, "probe", j))
        reps.append(t.view(torch.int16))
    return reps


def _gen_state(w, Ln):
    master = W.normal_f32(Ln, w.master_sigma, W.seed(w.cfg, 0, "master"), DEV)
    m = W.normal_f32(Ln, w.m_sigma, W.seed(w.cfg, 0, "m"), DEV)
    v = W.square_normal_f32(Ln, w.v_sigma, W.seed(w.cfg, 0, "v"), DEV)
    return master, m, v


@pytest.mark.parametrize("name", ["gpt2_small", "frag"])
def test_workload_every_rank_full_compare(gpu, name):
    """GPT-2-small shape (D = 8) and the fragmentation stress (D = 16, +-65504
    probes): every rank, every element compared; for the stress workload also
    force_all_reduce over the whole buffer and the step on its output."""
    w = W.get(name)
    lay = OL.build_layout(w.param_numel, w.bucket_numel, w.dp_size)
    N = lay.buffer_numel
    reps_d = _gen_world(w, N)
    reps_h = [host_u16(x) for x in reps_d]
    hpk = hp_kwargs(w.hp, 1)
    hpa = ON.hp_array(w.hp, 1)
    far_h = far_d = None
    if name == "frag":
        plan0 = gpu.build_range_map(w.param_numel, w.bucket_numel, w.dp_size, 0)
        far_d = torch.empty(N, dtype=torch.int16, device=DEV)
        gpu.force_all_reduce(plan0, reps_d, w.scale, far_d)
        far_h = host_u16(far_d)
        assert_bf16(far_h, OS.all_reduce(reps_h, w.scale), "force_all_reduce (whole buffer)")
    par = torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV)
    want_par = np.full(N, SENTINEL, np.uint16)
    for r in w.verify_ranks:
        plan = gpu.build_range_map(w.param_numel, w.bucket_numel, w.dp_size, r)
        Ln = plan.shard_numel
        st = _gen_state(w, Ln)
        st_h = [host_f32(x) for x in st]
        gpu.sharded_adam_step(plan, reps_d, gpu.WORLD, w.scale, *st, par, gpu.WORLD, **hpk)
        OS.rank_step(lay, r, reps_h, OS.WORLD, w.scale, *st_h, hpa, want_par, OS.WORLD)
        for got, want, nm in zip(st, st_h, ("master", "exp_avg", "exp_avg_sq")):
            assert_f32(host_f32(got), want, f"{name} r={r} {nm}")
        if far_d is not None:
            st2 = _gen_state(w, Ln)
            par2 = torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV)
            gpu.sharded_adam_step(plan, [far_d], gpu.WORLD, 1.0, *st2, par2, gpu.WORLD, **hpk)
            for got, want, nm in zip(st2, st_h, ("master", "exp_avg", "exp_avg_sq")):
                assert_f32(host_f32(got), want, f"{name} r={r} {nm} via force_all_reduce")
            del st2, par2
        del st
    # all ranks wrote their owned ranges; padding keeps the sentinel
    assert_bf16(host_u16(par), want_par, f"{name} params (all ranks)")
    del reps_d, far_d, par
    free()


def test_state_beyond_the_infinity_cache(gpu):
    """A shard whose fp32 state (12 bytes per slot) exceeds 1 GiB, well
    beyond the 256 MB Infinity Cache, takes the step's and the write-back's
    non-temporal state accesses: GPT-2 small's parameters twice over plus
    three ragged ones at D = 2 (L about 124 M slots, 1.49 GB of state), rank
    1 in WORLD and rank 0 in LOCAL coordinates, every element compared, main
    grad included; then writeback_params of the updated master equals the
    step's parameters."""
    sizes = W.gpt2_small_params() * 2 + [4093, 1, 77777]
    bucket, D = 40_000_000, 2
    lay = OL.build_layout(sizes, bucket, D)
    N = lay.buffer_numel
    reps_d = [W.normal_bf16(N, 1e-3, W.seed(2, 5, "grad", j), DEV).view(torch.int16) for j in range(D)]
    reps_h = [host_u16(x) for x in reps_d]
    hp = W.get("gpt2_small").hp
    for r, c in ((1, gpu.WORLD), (0, gpu.LOCAL)):
        Ln = OL.shard_numel(lay, r)
        assert 12 * Ln > 1 << 30
        state = [W.f32_host(W.normal_f32(Ln, 0.02, W.seed(2, 5, "master", r), DEV)),
                 W.f32_host(W.normal_f32(Ln, 1e-3, W.seed(2, 5, "m", r), DEV)),
                 W.f32_host(W.square_normal_f32(Ln, 1e-3, W.seed(2, 5, "v", r), DEV))]
        new_state, par_h = run_rank_step(gpu, sizes, bucket, D, r, reps_h, state, 1.0 / D, hp, 3, c, c,
                                         reps_d=reps_d if c == gpu.WORLD else None)
        # writeback_params of the updated master (non-temporal loads here)
        # gives the step's parameter bytes, sentinels elsewhere included
        plan = gpu.build_range_map(sizes, bucket, D, r)
        par2 = torch.full((par_h.size,), SENTINEL, dtype=torch.int16, device=DEV)
        gpu.writeback_params(plan, to_dev(new_state[0]), par2, c)
        assert_bf16(host_u16(par2), par_h, f"writeback_params r={r}")
        del par2
        free()
    del reps_d
    free()


def test_buffers_object_equals_tensor_lists(gpu):
    """zdo.Buffers (checked once, reused) gives the same bytes as lists of
    tensors, per bucket and whole; a too-short buffer set is refused."""
    rng = np.random.default_rng(11)
    sizes, bucket, D = [700, 5, 1300, 64, 999], 1500, 4
    lay = OL.build_layout(sizes, bucket, D)
    N = lay.buffer_numel
    reps = [to_dev(bf16_host(rng, N)) for _ in range(D)]
    plan = gpu.build_range_map(sizes, bucket, D, 2)
    Ln = plan.shard_numel
    st0 = [(rng.standard_normal(Ln) * 0.02).astype(np.float32) for _ in range(2)] + \
          [((rng.standard_normal(Ln) * 1e-3) ** 2).astype(np.float32)]
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=3)
    results = []
    for use_buffers in (False, True):
        g = gpu.Buffers(reps, "replicas") if use_buffers else reps
        st = [to_dev(x) for x in st0]
        par = torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV)
        for b in reversed(range(plan.buckets().size)):
            gpu.sharded_adam_step(plan, g, gpu.WORLD, 0.25, *st, par, gpu.WORLD, buckets=(b, b + 1), **hp)
        red = torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV)
        gpu.reduce_scatter_local(plan, g, gpu.WORLD, 0.25, red, gpu.WORLD)
        results.append([host_f32(x) for x in st] + [host_u16(par), host_u16(red)])
    for a, b in zip(*results):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    short = gpu.Buffers([r[: N - 1] for r in reps], "replicas")
    with pytest.raises(ValueError, match="elements per buffer"):
        gpu.reduce_scatter_local(plan, short, gpu.WORLD, 0.25, red, gpu.WORLD)
    free()


# ---- edge cases of size and arithmetic --------------------------------------------------------

@pytest.mark.parametrize("D", [64, 48])
def test_max_replicas_runtime_path(gpu, D):
    """D = 64 (the ABI maximum) and D = 48 take the kernels' runtime-D loop."""
    rng = np.random.default_rng(600 + D)
    sizes, bucket = [7000, 3, 65536, 1, 2500], 20000
    lay = OL.build_layout(sizes, bucket, D)
    reps_h = [bf16_host(rng, lay.buffer_numel, 1e-2) for _ in range(D)]
    hp = W.get("tiny").hp
    for r in (0, D // 3, D - 1):
        Ln = OL.shard_numel(lay, r)
        st = [(rng.standard_normal(Ln) * 0.02).astype(np.float32), np.zeros(Ln, np.float32),
              np.zeros(Ln, np.float32)]
        run_rank_step(gpu, sizes, bucket, D, r, reps_h, st, 1.0 / D, hp, 2, gpu.WORLD, gpu.LOCAL)
        plan = gpu.build_range_map(sizes, bucket, D, r)
        out = torch.full((lay.buffer_numel,), SENTINEL, dtype=torch.int16, device=DEV)
        gpu.reduce_scatter_local(plan, [to_dev(x) for x in reps_h], gpu.WORLD, 1.0 / D, out, gpu.WORLD)
        want = np.full(lay.buffer_numel, SENTINEL, np.uint16)
        OS.reduce_scatter(lay, r, reps_h, OS.WORLD, 1.0 / D, want, OS.WORLD)
        assert_bf16(host_u16(out), want, f"rs D={D} r={r}")
    free()


@pytest.mark.parametrize("scale", [0.0, -1.0, 3.0e38, 1.0e-40, float(np.float32(7.0 / 3.0))])
def test_unusual_scales(gpu, scale):
    """Zero, negative, overflowing and subnormal scales take the same rounding
    path on both sides (bf16 of each scaled term, Inf and subnormals kept)."""
    rng = np.random.default_rng(7)
    sizes, bucket, D = [3000, 5000], 4000, 4
    lay = OL.build_layout(sizes, bucket, D)
    reps_h = [bf16_host(rng, lay.buffer_numel, 1.0) for _ in range(D)]
    for r in range(D):
        Ln = OL.shard_numel(lay, r)
        st = [(rng.standard_normal(Ln) * 0.02).astype(np.float32), np.zeros(Ln, np.float32),
              np.zeros(Ln, np.float32)]
        run_rank_step(gpu, sizes, bucket, D, r, reps_h, st, scale, W.get("tiny").hp, 1, gpu.WORLD, gpu.WORLD)
    free()


def test_many_single_element_parameters(gpu):
    """40,000 one-element parameters and a few larger ones: thousands of pieces
    per rank, every chunk an edge of some piece but the runs coalesce."""
    rng = np.random.default_rng(9)
    sizes = [1] * 40000 + [4097, 1, 33, 1, 70000]
    bucket, D = 9000, 8
    lay = OL.build_layout(sizes, bucket, D)
    reps_h = [bf16_host(rng, lay.buffer_numel, 1e-2) for _ in range(D)]
    for r in (0, 5, 7):
        Ln = OL.shard_numel(lay, r)
        st = [(rng.standard_normal(Ln) * 0.02).astype(np.float32), (rng.standard_normal(Ln) * 1e-3).astype(np.float32),
              ((rng.standard_normal(Ln) * 1e-3) ** 2).astype(np.float32)]
        run_rank_step(gpu, sizes, bucket, D, r, reps_h, st, 0.125, W.get("tiny").hp, 4, gpu.LOCAL, gpu.WORLD)
    free()


# ---- bucket by bucket -------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["frag", "layout"])
def test_bucket_ranges(gpu, name):
    """Page 1, §2/§4.2: buckets handled one at a time as their grads become
    ready. Per-bucket calls over every bucket, in reverse order, equal the full
    call and the oracle bit for bit; a partial range touches its buckets only;
    an empty range nothing; bad ranges are EINVAL."""
    if name == "frag":
        w = W.get("frag")
        sizes, bucket, D, r = w.param_numel, w.bucket_numel, w.dp_size, 3
        lay = OL.build_layout(sizes, bucket, D)
        reps_d = _gen_world(w, lay.buffer_numel)
        reps_h = [host_u16(x) for x in reps_d]
    else:
        rng = np.random.default_rng(77)
        sizes, bucket, D, r = [3000, 1, 9000, 17, 4500, 2, 7000, 300, 11000], 6000, 4, 1
        lay = OL.build_layout(sizes, bucket, D)
        reps_h = [bf16_host(rng, lay.buffer_numel) for _ in range(D)]
        reps_d = [to_dev(x) for x in reps_h]
    plan = gpu.build_range_map(sizes, bucket, D, r)
    nb = len(lay.buckets)
    assert nb >= 3
    N, Ln = plan.buffer_numel, plan.shard_numel
    hp = W.get("tiny").hp
    rng = np.random.default_rng(5)
    st0 = [(rng.standard_normal(Ln) * 0.02).astype(np.float32), (rng.standard_normal(Ln) * 1e-3).astype(np.float32),
           ((rng.standard_normal(Ln) * 1e-3) ** 2).astype(np.float32)]
    scale = 1.0 / D

    def run(ranges):
        st = [to_dev(x) for x in st0]
        par = torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV)
        for b0, b1 in ranges:
            gpu.sharded_adam_step(plan, reps_d, gpu.WORLD, scale, *st, par, gpu.WORLD, buckets=(b0, b1),
                                  **hp_kwargs(hp, 2))
        return [host_f32(x) for x in st], host_u16(par)

    def oracle(ranges):
        st = [x.copy() for x in st0]
        par = np.full(N, SENTINEL, np.uint16)
        for b0, b1 in ranges:
            OS.rank_step(lay, r, reps_h, OS.WORLD, scale, *st, ON.hp_array(hp, 2), par, OS.WORLD, buckets=(b0, b1))
        return st, par

    for ranges in ([(b, b + 1) for b in reversed(range(nb))], [(0, nb)], [(2, nb - 1)], [(1, 1)]):
        got_st, got_par = run(ranges)
        want_st, want_par = oracle(ranges)
        for g, wv, nm in zip(got_st, want_st, ("master", "exp_avg", "exp_avg_sq")):
            assert_f32(g, wv, f"{name} {ranges[:2]} {nm}")
        assert_bf16(got_par, want_par, f"{name} {ranges[:2]} params")
    # the full call equals the per-bucket calls
    st = [to_dev(x) for x in st0]
    par = torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV)
    gpu.sharded_adam_step(plan, reps_d, gpu.WORLD, scale, *st, par, gpu.WORLD, **hp_kwargs(hp, 2))
    per_st, per_par = run([(b, b + 1) for b in reversed(range(nb))])
    assert all(np.array_equal(host_f32(a).view(np.uint32), b.view(np.uint32)) for a, b in zip(st, per_st))
    assert np.array_equal(host_u16(par), per_par)
    # reduce-scatter in two halves, upper half first
    out = torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV)
    gpu.reduce_scatter_local(plan, reps_d, gpu.WORLD, scale, out, gpu.WORLD, buckets=(nb // 2, nb))
    gpu.reduce_scatter_local(plan, reps_d, gpu.WORLD, scale, out, gpu.WORLD, buckets=(0, nb // 2))
    want = np.full(N, SENTINEL, np.uint16)
    OS.reduce_scatter(lay, r, reps_h, OS.WORLD, scale, want, OS.WORLD)
    assert_bf16(host_u16(out), want, f"{name} rs halves")
    for bad in ((2, 1), (-1, 2), (0, nb + 1)):
        with pytest.raises(gpu.ZdoError) as e:
            gpu.sharded_adam_step(plan, reps_d, gpu.WORLD, scale, *st, par, gpu.WORLD, buckets=bad,
                                  **hp_kwargs(hp, 2))
        assert e.value.code == gpu.EINVAL
        with pytest.raises(gpu.ZdoError) as e:
            gpu.reduce_scatter_local(plan, reps_d, gpu.WORLD, scale, out, gpu.WORLD, buckets=bad)
        assert e.value.code == gpu.EINVAL
    del reps_d
    free()


# ---- several distributed-optimizer instances ----------------------------------------------

def _own_mask(lay, r, Ln):
    own = np.zeros(Ln, bool)
    for pc in OL.rank_pieces(lay, r):
        own[pc.shard_offset:pc.shard_offset + pc.gbuf_world.size] = True
    return own


@pytest.mark.parametrize("D,n_inst,coords", [(4, 2, "world"), (8, 4, "local"), (2, 3, "world"), (16, 2, "local"),
                                             (3, 5, "world"), (1, 4, "local"), (5, 1, "world"), (32, 2, "local")])
def test_two_level_instances(gpu, D, n_inst, coords):
    """Page 1, §5: the reduce-scatter runs within each instance of D ranks and
    an all-reduce across the n_inst instances follows. The oracle composes one
    reduce-scatter per instance and the step on the instance results (scale
    1). On the GPU the same composition through the existing calls, and the
    one-pass sharded_adam_step_instances, both bit for bit against it."""
    rng = np.random.default_rng(100 * D + n_inst)
    sizes, bucket = [5000, 13, 20000, 1, 4097, 2200], 9000
    lay = OL.build_layout(sizes, bucket, D)
    N = lay.buffer_numel
    reps_h = [[bf16_host(rng, N) for _ in range(D)] for _ in range(n_inst)]
    scale = float(np.float32(1.0 / (D * n_inst)))
    hp = W.get("tiny").hp
    gc = gpu.WORLD if coords == "world" else gpu.LOCAL
    for r in sorted({0, D - 1, int(rng.integers(D))}):
        plan = gpu.build_range_map(sizes, bucket, D, r)
        Ln = plan.shard_numel
        src_h = [[x if gc == gpu.WORLD else OS.local_slices(lay, r, x) for x in inst] for inst in reps_h]
        src_d = [[to_dev(x) for x in inst] for inst in src_h]
        # oracle: reduce-scatter within each instance, then the step on the results
        rs_h = []
        for i in range(n_inst):
            want = np.zeros(Ln, np.uint16)
            OS.reduce_scatter(lay, r, src_h[i], gc, scale, want, OS.LOCAL)
            rs_h.append(want)
        want_red = np.zeros(Ln, np.uint16)
        OS.reduce_scatter(lay, r, rs_h, OS.LOCAL, 1.0, want_red, OS.LOCAL)
        state_h = [(rng.standard_normal(Ln) * 0.02).astype(np.float32),
                   (rng.standard_normal(Ln) * 1e-3).astype(np.float32),
                   ((rng.standard_normal(Ln) * 1e-3) ** 2).astype(np.float32)]
        want = [x.copy() for x in state_h]
        want_par = np.full(max(N, 8), SENTINEL, np.uint16)
        want_mg = np.full(max(Ln, 8), -7.0, np.float32)
        OS.rank_step(lay, r, rs_h, OS.LOCAL, 1.0, *want, ON.hp_array(hp, 3), want_par, OS.WORLD, want_mg[:Ln])
        own = _own_mask(lay, r, Ln)
        assert np.array_equal(want_mg[:Ln][own], ON.widen(want_red)[own])

        # GPU, composed: one reduce_scatter_local per instance, then the step
        rs_d = []
        for i in range(n_inst):
            out = torch.zeros(Ln, dtype=torch.int16, device=DEV)
            gpu.reduce_scatter_local(plan, src_d[i], gc, scale, out, gpu.LOCAL)
            assert_bf16(host_u16(out), rs_h[i], f"instance {i} rs r={r}")
            rs_d.append(out)
        red = torch.zeros(Ln, dtype=torch.int16, device=DEV)
        gpu.reduce_scatter_local(plan, rs_d, gpu.LOCAL, 1.0, red, gpu.LOCAL)
        assert_bf16(host_u16(red), want_red, f"all-reduce across instances r={r}")

        def run(fused: bool):
            master, m, v = (to_dev(x) for x in state_h)
            par = torch.full((max(N, 8),), SENTINEL, dtype=torch.int16, device=DEV)
            mg = torch.full((max(Ln, 8),), -7.0, dtype=torch.float32, device=DEV)
            if fused:
                gpu.sharded_adam_step_instances(plan, src_d, gc, scale, master, m, v, par, gpu.WORLD,
                                                main_grad_out=mg, **hp_kwargs(hp, 3))
            else:
                gpu.sharded_adam_step(plan, rs_d, gpu.LOCAL, 1.0, master, m, v, par, gpu.WORLD, main_grad_out=mg,
                                      **hp_kwargs(hp, 3))
            what = f"{'one pass' if fused else 'composed'} r={r}"
            for got, w, name in zip((master, m, v), want, ("master", "exp_avg", "exp_avg_sq")):
                assert_f32(host_f32(got), w, f"{name} {what}")
            assert_bf16(host_u16(par), want_par, f"params {what}")
            assert_f32(host_f32(mg), want_mg, f"main grad {what}")

        run(False)
        run(True)
    free()


def test_instances_one_instance_is_the_plain_step(gpu):
    """n_instances = 1 is sharded_adam_step on the D contributions."""
    rng = np.random.default_rng(77)
    sizes, bucket, D, r = [3000, 7, 9000, 515], 5000, 8, 3
    plan = gpu.build_range_map(sizes, bucket, D, r)
    reps = [to_dev(bf16_host(rng, plan.buffer_numel)) for _ in range(D)]
    Ln = plan.shard_numel
    st0 = [(rng.standard_normal(Ln) * 0.02).astype(np.float32), np.zeros(Ln, np.float32), np.zeros(Ln, np.float32)]
    hp = hp_kwargs(W.get("tiny").hp, 1)
    outs = []
    for fused in (False, True):
        st = [to_dev(x) for x in st0]
        par = torch.full((plan.buffer_numel,), SENTINEL, dtype=torch.int16, device=DEV)
        if fused:
            gpu.sharded_adam_step_instances(plan, [reps], gpu.WORLD, 0.125, *st, par, gpu.WORLD, **hp)
        else:
            gpu.sharded_adam_step(plan, reps, gpu.WORLD, 0.125, *st, par, gpu.WORLD, **hp)
        outs.append([host_f32(x) for x in st] + [host_u16(par)])
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
    # argument checks
    st = [to_dev(x) for x in st0]
    with pytest.raises(gpu.ZdoError) as e:
        gpu.sharded_adam_step_instances(plan, [], gpu.WORLD, 1.0, *st, None, gpu.WORLD, **hp)
    assert e.value.code == gpu.EINVAL
    with pytest.raises(gpu.ZdoError) as e:
        gpu.sharded_adam_step_instances(plan, [reps] * 9, gpu.WORLD, 1.0, *st, None, gpu.WORLD, **hp)  # 72 > 64
    assert e.value.code == gpu.EINVAL
    with pytest.raises(ValueError):
        gpu.sharded_adam_step_instances(plan, [reps, reps[:7]], gpu.WORLD, 1.0, *st, None, gpu.WORLD, **hp)
    free()



# ---- parameter all-gather ----------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(8))
def test_all_gather_random_layouts(gpu, seed):
    """Rank j's range of every padded bucket from params[j]: out of place into
    a fresh buffer, and in place into a rank's own buffer (whose own ranges
    are left as they are); the sources stay untouched."""
    pr = random.Random(3000 + seed)
    rng = np.random.default_rng(3000 + seed)
    sizes, bucket, D = _random_layout(pr)
    lay = OL.build_layout(sizes, bucket, D)
    N = lay.buffer_numel
    params_h = [bf16_host(rng, N, 1.0) for _ in range(D)]
    params_d = [to_dev(x) for x in params_h]
    plan = gpu.build_range_map(sizes, bucket, D, pr.randrange(D))
    out = torch.full((max(N, 8),), SENTINEL, dtype=torch.int16, device=DEV)
    gpu.all_gather_params(plan, params_d, out)
    want = np.full(max(N, 8), SENTINEL, np.uint16)
    OS.all_gather(lay, params_h, want)
    assert_bf16(host_u16(out), want, "out of place")
    for r in sorted({0, D - 1, pr.randrange(D)}):
        bufs = [to_dev(x) for x in params_h]
        gpu.all_gather_params(plan, bufs, bufs[r])
        w = params_h[r].copy()
        OS.all_gather(lay, params_h, w)
        assert_bf16(host_u16(bufs[r]), w, f"in place r={r}")
        for j in range(D):
            if j != r:
                assert_bf16(host_u16(bufs[j]), params_h[j], f"source {j} untouched")
    free()


@pytest.mark.parametrize("name", ["tiny", "frag"])
def test_zero1_loop_step_then_all_gather(gpu, name):
    """Page 1, §4.4: every rank steps its shard and writes back into its own
    copy of the parameter buffer, then every rank all-gathers in place; all
    D buffers end equal to the oracle's same loop, element for element."""
    w = W.get(name)
    lay = OL.build_layout(w.param_numel, w.bucket_numel, w.dp_size)
    N, D = lay.buffer_numel, w.dp_size
    rng = np.random.default_rng(41)
    reps_d = _gen_world(w, N)
    reps_h = [host_u16(x) for x in reps_d]
    hpk = hp_kwargs(w.hp, 2)
    hpa = ON.hp_array(w.hp, 2)
    before = bf16_host(rng, N, 0.02)
    bufs_d, bufs_h = [], []
    for r in range(D):
        plan = gpu.build_range_map(w.param_numel, w.bucket_numel, D, r)
        st = _gen_state(w, plan.shard_numel)
        st_h = [host_f32(x) for x in st]
        pb_d, pb_h = to_dev(before), before.copy()
        gpu.sharded_adam_step(plan, reps_d, gpu.WORLD, w.scale, *st, pb_d, gpu.WORLD, **hpk)
        OS.rank_step(lay, r, reps_h, OS.WORLD, w.scale, *st_h, hpa, pb_h, OS.WORLD)
        assert_bf16(host_u16(pb_d), pb_h, f"{name} r={r} write-back")
        bufs_d.append(pb_d)
        bufs_h.append(pb_h)
        del st
    want = before.copy()
    OS.all_gather(lay, bufs_h, want)
    for r in range(D):
        gpu.all_gather_params(gpu.build_range_map(w.param_numel, w.bucket_numel, D, r), bufs_d, bufs_d[r])
    for r in range(D):
        assert_bf16(host_u16(bufs_d[r]), want, f"{name} rank {r} after the all-gather")
    # argument checks
    plan = gpu.build_range_map(w.param_numel, w.bucket_numel, D, 0)
    with pytest.raises(gpu.ZdoError) as e:
        gpu.all_gather_params(plan, bufs_d[:-1], bufs_d[0])
    assert e.value.code == gpu.EINVAL
    big = torch.zeros(N + 64, dtype=torch.int16, device=DEV)
    with pytest.raises(gpu.ZdoError) as e:                               # overlaps without coinciding
        gpu.all_gather_params(plan, [big[:N]] + bufs_d[1:], big[8:8 + N])
    assert e.value.code == gpu.EALIAS
    del reps_d, bufs_d
    free()


@pytest.mark.parametrize("off_bytes,D", [(16, 4), (48, 4), (16, 32), (48, 32)])
def test_buffers_off_the_cache_line(gpu, off_bytes, D):
    """The ABI asks for 16-byte alignment only; the kernels' tiles are laid
    out for 128-byte lines. Every buffer here starts off_bytes past a line:
    reduce-scatter, the fused step (at D = 32 whole tiles take the 16-byte
    reduction), the clipped path and the all-gather stay bit-exact against
    the oracle."""
    rng = np.random.default_rng(off_bytes + D)
    if D == 4:
        sizes, bucket = [5000, 13, 20000, 1, 4097, 777], 9000
    else:
        sizes, bucket = [500000, 13, 200000, 1, 40097, 777], 300000
    lay = OL.build_layout(sizes, bucket, D)
    N = lay.buffer_numel

    def view(n, dtype, fill):
        per = off_bytes // (2 if dtype == torch.int16 else 4)
        big = torch.full((n + per + 64,), fill, dtype=dtype, device=DEV)
        v = big[per:per + n]
        assert v.data_ptr() % 128 == off_bytes
        return v

    reps_h = [bf16_host(rng, N) for _ in range(D)]
    reps_d = []
    for x in reps_h:
        v = view(N, torch.int16, 0)
        v.copy_(to_dev(x))
        reps_d.append(v)
    hp = W.get("tiny").hp
    r = 2
    plan = gpu.build_range_map(sizes, bucket, D, r)
    Ln = plan.shard_numel
    # reduce-scatter
    out = view(Ln, torch.int16, SENTINEL)
    gpu.reduce_scatter_local(plan, reps_d, gpu.WORLD, 0.25, out, gpu.LOCAL)
    want = np.full(Ln, SENTINEL, np.uint16)
    OS.reduce_scatter(lay, r, reps_h, OS.WORLD, 0.25, want, OS.LOCAL)
    assert_bf16(host_u16(out), want, "reduce-scatter")
    # fused step
    st_h = [(rng.standard_normal(Ln) * 0.02).astype(np.float32), np.zeros(Ln, np.float32),
            np.zeros(Ln, np.float32)]
    st = []
    for x in st_h:
        v = view(Ln, torch.float32, 0.0)
        v.copy_(to_dev(x))
        st.append(v)
    par = view(N, torch.int16, SENTINEL)
    mg = view(Ln, torch.float32, -7.0)
    gpu.sharded_adam_step(plan, reps_d, gpu.WORLD, 0.25, *st, par, gpu.WORLD, main_grad_out=mg, **hp_kwargs(hp, 1))
    want_st = [x.copy() for x in st_h]
    want_par = np.full(N, SENTINEL, np.uint16)
    want_mg = np.full(Ln, -7.0, np.float32)
    OS.rank_step(lay, r, reps_h, OS.WORLD, 0.25, *want_st, ON.hp_array(hp, 1), want_par, OS.WORLD, want_mg)
    for got, w_, nm in zip(st, want_st, ("master", "exp_avg", "exp_avg_sq")):
        assert_f32(host_f32(got), w_, nm)
    assert_bf16(host_u16(par), want_par, "params")
    assert_f32(host_f32(mg), want_mg, "main grad")
    # clipped path from the reduced gradient
    ws = torch.empty(plan.norm_workspace_bytes + off_bytes, dtype=torch.uint8, device=DEV)[off_bytes:]
    parts = torch.zeros(1, dtype=torch.float64, device=DEV)
    red = view(Ln, torch.int16, 0)
    gpu.grad_norm_sq(plan, reps_d, gpu.WORLD, 0.25, ws, parts, red, gpu.LOCAL)
    coeff = torch.empty(1, dtype=torch.float32, device=DEV)
    gpu.clip_coefficient(parts, 0.01, coeff)
    c = float(coeff.item())
    st2 = [view(Ln, torch.float32, 0.0) for _ in range(3)]
    for v, x in zip(st2, st_h):
        v.copy_(to_dev(x))
    gpu.sharded_adam_step_clipped(plan, [red], gpu.LOCAL, 1.0, *st2, None, gpu.WORLD, grad_coeff=coeff,
                                  **hp_kwargs(hp, 1))
    want2 = [x.copy() for x in st_h]
    OS.rank_step(lay, r, reps_h, OS.WORLD, 0.25, *want2, ON.hp_array(hp, 1), grad_coeff=c)
    for got, w_, nm in zip(st2, want2, ("master", "exp_avg", "exp_avg_sq")):
        assert_f32(host_f32(got), w_, nm + " (clipped)")
    # all-gather in place into rank r's buffer
    bufs_h = [bf16_host(rng, N) for _ in range(D)]
    bufs = []
    for x in bufs_h:
        v = view(N, torch.int16, 0)
        v.copy_(to_dev(x))
        bufs.append(v)
    gpu.all_gather_params(plan, bufs, bufs[r])
    want_g = bufs_h[r].copy()
    OS.all_gather(lay, bufs_h, want_g)
    assert_bf16(host_u16(bufs[r]), want_g, "all-gather")
    free()


@pytest.mark.parametrize("name", ["frag", "many", "d32"])
def test_bucket_lists(gpu, name):
    """Page 1, §4.2: several bucket ranges ready together go in one launch
    (sharded_adam_step_bucket_list, reduce_scatter_local_bucket_list).
    Groups of non-adjacent buckets, launched group by group in shuffled
    order, equal the full call and the oracle bit for bit; a list with more
    than 16 separate runs (two launches) too; overlapping or out-of-range
    lists are EINVAL and an empty list changes nothing. "d32": 32
    contributions, so that whole tiles take the 16-byte reduction inside
    launches of several runs."""
    if name == "frag":
        w = W.get("frag")
        sizes, bucket, D, r = w.param_numel, w.bucket_numel, w.dp_size, 5
        lay = OL.build_layout(sizes, bucket, D)
        reps_d = _gen_world(w, lay.buffer_numel)
        reps_h = [host_u16(x) for x in reps_d]
    elif name == "many":
        rng = np.random.default_rng(78)
        pr = random.Random(78)
        sizes = [pr.choice([1, 7, 300, 2048, 5000]) for _ in range(120)]
        bucket, D, r = 2000, 3, 2
        lay = OL.build_layout(sizes, bucket, D)
        reps_h = [bf16_host(rng, lay.buffer_numel) for _ in range(D)]
        reps_d = [to_dev(x) for x in reps_h]
    else:
        rng = np.random.default_rng(79)
        pr = random.Random(79)
        sizes = [pr.choice([1, 70, 3000, 9000, 40000]) for _ in range(260)]
        bucket, D, r = 60000, 32, 17
        lay = OL.build_layout(sizes, bucket, D)
        reps_h = [bf16_host(rng, lay.buffer_numel) for _ in range(D)]
        reps_d = [to_dev(x) for x in reps_h]
    plan = gpu.build_range_map(sizes, bucket, D, r)
    nb = len(lay.buckets)
    N, Ln = plan.buffer_numel, plan.shard_numel
    hp = W.get("tiny").hp
    rng = np.random.default_rng(6)
    st0 = [(rng.standard_normal(Ln) * 0.02).astype(np.float32), (rng.standard_normal(Ln) * 1e-3).astype(np.float32),
           ((rng.standard_normal(Ln) * 1e-3) ** 2).astype(np.float32)]
    scale = 1.0 / D
    want_st = [x.copy() for x in st0]
    want_par = np.full(N, SENTINEL, np.uint16)
    OS.rank_step(lay, r, reps_h, OS.WORLD, scale, *want_st, ON.hp_array(hp, 2), want_par, OS.WORLD)
    want_rs = np.full(N, SENTINEL, np.uint16)
    OS.reduce_scatter(lay, r, reps_h, OS.WORLD, scale, want_rs, OS.WORLD)

    def check(groups, what):
        st = [to_dev(x) for x in st0]
        par = torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV)
        out = torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV)
        for g in groups:
            gpu.sharded_adam_step(plan, reps_d, gpu.WORLD, scale, *st, par, gpu.WORLD, buckets=g, **hp_kwargs(hp, 2))
            gpu.reduce_scatter_local(plan, reps_d, gpu.WORLD, scale, out, gpu.WORLD, buckets=g)
        for x, wv, nm in zip(st, want_st, ("master", "exp_avg", "exp_avg_sq")):
            assert_f32(host_f32(x), wv, f"{name} {what} {nm}")
        assert_bf16(host_u16(par), want_par, f"{name} {what} params")
        assert_bf16(host_u16(out), want_rs, f"{name} {what} reduce-scatter")

    # three groups of scattered single buckets and pairs, shuffled
    pr = random.Random(9)
    order = list(range(nb))
    pr.shuffle(order)
    groups = [[(b, b + 1) for b in order[k::3]] for k in range(3)]
    pr.shuffle(groups)
    check(groups, "three scattered groups")
    # every other bucket, then the rest: more than 16 runs in one list when
    # there are more than 32 buckets
    evens = [(b, b + 1) for b in range(0, nb, 2)]
    odds = [(b, b + 1) for b in range(1, nb, 2)][::-1]
    if name != "frag":
        assert len(evens) > 16
    check([evens, odds], "alternate buckets")
    # one list covering everything (touching ranges merge into one run)
    check([[(b, b + 1) for b in reversed(range(nb))]], "all buckets, touching")
    # errors and the empty list
    st = [to_dev(x) for x in st0]
    par = torch.full((N,), SENTINEL, dtype=torch.int16, device=DEV)
    for bad in ([(0, 2), (1, 3)], [(0, nb + 1)], [(2, 1)], [(-1, 1)]):
        with pytest.raises(gpu.ZdoError) as e:
            gpu.sharded_adam_step(plan, reps_d, gpu.WORLD, scale, *st, par, gpu.WORLD, buckets=bad,
                                  **hp_kwargs(hp, 2))
        assert e.value.code == gpu.EINVAL
        with pytest.raises(gpu.ZdoError) as e:
            gpu.reduce_scatter_local(plan, reps_d, gpu.WORLD, scale, par, gpu.WORLD, buckets=bad)
        assert e.value.code == gpu.EINVAL
    gpu.sharded_adam_step(plan, reps_d, gpu.WORLD, scale, *st, par, gpu.WORLD, buckets=[], **hp_kwargs(hp, 2))
    gpu.sharded_adam_step(plan, reps_d, gpu.WORLD, scale, *st, par, gpu.WORLD, buckets=[(3, 3)], **hp_kwargs(hp, 2))
    assert all(np.array_equal(host_f32(x).view(np.uint32), y.view(np.uint32)) for x, y in zip(st, st0))
    assert (host_u16(par) == SENTINEL).all()
    del reps_d
    free()


@pytest.mark.parametrize("seed", range(3))
def test_d32_whole_tiles_and_edges(gpu, seed):
    """32 contributions: whole tiles take the 16-byte reduction with the
    cross-lane move to the quads; tiles at a segment's ends take the quads
    one at a time, partial quads slot by slot. Layouts whose buckets start
    and end off every 64-element line, so that both paths and the seams
    between them run in every rank's segments; all ranks are compared with
    the oracle, WORLD and LOCAL coordinates."""
    pr = random.Random(4400 + seed)
    rng = np.random.default_rng(4400 + seed)
    D = 32
    sizes = []
    while sum(sizes) < 32 * 9000:
        sizes.append(pr.choice([pr.randint(1, 70), pr.randint(500, 3000), pr.randint(20000, 90000)]))
    bucket = pr.randint(sum(sizes) // 6, sum(sizes) // 3)
    lay = OL.build_layout(sizes, bucket, D)
    N = lay.buffer_numel
    assert all(any(OL.rank_range(b, D, r).start % 64 for b in lay.buckets) for r in (1, D - 1))
    reps_h = [bf16_host(rng, N, pr.choice([1e-3, 1.0])) for _ in range(D)]
    hp = W.get("tiny").hp
    for r in sorted({0, 1, pr.randrange(D), D - 1}):
        Ln = OL.shard_numel(lay, r)
        state = [(rng.standard_normal(Ln) * 0.02).astype(np.float32),
                 (rng.standard_normal(Ln) * 1e-3).astype(np.float32),
                 ((rng.standard_normal(Ln) * 1e-3) ** 2).astype(np.float32)]
        c = gpu.WORLD if r % 2 else gpu.LOCAL
        run_rank_step(gpu, sizes, bucket, D, r, reps_h, state, 1.0 / D, hp, 5, c, gpu.LOCAL if r % 2 else gpu.WORLD)
    free()
