"""Pins of the oracle's element arithmetic (oracle/step.c):
  * bf16 rounding against torch's own fp32 -> bf16 conversion (library routine);
  * the reduction against the worked AllReduce example of the distributed
    training notes (section "AllReduce") and against exact rational sums;
  * scaling before the reduction (page "04 · 分布式优化器", §5) as an
    observable order;
  * Adam against closed forms at step 1 and against torch.optim.AdamW;
  * the global-norm clipping of the distributed-training notes (§8.3) against
    exact integer sums and torch.nn.utils.clip_grad_norm_.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle.numerics as N
import oracle.step as S
import oracle.layout as L

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def torch_widen(h: np.ndarray) -> np.ndarray:
    return torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).float().numpy()


def is_nan_bf16(h):
    return ((h & 0x7F80) == 0x7F80) & ((h & 0x7F) != 0)


# ---- bf16 ---------------------------------------------------------------------

def test_narrow_matches_torch_structured():
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000], dtype=np.uint32)
    bits = (hi[:, None] | lows[None, :]).ravel()
    x = bits.view(np.float32)
    got, want = N.narrow(x), torch_bf16_bits(x)
    nan = np.isnan(x)
    assert np.array_equal(is_nan_bf16(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_narrow_matches_torch_random():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    got, want = N.narrow(x), torch_bf16_bits(x)
    nan = np.isnan(x)
    assert np.array_equal(is_nan_bf16(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_widen_exact():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got, want = N.widen(h), torch_widen(h)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def test_narrow_special_values():
    f = np.float32

    def b(u):
        return np.array([u], np.uint32).view(np.float32)[0]

    cases = [
        (f(65504.0), 0x4780),                 # fp16 max is not a bf16: rounds to 65536
        (f(-65504.0), 0xC780),
        (f(3.0e38), 0x7F62),
        (b(0x7F7FFFFF), 0x7F80),              # largest float rounds to +Inf
        (f(np.inf), 0x7F80), (f(-np.inf), 0xFF80),
        (f(0.0), 0x0000), (f(-0.0), 0x8000),
        (b(0x00000001), 0x0000),              # tiny subnormal -> +0
        (b(0x00008000), 0x0000),              # tie, to even (0)
        (b(0x00018000), 0x0002),              # tie, to even (2)
        (b(0x00010001), 0x0001),              # bf16 subnormal kept
        (f(1.0 + 2**-8), 0x3F80),             # halfway, to even
        (f(1.0 + 3 * 2**-8), 0x3F82),         # halfway, to even (up)
    ]
    x = np.array([c[0] for c in cases], dtype=np.float32)
    assert [int(v) for v in N.narrow(x)] == [c[1] for c in cases]
    nan = np.array([0x7F800001, 0xFFFFFFFF, 0x7FC00000], np.uint32).view(np.float32)
    assert is_nan_bf16(N.narrow(nan)).all()


# ---- reduction -------------------------------------------------------------------

def _golden_allreduce():
    rows = []
    with open(os.path.join(GOLDEN, "allreduce_example.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                tag, *vals = line.split()
                rows.append((tag, [float(v) for v in vals]))
    ranks = [v for t, v in rows if t == "rank"]
    total = [v for t, v in rows if t == "sum"][0]
    return ranks, total


def test_allreduce_worked_example():
    ranks, total = _golden_allreduce()
    reps = [torch_bf16_bits(np.array(r, np.float32)) for r in ranks]
    got = N.widen(S.all_reduce(reps, 1.0))
    assert got.tolist() == total
    # the same through the layout: one 2-element parameter at D=3 is padded to 3
    lay = L.build_layout([2], 10, 3)
    assert lay.buffer_numel == 3
    padded = [np.concatenate([r, np.zeros(1, np.uint16)]) for r in reps]
    out = np.full(3, 0xFFFF, np.uint16)
    for r in range(3):
        S.reduce_scatter(lay, r, padded, S.WORLD, 1.0, out, S.WORLD)
    assert N.widen(out).tolist() == total + [0.0]


def test_single_contribution_is_identity():
    rng = np.random.default_rng(3)
    h = rng.integers(0, 1 << 16, size=200_000, dtype=np.uint32).astype(np.uint16)
    got = S.all_reduce([h], 1.0)
    nan = is_nan_bf16(h)
    assert np.array_equal(is_nan_bf16(got), nan)
    assert np.array_equal(got[~nan], h[~nan])


def _exact(h):
    return Fraction(float(torch_widen(np.array([h], np.uint16))[0]))


def _fits_f32(x: Fraction) -> bool:
    d = float(x)
    return Fraction(d) == x and math.isfinite(d) and float(np.float32(d)) == d


def _rational_check(reps_f32, scale, got, expect_all_checked=False):
    """Where every partial sum of the scaled bf16 terms is a float32, the fp32
    running sum is exact, so the oracle must equal bf16(exact sum)."""
    D = len(reps_f32)
    terms = [torch_bf16_bits((torch.from_numpy(r) * torch.tensor(scale, dtype=torch.float32)).numpy())
             for r in [torch_widen(torch_bf16_bits(r)) for r in reps_f32]]
    n = reps_f32[0].size
    checked = 0
    for i in range(n):
        acc = Fraction(0)
        ok = True
        for j in range(D):
            acc += _exact(terms[j][i])
            if not _fits_f32(acc):
                ok = False
                break
        if not ok:
            continue
        checked += 1
        want = torch_bf16_bits(np.array([float(acc)], np.float32))[0]
        assert got[i] == want, (i, float(acc))
    if expect_all_checked:
        assert checked == n
    return checked


@pytest.mark.parametrize("D,scale", [(2, 1.0), (3, 0.5), (4, 0.25), (8, 0.125), (16, 1.0), (32, 1 / 32)])
def test_reduce_equals_exact_sum(D, scale):
    rng = np.random.default_rng(100 + D)
    n = 3000
    reps_f32 = [(rng.standard_normal(n) * 1e-2).astype(np.float32) for _ in range(D)]
    reps = [torch_bf16_bits(r) for r in reps_f32]
    got = S.all_reduce(reps, scale)
    checked = _rational_check(reps_f32, scale, got)
    assert checked > 0.9 * n


def test_reduce_small_integers_exact():
    rng = np.random.default_rng(11)
    D, n = 32, 5000
    reps_f32 = [rng.integers(-100, 100, size=n).astype(np.float32) for _ in range(D)]
    got = S.all_reduce([torch_bf16_bits(r) for r in reps_f32], 1.0)
    want = np.sum(np.stack(reps_f32).astype(np.int64), axis=0).astype(np.float32)
    # sums of 32 integers below 100 stay below 3200 < 2^24: exact, then one bf16 rounding
    assert np.array_equal(got, torch_bf16_bits(want))


def test_reduce_order_is_fixed_rank_order():
    # 2^24 + 1 + 1 in fp32: left to right loses both ones, the reverse keeps them
    big = torch_bf16_bits(np.array([2.0**24], np.float32))
    one = torch_bf16_bits(np.array([1.0], np.float32))
    got = N.widen(S.all_reduce([big, one, one], 1.0))[0]
    assert got == 2.0**24
    got_rev = N.widen(S.all_reduce([one, one, big], 1.0))[0]
    assert got_rev == 2.0**24   # 2^24 + 2 -> bf16 rounds to 2^24 as well
    # the running sum starts from rank 0's term, so -0 + -0 stays -0
    nz = np.array([0x8000], np.uint16)
    assert S.all_reduce([nz, nz, nz], 1.0)[0] == 0x8000
    # cancellation shows the order: 2^25 - 2^25 + 1 = 1 in rank order, while
    # any order that adds the 1 to a +-2^25 first loses it to rounding
    vals = [2.0**25, -2.0**25, 1.0]
    reps = [torch_bf16_bits(np.array([x], np.float32)) for x in vals]
    assert N.widen(S.all_reduce(reps, 1.0))[0] == 1.0
    assert N.widen(S.all_reduce(reps[::-1], 1.0))[0] == 0.0
    assert N.widen(S.all_reduce([reps[0], reps[2], reps[1]], 1.0))[0] == 0.0


def test_scale_applied_before_reduce():
    # page 1, §5: the scaling factor multiplies the buffer before the collective;
    # with a scale that is not a power of two the order is observable
    rng = np.random.default_rng(5)
    D, n = 8, 4000
    scale = float(np.float32(1.0 / 3.0))
    reps_f32 = [(rng.standard_normal(n) * 1e-2).astype(np.float32) for _ in range(D)]
    reps = [torch_bf16_bits(r) for r in reps_f32]
    got = S.all_reduce(reps, scale)
    assert _rational_check(reps_f32, scale, got) > 0.5 * n
    sum_then_scale = []
    for i in range(n):
        tot = sum(_exact(reps[j][i]) for j in range(D)) * Fraction(scale)
        sum_then_scale.append(float(tot))
    sum_then_scale = torch_bf16_bits(np.array(sum_then_scale, np.float32))
    assert (sum_then_scale != got).sum() > 0.02 * n
    # with a power-of-two scale both orders agree wherever the sum is exact
    got2 = S.all_reduce(reps, 0.125)
    plain = S.all_reduce(reps, 1.0)
    same = N.narrow(N.widen(plain) * np.float32(0.125))
    assert np.array_equal(got2, same)


# ---- Adam -------------------------------------------------------------------------

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def test_bias_correction():
    for beta in (0.9, 0.999, 0.95, 0.5):
        b = float(np.float32(beta))
        for t in (1, 2, 3, 10, 100, 1000):
            got = N.bias_correction(beta, t)
            want = float(np.float32(1.0 - b**t))
            assert abs(got - want) <= float(np.spacing(np.float32(want))), (beta, t)
    # at t = 1, 1 - b1 is exact in fp32 (Sterbenz) and both forms agree
    assert N.bias_correction(0.9, 1) == float(np.float32(1.0) - np.float32(0.9))


def test_adam_step1_closed_form():
    rng = np.random.default_rng(21)
    n = 100_000
    g = torch_bf16_bits((rng.standard_normal(n) * 1e-2).astype(np.float32))
    g[:4] = torch_bf16_bits(np.array([0.0, -0.0, 1e-30, -3.0], np.float32))
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    p, m, v = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    hp = N.hp_array(HP, 1)
    N.adam(g, p, m, v, hp)
    gf = N.widen(g).astype(np.float64)
    b1, b2 = np.float32(HP["beta1"]), np.float32(HP["beta2"])
    # m' = (1-b1) g and v' = (1-b2) g^2 (each a single rounding of an exact product)
    assert np.array_equal(m, (np.float32(1) - b1) * N.widen(g))
    assert np.array_equal(v, (np.float32(1) - b2) * (N.widen(g) * N.widen(g)))
    # p' = p - lr (g / (|g| + eps) + wd p), to a few ulp of the update
    upd = HP["lr"] * (gf / (np.abs(gf) + HP["eps"]) + HP["weight_decay"] * p0.astype(np.float64))
    want = p0.astype(np.float64) - upd
    err = np.abs(p.astype(np.float64) - want)
    tol = np.spacing(np.abs(p)).astype(np.float64) + 8 * np.spacing(np.abs(upd).astype(np.float32)).astype(np.float64)
    assert (err <= tol).all()
    # g = 0: only the decay acts; sign of the step follows sign of g
    assert p[0] == np.float32(p0[0] - np.float32(HP["lr"]) * (np.float32(HP["weight_decay"]) * p0[0]))
    big = np.abs(gf) > 1e-4
    assert np.all(np.sign(p0[big] - p[big] - HP["lr"] * HP["weight_decay"] * p0[big]) == np.sign(gf[big]))


def test_adam_special_cases():
    rng = np.random.default_rng(22)
    n = 10_000
    g = torch_bf16_bits((rng.standard_normal(n) * 1e-2).astype(np.float32))
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m0 = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v0 = ((rng.standard_normal(n) * 1e-3) ** 2).astype(np.float32)
    # lr = 0: parameters unchanged, moments still move
    p, m, v = p0.copy(), m0.copy(), v0.copy()
    N.adam(g, p, m, v, N.hp_array(dict(HP, lr=0.0), 3))
    assert np.array_equal(p, p0) and not np.array_equal(m, m0)
    # beta1 = beta2 = 0 at t = 1: m' = g, v' = g^2, update = g / (|g| + eps)
    p = p0.copy(); m = m0.copy(); v = v0.copy()
    N.adam(g, p, m, v, N.hp_array(dict(HP, beta1=0.0, beta2=0.0, weight_decay=0.0), 1))
    gw = N.widen(g)
    assert np.array_equal(m, gw) and np.array_equal(v, gw * gw)
    want = p0.astype(np.float64) - 1e-3 * gw / (np.abs(gw).astype(np.float64) + 1e-8)
    assert np.allclose(p, want, rtol=1e-6, atol=1e-9)
    # NaN / Inf in the gradient propagate into master (no found-inf skip)
    g2 = g.copy()
    g2[:3] = torch_bf16_bits(np.array([np.nan, np.inf, -np.inf], np.float32))
    p = p0.copy(); m = m0.copy(); v = v0.copy()
    N.adam(g2, p, m, v, N.hp_array(HP, 2))
    assert np.isnan(p[:3]).all() and np.isfinite(p[3:]).all()


def test_adam_matches_torch_adamw():
    """Ten steps against torch.optim.AdamW (CPU, fp32, single-tensor form): the
    same update in another rounding order."""
    rng = np.random.default_rng(23)
    n = 50_000
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    p, m, v = p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    tp = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    # the step's hyper-parameters are fp32 values; hand torch the same values
    f = {k: float(np.float32(x)) for k, x in HP.items()}
    opt = torch.optim.AdamW([tp], lr=f["lr"], betas=(f["beta1"], f["beta2"]), eps=f["eps"],
                            weight_decay=f["weight_decay"], foreach=False, fused=False)
    for t in range(1, 11):
        g = torch_bf16_bits((rng.standard_normal(n) * 1e-2).astype(np.float32))
        N.adam(g, p, m, v, N.hp_array(HP, t))
        tp.grad = torch.from_numpy(N.widen(g))
        opt.step()
        st = opt.state[tp]
        # near p = 0 the two rounding orders differ by a few ulp of the update
        # (lr * |u| <= ~1e-3, ulp ~ 1e-10) per step, accumulated over t steps
        np.testing.assert_allclose(p, tp.detach().numpy(), rtol=1e-6, atol=5e-10 * t)
        # m' and v' are sums of two terms; where they cancel, two rounding orders
        # differ by a few ulp of the terms (|m| ~ 1e-3, |v| ~ 1e-7), not of the sum
        np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-5, atol=1e-9)
        np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-5, atol=1e-13)


def test_step_is_reduce_then_adam():
    rng = np.random.default_rng(24)
    D, n = 5, 20_000
    reps = [torch_bf16_bits((rng.standard_normal(n) * 1e-2).astype(np.float32)) for _ in range(D)]
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m0 = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v0 = ((rng.standard_normal(n) * 1e-3) ** 2).astype(np.float32)
    hp = N.hp_array(HP, 4)
    a = [p0.copy(), m0.copy(), v0.copy()]
    pa, mga = np.zeros(n, np.uint16), np.zeros(n, np.float32)
    N.step(reps, 0.2, *a, hp, pa, mga)
    red = N.reduce(reps, 0.2)
    b = [p0.copy(), m0.copy(), v0.copy()]
    pb = np.zeros(n, np.uint16)
    N.adam(red, *b, hp, pb)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    assert np.array_equal(pa, pb)
    assert np.array_equal(mga, N.widen(red))
    assert np.array_equal(pa, torch_bf16_bits(a[0]))


# ---- global-norm clipping ----------------------------------------------------------------

def test_norm_sq_exact_on_integers():
    # squares of integers below 2^8, summed: exact in fp64, so any order agrees
    rng = np.random.default_rng(31)
    D, n = 4, 20_000
    ints = [rng.integers(-60, 60, size=n) for _ in range(D)]
    reps = [torch_bf16_bits(x.astype(np.float32)) for x in ints]
    total = np.sum(np.stack(ints), axis=0)                # |sum| < 240: exact in bf16
    want = float(np.sum(total.astype(np.int64) ** 2))
    assert N.norm_sq(reps, 1.0) == want
    # the scale applies to each term before the sum (page 1, §5): scale 1/2 -> (sum/2)^2
    assert N.norm_sq(reps, 0.5) == float(np.sum((total.astype(np.float64) / 2) ** 2))


def test_clip_coefficient_matches_torch():
    """The coefficient, applied to a gradient, gives torch.nn.utils.clip_grad_norm_'s
    clipped gradient (fp32) to within a few ulp."""
    rng = np.random.default_rng(32)
    for max_norm in (0.05, 0.5, 1.0, 10.0, 1e4):
        shards = [(rng.standard_normal(4000) * 1e-2).astype(np.float32) for _ in range(4)]
        parts = [float(np.sum(x.astype(np.float64) ** 2)) for x in shards]
        coeff, norm = N.clip_coefficient(parts, max_norm)
        assert abs(norm - np.sqrt(sum(parts))) <= 1e-12 * norm
        ps = [torch.nn.Parameter(torch.zeros(4000)) for _ in range(4)]
        for p, x in zip(ps, shards):
            p.grad = torch.from_numpy(x.copy())
        total = torch.nn.utils.clip_grad_norm_(ps, max_norm, norm_type=2.0, foreach=False)
        assert abs(float(total) - norm) <= 1e-6 * norm
        for p, x in zip(ps, shards):
            mine = x * np.float32(coeff)
            np.testing.assert_allclose(mine, p.grad.numpy(), rtol=4e-7, atol=1e-12)


def test_clip_coefficient_special_cases():
    # below the threshold nothing is clipped
    assert N.clip_coefficient([0.25, 0.0], 1.0)[0] == 1.0
    assert N.clip_coefficient([0.0], 1.0)[0] == 1.0
    # above it the clipped norm is max_norm: coefficient * norm == max_norm (up to the 1e-6)
    c, norm = N.clip_coefficient([16.0, 9.0], 1.0)
    assert norm == 5.0 and abs(c * 5.0 - 1.0) < 1e-6
    # a norm that is not finite is found-inf: NaN coefficient, the step is skipped
    assert np.isnan(N.clip_coefficient([1.0, np.inf], 1.0)[0])
    assert np.isnan(N.clip_coefficient([np.nan, 1.0], 1.0)[0])
    # parts are summed in index order
    big, tiny = 2.0**60, 1.0
    assert N.clip_coefficient([big, tiny, -big], 1.0)[1] == 0.0
    assert N.clip_coefficient([big, -big, tiny], 1.0)[1] == 1.0


def test_clipped_step():
    rng = np.random.default_rng(33)
    D, n = 4, 10_000
    reps = [torch_bf16_bits((rng.standard_normal(n) * 1e-2).astype(np.float32)) for _ in range(D)]
    p0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m0 = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    v0 = ((rng.standard_normal(n) * 1e-3) ** 2).astype(np.float32)
    hp = N.hp_array(HP, 5)
    # coefficient 1 is the unclipped step, bit for bit
    a = [p0.copy(), m0.copy(), v0.copy()]
    b = [p0.copy(), m0.copy(), v0.copy()]
    N.step(reps, 0.25, *a, hp)
    N.step(reps, 0.25, *b, hp, grad_coeff=1.0)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    # a coefficient c is Adam on the main grad multiplied by c (one fp32 product)
    c = float(np.float32(0.3721))
    mg = np.zeros(n, np.float32)
    st = [p0.copy(), m0.copy(), v0.copy()]
    N.step(reps, 0.25, *st, hp, main_grad_out=mg, grad_coeff=c)
    red = N.reduce(reps, 0.25)
    assert np.array_equal(mg, N.widen(red) * np.float32(c))
    ref = [p0.copy(), m0.copy(), v0.copy()]
    N.adam(red, *ref, hp)
    assert not np.array_equal(ref[1], st[1])
    # closed form at step 1 from zero state: the moments see the clipped grad g'
    z = [p0.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)]
    g1 = np.zeros(n, np.float32)
    N.step(reps, 0.25, *z, N.hp_array(HP, 1), main_grad_out=g1, grad_coeff=c)
    b1, b2 = np.float32(HP["beta1"]), np.float32(HP["beta2"])
    assert np.array_equal(z[1], (np.float32(1) - b1) * g1)
    assert np.array_equal(z[2], (np.float32(1) - b2) * (g1 * g1))
    # a NaN coefficient (found-inf) through the rank composition changes nothing
    lay = L.build_layout([3000, 7000], 4000, D)
    st2 = [S.gather_shard(lay, 1, x) for x in (np.resize(p0, lay.buffer_numel),) * 3]
    before = [x.copy() for x in st2]
    par = np.full(lay.buffer_numel, 0x7FBF, np.uint16)
    full = [np.resize(r, lay.buffer_numel) for r in reps]
    S.rank_step(lay, 1, full, S.WORLD, 0.25, *st2, hp, par, S.WORLD, grad_coeff=float("nan"))
    for x, y in zip(st2, before):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    assert (par == 0x7FBF).all()
