"""Pins of the oracle's rank-level composition (oracle.step) against what the
pages fix about sharding:
  * page "04 · 分布式优化器", §2/§3: each rank updates only its range and the
    ranks together cover the buffer, so the union of the D rank steps must
    equal the unsharded step, bit for bit (the page "Megatron-LM 与 ZeRO",
    section "最小语义 reference", checks sharding the same way: every shard
    stepped on the CPU one after another, then compared with the dense
    update);
  * §5: force_all_reduce yields the full reduced buffer, whose restriction
    to rank r's range is rank r's reduce-scatter;
  * §4.3: the write-back touches the owned range only.
"""

import random

import numpy as np
import pytest
import torch

import oracle.layout as L
import oracle.numerics as N
import oracle.step as S
import workloads as W

HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def make_inputs(lay, rng, sigma=1e-2, zero_padding=True):
    Nn = lay.buffer_numel
    D = lay.dp_size
    grads = [bf16(rng.standard_normal(Nn) * sigma) for _ in range(D)]
    if zero_padding:
        owned = np.zeros(Nn, bool)
        for r in lay.param_world:
            owned[r.start:r.end] = True
        for g in grads:
            g[~owned] = 0
    master = (rng.standard_normal(Nn) * 0.02).astype(np.float32)
    m = (rng.standard_normal(Nn) * 1e-3).astype(np.float32)
    v = ((rng.standard_normal(Nn) * 1e-3) ** 2).astype(np.float32)
    return grads, master, m, v


def sharded_vs_unsharded(lay, grads, master, m, v, scale, t, grad_coords=S.WORLD, param_coords=S.WORLD):
    hp = N.hp_array(HP, t)
    Nn = lay.buffer_numel
    # unsharded
    mw, mm, vv = master.copy(), m.copy(), v.copy()
    pw = np.full(Nn, 0x7FBF, np.uint16)
    S.unsharded_step(lay, grads, scale, mw, mm, vv, hp, pw)
    # sharded, rank by rank
    ms, ms_m, ms_v = master.copy(), m.copy(), v.copy()
    ps = np.full(Nn, 0x7FBF, np.uint16)
    for r in range(lay.dp_size):
        sm = S.gather_shard(lay, r, ms)
        sm_m = S.gather_shard(lay, r, ms_m)
        sm_v = S.gather_shard(lay, r, ms_v)
        reps = grads if grad_coords == S.WORLD else [S.local_slices(lay, r, g) for g in grads]
        if param_coords == S.WORLD:
            S.rank_step(lay, r, reps, grad_coords, scale, sm, sm_m, sm_v, hp, ps, S.WORLD)
        else:
            pl = np.full(L.shard_numel(lay, r), 0x7FBF, np.uint16)
            S.rank_step(lay, r, reps, grad_coords, scale, sm, sm_m, sm_v, hp, pl, S.LOCAL)
            S.scatter_shard(lay, r, pl, ps)
        S.scatter_shard(lay, r, sm, ms)
        S.scatter_shard(lay, r, sm_m, ms_m)
        S.scatter_shard(lay, r, sm_v, ms_v)
    for a, b in ((mw, ms), (mm, ms_m), (vv, ms_v)):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(pw, ps)
    return ms, ms_m, ms_v, ps


def test_tiny_ten_steps_union_equals_unsharded():
    w = W.get("tiny")
    lay = L.build_layout(w.param_numel, w.bucket_numel, w.dp_size)
    rng = np.random.default_rng(1)
    _, master, m, v = make_inputs(lay, rng)
    m[:] = 0
    v[:] = 0
    for t in range(1, 11):
        grads = [bf16(rng.standard_normal(1000) * w.grad_sigma) for _ in range(4)]
        master, m, v, params = sharded_vs_unsharded(lay, grads, master, m, v, w.scale, t)
    assert np.array_equal(params, bf16(master))


@pytest.mark.parametrize("seed", range(12))
def test_random_layouts_union_equals_unsharded(seed):
    rng = np.random.default_rng(seed)
    pr = random.Random(seed)
    sizes = [pr.randint(1, 300) for _ in range(pr.randint(1, 25))]
    D = pr.choice([1, 2, 3, 4, 5, 8, 16])
    lay = L.build_layout(sizes, pr.randint(1, 1500), D)
    grads, master, m, v = make_inputs(lay, rng)
    scale = pr.choice([1.0, 0.5, 1.0 / D, 1.0 / 3.0])
    gc = pr.choice([S.WORLD, S.LOCAL])
    pc = pr.choice([S.WORLD, S.LOCAL])
    sharded_vs_unsharded(lay, grads, master, m, v, scale, pr.randint(1, 50), gc, pc)


def test_split_parameter_is_updated_as_one():
    # the Tiny workload's second parameter is cut 130 / 170 between ranks 0 and 1
    w = W.get("tiny")
    lay = L.build_layout(w.param_numel, w.bucket_numel, w.dp_size)
    rng = np.random.default_rng(2)
    grads, master, m, v = make_inputs(lay, rng)
    ms, _, _, _ = sharded_vs_unsharded(lay, grads, master, m, v, 0.25, 1)
    whole_m, whole_mm, whole_v = master[120:420].copy(), m[120:420].copy(), v[120:420].copy()
    N.step([g[120:420] for g in grads], 0.25, whole_m, whole_mm, whole_v, N.hp_array(HP, 1))
    assert np.array_equal(ms[120:420], whole_m)


def test_all_reduce_restricted_is_reduce_scatter():
    pr = random.Random(9)
    rng = np.random.default_rng(9)
    for _ in range(10):
        sizes = [pr.randint(1, 200) for _ in range(pr.randint(1, 20))]
        D = pr.choice([2, 3, 4, 7, 16])
        lay = L.build_layout(sizes, pr.randint(1, 800), D)
        grads = [bf16(rng.standard_normal(lay.buffer_numel)) for _ in range(D)]
        full = S.all_reduce(grads, 0.5)
        union = np.full(lay.buffer_numel, 0xFFFF, np.uint16)
        for r in range(D):
            out_w = np.full(lay.buffer_numel, 0xFFFF, np.uint16)
            S.reduce_scatter(lay, r, grads, S.WORLD, 0.5, out_w, S.WORLD)
            mine = np.zeros(lay.buffer_numel, bool)
            for rg, _ in L.rank_ranges(lay, r):
                mine[rg.start:rg.end] = True
            assert np.array_equal(out_w[mine], full[mine])
            assert (out_w[~mine] == 0xFFFF).all()
            union[mine] = out_w[mine]
            # LOCAL coordinates hold the same values at the shard positions
            out_l = np.full(L.shard_numel(lay, r), 0xFFFF, np.uint16)
            S.reduce_scatter(lay, r, grads, S.WORLD, 0.5, out_l, S.LOCAL)
            assert np.array_equal(out_l, S.local_slices(lay, r, out_w, fill=0xFFFF))
        assert np.array_equal(union, full)


def test_fused_equals_reduce_then_prereduced_step():
    # reduce-scatter first, then the step with the one pre-reduced contribution and scale 1
    w = W.get("tiny")
    lay = L.build_layout([7, 33, 64, 5, 91], 100, 4)
    rng = np.random.default_rng(4)
    grads, master, m, v = make_inputs(lay, rng)
    hp = N.hp_array(HP, 3)
    for r in range(4):
        a = [S.gather_shard(lay, r, x) for x in (master, m, v)]
        b = [x.copy() for x in a]
        pa = np.zeros(lay.buffer_numel, np.uint16)
        pb = np.zeros(lay.buffer_numel, np.uint16)
        S.rank_step(lay, r, grads, S.WORLD, 0.25, *a, hp, pa, S.WORLD)
        red = np.zeros(lay.buffer_numel, np.uint16)
        S.reduce_scatter(lay, r, grads, S.WORLD, 0.25, red, S.WORLD)
        S.rank_step(lay, r, [red], S.WORLD, 1.0, *b, hp, pb, S.WORLD)
        for x, y in zip(a, b):
            assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
        assert np.array_equal(pa, pb)
    del w


def test_writeback_touches_owned_range_only():
    lay = L.build_layout([13, 300, 2, 77], 150, 4)    # two buckets, padding in each
    rng = np.random.default_rng(5)
    grads, master, m, v = make_inputs(lay, rng)
    hp = N.hp_array(HP, 1)
    owned_any = np.zeros(lay.buffer_numel, bool)
    for r in range(4):
        p = np.full(lay.buffer_numel, 0x7FBF, np.uint16)
        sm = [S.gather_shard(lay, r, x) for x in (master, m, v)]
        S.rank_step(lay, r, grads, S.WORLD, 0.25, *sm, hp, p, S.WORLD)
        mine = np.zeros(lay.buffer_numel, bool)
        for pc in L.rank_pieces(lay, r):
            mine[pc.gbuf_world.start:pc.gbuf_world.end] = True
        assert (p[~mine] == 0x7FBF).all()
        assert (p[mine] != 0x7FBF).all()
        owned_any |= mine
        # writeback of the updated master gives the same bytes
        q = np.full(lay.buffer_numel, 0x7FBF, np.uint16)
        S.writeback(lay, r, sm[0], q, S.WORLD)
        assert np.array_equal(p, q)
    # every parameter element is owned by someone; padding by no one
    params = np.zeros(lay.buffer_numel, bool)
    for rg in lay.param_world:
        params[rg.start:rg.end] = True
    assert np.array_equal(owned_any, params)


def test_resume_is_bit_exact():
    w = W.get("tiny")
    lay = L.build_layout(w.param_numel, w.bucket_numel, w.dp_size)
    rng = np.random.default_rng(6)
    steps = [[bf16(rng.standard_normal(1000) * 1e-2) for _ in range(4)] for _ in range(10)]
    master0 = (rng.standard_normal(1000) * 0.02).astype(np.float32)
    for r in range(4):
        st = [S.gather_shard(lay, r, master0), np.zeros(252, np.float32), np.zeros(252, np.float32)]
        st = [np.resize(x, L.shard_numel(lay, r)) for x in st]
        a = [x.copy() for x in st]
        for t in range(1, 11):
            S.rank_step(lay, r, steps[t - 1], S.WORLD, 0.25, *a, N.hp_array(HP, t))
        b = [x.copy() for x in st]
        for t in range(1, 6):
            S.rank_step(lay, r, steps[t - 1], S.WORLD, 0.25, *b, N.hp_array(HP, t))
        saved = [x.tobytes() for x in b]
        b = [np.frombuffer(s, np.float32).copy() for s in saved]
        for t in range(6, 11):
            S.rank_step(lay, r, steps[t - 1], S.WORLD, 0.25, *b, N.hp_array(HP, t))
        for x, y in zip(a, b):
            assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


def test_segmentation_invariance():
    # per-piece calls and one call per contiguous owned run give the same bytes
    lay = L.build_layout([5, 17, 1, 1, 40, 3, 260, 9], 64, 4)
    rng = np.random.default_rng(8)
    grads, master, m, v = make_inputs(lay, rng)
    hp = N.hp_array(HP, 2)
    for r in range(4):
        a = [S.gather_shard(lay, r, x) for x in (master, m, v)]
        b = [x.copy() for x in a]
        pa = np.zeros(lay.buffer_numel, np.uint16)
        pb = np.zeros(lay.buffer_numel, np.uint16)
        S.rank_step(lay, r, grads, S.WORLD, 0.25, *a, hp, pa, S.WORLD)
        runs = []
        for pc in L.rank_pieces(lay, r):
            if runs and runs[-1][1] == pc.gbuf_world.start:
                runs[-1][1] = pc.gbuf_world.end
            else:
                runs.append([pc.gbuf_world.start, pc.gbuf_world.end, pc.shard_offset])
        for ws, we, k0 in runs:
            k1 = k0 + we - ws
            N.step([g[ws:we] for g in grads], 0.25, b[0][k0:k1], b[1][k0:k1], b[2][k0:k1], hp, pb[ws:we])
        for x, y in zip(a, b):
            assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
        assert np.array_equal(pa, pb)


def test_bucket_ranges_compose_to_the_full_step():
    # page 1, §2/§4.2: buckets are handled one at a time as they become ready;
    # the per-bucket steps over a partition of the buckets, in any order, are the full step
    lay = L.build_layout([300, 5, 70, 1000, 2, 640, 33], 350, 4)
    assert len(lay.buckets) >= 4
    rng = np.random.default_rng(12)
    grads, master, m, v = make_inputs(lay, rng)
    hp = N.hp_array(HP, 2)
    nb = len(lay.buckets)
    for r in range(4):
        full = [S.gather_shard(lay, r, x) for x in (master, m, v)]
        pf = np.full(lay.buffer_numel, 0x7FBF, np.uint16)
        S.rank_step(lay, r, grads, S.WORLD, 0.25, *full, hp, pf, S.WORLD)
        parts = [S.gather_shard(lay, r, x) for x in (master, m, v)]
        pp = np.full(lay.buffer_numel, 0x7FBF, np.uint16)
        for b in reversed(range(nb)):
            S.rank_step(lay, r, grads, S.WORLD, 0.25, *parts, hp, pp, S.WORLD, buckets=(b, b + 1))
        for x, y in zip(full, parts):
            assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
        assert np.array_equal(pf, pp)
        rf = np.full(lay.buffer_numel, 0xFFFF, np.uint16)
        S.reduce_scatter(lay, r, grads, S.WORLD, 0.25, rf, S.WORLD)
        rp = np.full(lay.buffer_numel, 0xFFFF, np.uint16)
        S.reduce_scatter(lay, r, grads, S.WORLD, 0.25, rp, S.WORLD, buckets=(nb // 2, nb))
        S.reduce_scatter(lay, r, grads, S.WORLD, 0.25, rp, S.WORLD, buckets=(0, nb // 2))
        assert np.array_equal(rf, rp)


def test_two_level_reduction_of_instances():
    """Page 1, §5: with several distributed-optimizer instances, the
    reduce-scatter runs within each instance and an all-reduce across the
    instances follows. Reading: each instance's bf16 reduce-scatter result,
    summed over instances in instance order (fp32, one rounding)."""
    D, n_inst = 4, 3
    lay = L.build_layout([700, 9, 1300, 64], 900, D)
    rng = np.random.default_rng(13)
    reps = [[bf16(rng.standard_normal(lay.buffer_numel) * 1e-2) for _ in range(D)] for _ in range(n_inst)]
    hp = N.hp_array(HP, 1)
    for r in range(D):
        rs = []
        for i in range(n_inst):
            out = np.zeros(L.shard_numel(lay, r), np.uint16)
            S.reduce_scatter(lay, r, reps[i], S.WORLD, 0.125, out, S.LOCAL)
            rs.append(out)
        # the all-reduce across instances over the rank's range
        red = np.zeros(L.shard_numel(lay, r), np.uint16)
        S.reduce_scatter(lay, r, rs, S.LOCAL, 1.0, red, S.LOCAL)
        # element by element, bf16(sum_i bf16(sum_j bf16(s g_ij))) evaluated
        # again with numpy float32 operations, apart from the C arithmetic
        for pc in L.rank_pieces(lay, r)[:3]:
            for e in range(0, pc.gbuf_world.size, 37):
                w_ = pc.gbuf_world.start + e
                k = pc.shard_offset + e
                total = 0.0
                for i in range(n_inst):
                    inner = np.float32(0.0)
                    for j in range(D):
                        t = N.widen(N.narrow(np.array([N.widen(reps[i][j][w_:w_ + 1])[0] * np.float32(0.125)],
                                                      np.float32)))[0]
                        inner = np.float32(inner + t) if j else t
                    total = np.float32(total + N.widen(N.narrow(np.array([inner], np.float32)))[0]) if i else \
                        N.widen(N.narrow(np.array([inner], np.float32)))[0]
                assert red[k] == N.narrow(np.array([total], np.float32))[0]
        # one instance: the two levels are the plain reduce-scatter
        one = np.zeros(L.shard_numel(lay, r), np.uint16)
        S.reduce_scatter(lay, r, [rs[0]], S.LOCAL, 1.0, one, S.LOCAL)
        assert np.array_equal(one, rs[0])
        # the step on the instances' results (n contributions, scale 1) is the
        # step on the two-level reduced gradient
        a = [S.gather_shard(lay, r, x) for x in (np.zeros(lay.buffer_numel, np.float32),) * 3]
        b = [x.copy() for x in a]
        S.rank_step(lay, r, rs, S.LOCAL, 1.0, *a, hp)
        S.rank_step(lay, r, [red], S.LOCAL, 1.0, *b, hp)
        for x, y in zip(a, b):
            assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    # two levels differ from one flat sum over all D * n_inst contributions on some elements
    flat = S.all_reduce([x for inst in reps for x in inst], 0.125)
    two = [S.all_reduce(inst, 0.125) for inst in reps]
    assert (S.all_reduce(two, 1.0) != flat).any()


@pytest.mark.parametrize("seed", range(8))
def test_all_gather_closes_the_zero1_loop(seed):
    """Page 1, §4.4: reduce-scatter of the grads, the sharded step, then the
    all-gather of the parameters closes the ZeRO-1 loop: every rank writes
    back into its own copy of the parameter buffer, and the all-gather of
    those D buffers equals the unsharded step's parameters at every element
    (padding keeps the buffer's prior contents), in a fresh buffer and in
    place into any rank's buffer."""
    rng = np.random.default_rng(500 + seed)
    pr = random.Random(500 + seed)
    sizes = [pr.randint(1, 400) for _ in range(pr.randint(1, 25))]
    D = pr.choice([1, 2, 3, 4, 5, 8, 16])
    lay = L.build_layout(sizes, pr.randint(1, 2000), D)
    Nn = lay.buffer_numel
    grads, master, m, v = make_inputs(lay, rng)
    scale = pr.choice([1.0, 1.0 / D])
    hp = N.hp_array(HP, pr.randint(1, 20))
    before = bf16(master)
    before[rng.random(Nn) < 0.1] = 0x7FBF          # prior contents, padding included
    want = before.copy()
    S.unsharded_step(lay, grads, scale, master.copy(), m.copy(), v.copy(), hp, want)
    bufs = []
    for r in range(D):
        pb = before.copy()
        S.rank_step(lay, r, grads, S.WORLD, scale, S.gather_shard(lay, r, master), S.gather_shard(lay, r, m),
                    S.gather_shard(lay, r, v), hp, pb, S.WORLD)
        bufs.append(pb)
    if D > 1 and sum(1 for b in bufs if not np.array_equal(b, want)) < 2:
        pytest.skip("layout where at most one rank owns elements")
    out = np.full(Nn, 0x1234, np.uint16)
    S.all_gather(lay, bufs, out)
    assert np.array_equal(out, want)
    k = pr.randrange(D)
    S.all_gather(lay, bufs, bufs[k])
    assert np.array_equal(bufs[k], want)


# ---- the rank's squared gradient norm (distributed-training notes, §8.3) -------------------------

def _owner_scan(lay, D):
    """For every element of the padded buffer: the rank that owns it and
    whether a parameter sits there, found element by element from the
    bucket table (page 1, §3: rank r holds the r-th of D equal ranges of a
    padded bucket), without the range map."""
    Nn = lay.buffer_numel
    owner = np.full(Nn, -1, np.int64)
    is_param = np.zeros(Nn, bool)
    for b in lay.buckets:
        S_b = b.padded_numel // D
        for w in range(b.offset, b.offset + b.padded_numel):
            owner[w] = (w - b.offset) // S_b
            is_param[w] = w < b.offset + b.numel
    return owner, is_param


@pytest.mark.parametrize("seed", range(4))
def test_rank_norm_sq_exact_and_summing_to_the_global_norm(seed):
    """rank_norm_sq against an exact sum. Gradients are small integers (exact
    in bf16) and the scale a power of two, so every reduced value and every
    square is exact and the fp64 total is exact in any order. Padding holds
    large non-zero values, so counting a padding element would change the
    total. Checked in WORLD and LOCAL coordinates on multi-bucket padded
    layouts, and the ranks' parts add up to the squared norm of the
    all-reduced buffer over the parameter elements (padding excluded)."""
    rng = np.random.default_rng(900 + seed)
    D = int(rng.integers(2, 7))
    sizes = [int(x) for x in rng.integers(1, 90, size=int(rng.integers(4, 12)))]
    bucket = int(rng.integers(15, max(16, sum(sizes) // 3)))
    lay = L.build_layout(sizes, bucket, D)
    assert len(lay.buckets) > 1
    assert any(b.padded_numel > b.numel for b in lay.buckets)
    Nn = lay.buffer_numel
    owner, is_param = _owner_scan(lay, D)
    ints = [rng.integers(-8, 9, size=Nn) for _ in range(D)]
    for g in ints:
        g[~is_param] = 1000                 # padding: large, never counted
    grads = [bf16(g.astype(np.float32)) for g in ints]
    scale = 0.5
    total_int = np.sum(ints, axis=0)        # exact integer sums
    sq = (total_int.astype(np.float64) * scale) ** 2
    global_sq = 0.0
    for r in range(D):
        want = float(np.sum(sq[(owner == r) & is_param]))
        got_w = S.rank_norm_sq(lay, r, grads, S.WORLD, scale)
        assert got_w == want, f"rank {r} WORLD: {got_w} != {want}"
        loc = [S.local_slices(lay, r, g, fill=0x4000) for g in grads]   # 2.0 in the gap slots
        got_l = S.rank_norm_sq(lay, r, loc, S.LOCAL, scale)
        assert got_l == want, f"rank {r} LOCAL: {got_l} != {want}"
        global_sq += got_w
    red = N.widen(S.all_reduce(grads, scale)).astype(np.float64)
    assert global_sq == float(np.sum(red[is_param] ** 2))
    assert global_sq == float(np.sum(sq[is_param]))


@pytest.mark.parametrize("name", ["tiny", "gpt2_small", "llama3_8b", "llama3_70b", "frag"])
def test_rank_state_is_the_zero1_share(name):
    """Page "Megatron-LM 与 ZeRO" (its per-stage memory accounting): ZeRO
    stage 1 keeps the bf16 weights and gradients whole on every rank (2 + 2
    bytes per element) and gives each rank a 1/D share of the 12 bytes of
    fp32 Adam state; stages 2 and 3 shard the gradients, then the weights
    too, so a rank's bytes fall from stage 0 to stage 3. The ranks' owned
    elements count every parameter element once, and each rank's fp32 shard
    (its range of every padded bucket plus alignment gaps of fewer than 64
    slots) comes within 12 x 64 bytes per bucket of the stage-1 share
    12 N / D of the padded buffer."""
    w = W.get(name)
    lay = L.build_layout(w.param_numel, w.bucket_numel, w.dp_size)
    D, N, nb = w.dp_size, lay.buffer_numel, len(lay.buckets)
    assert sum(L.owned_numel(lay, r) for r in range(D)) == sum(w.param_numel)

    def rank_bytes(stage):
        per_element = {"weights": 2, "grads": 2, "adam": 12}
        sharded = {0: (), 1: ("adam",), 2: ("grads", "adam"), 3: ("weights", "grads", "adam")}[stage]
        return N * sum(b / D if part in sharded else b for part, b in per_element.items())

    stages = [rank_bytes(s) for s in range(4)]
    if D > 1:
        assert stages[3] < stages[2] < stages[1] < stages[0]
    for r in range(D):
        shard = L.shard_numel(lay, r)
        assert N // D <= shard < N // D + 64 * nb
        ours = 2 * N + 2 * N + 12 * shard     # whole bf16 parameter and grad buffers, the fp32 shard
        assert stages[1] <= ours < stages[1] + 12 * 64 * nb
