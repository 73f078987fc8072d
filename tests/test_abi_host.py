"""Host-side tests of the C-ABI (no GPU needed, no kernel launched): the
library loads and exports every symbol include/zdo.h declares, the plan's
layout and four-way range map equal the oracle's bit for bit, and bad
arguments come back as error codes."""

import ctypes
import os
import random
import re

import numpy as np
import pytest

import oracle.layout as OL
import workloads as W
import zero_distributed_optimizer_amd as Z

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "zdo.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    L = Z.require_library()
    names = header_functions()
    assert len(names) == 32, names
    assert sorted(Z.EXPORTS) == names
    for n in names:
        assert hasattr(L, n), n
    # the binding names the five calls of the method exactly
    for n in ("build_range_map", "reduce_scatter_local", "force_all_reduce", "sharded_adam_step",
              "writeback_params"):
        assert callable(getattr(Z, n))


def test_short_plan_names_equal_the_prefixed_ones():
    """plan_buckets, plan_pieces, plan_buffer_numel, plan_shard_numel and
    plan_destroy answer exactly as their zdo_plan_ twins (host-only plan)."""
    L = Z.require_library()
    w = W.get("frag")
    sizes = np.ascontiguousarray(np.asarray(w.param_numel[:3000], dtype=np.int64))
    h = ctypes.c_void_p()
    rc = L.build_range_map(sizes.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), int(sizes.size),
                           400_000, 16, 5, ctypes.byref(h))
    assert rc == 0
    try:
        assert L.plan_buffer_numel(h) == L.zdo_plan_buffer_numel(h) > 0
        assert L.plan_shard_numel(h) == L.zdo_plan_shard_numel(h) > 0
        for short, long_, dt, ct in ((L.plan_buckets, L.zdo_plan_buckets, Z.BUCKET_DTYPE, ctypes.c_int32),
                                     (L.plan_pieces, L.zdo_plan_pieces, Z.PIECE_DTYPE, ctypes.c_int64)):
            n1, n2 = ct(), ct()
            assert short(h, None, 0, ctypes.byref(n1)) == 0 == long_(h, None, 0, ctypes.byref(n2))
            assert n1.value == n2.value > 0
            a, b = np.zeros(n1.value, dt), np.zeros(n2.value, dt)
            assert short(h, a.ctypes.data, n1.value, ctypes.byref(n1)) == 0
            assert long_(h, b.ctypes.data, n2.value, ctypes.byref(n2)) == 0
            assert a.tobytes() == b.tobytes()
        assert L.plan_buckets(None, None, 0, ctypes.byref(ctypes.c_int32())) == Z.EINVAL
        assert L.plan_buffer_numel(None) == -1 and L.plan_shard_numel(None) == -1
    finally:
        L.plan_destroy(h)
    L.plan_destroy(None)


def test_no_alloc_norm_refuses_a_plan_beyond_its_scratch_before_anything_else():
    """A rank whose norm needs more than the static scratch array
    (ZDO_NO_ALLOC_SCRATCH_BYTES) is refused with EINVAL by the size check,
    which comes before every device check: the replica list is NULL here, so
    any other order would answer with a different message."""
    L = Z.require_library()
    sizes = np.array([(1 << 32) + (1 << 20)], dtype=np.int64)      # 2^32 + 2^20 elements, D = 1
    h = ctypes.c_void_p()
    assert L.build_range_map(sizes.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), 1, 1 << 40, 1, 0,
                             ctypes.byref(h)) == 0
    try:
        need = L.zdo_plan_norm_workspace_bytes(h)
        assert need > Z.NO_ALLOC_SCRATCH_BYTES
        out = ctypes.c_double()
        rc = L.grad_norm_sq_no_alloc(h, None, 1, Z.LOCAL, 1.0, None, Z.LOCAL, ctypes.byref(out), None)
        assert rc == Z.EINVAL
        assert b"scratch" in L.zdo_last_error()
        assert L.grad_norm_sq_no_alloc(None, None, 1, Z.LOCAL, 1.0, None, Z.LOCAL, None, None) == Z.EINVAL
    finally:
        L.zdo_plan_destroy(h)


def test_struct_layouts():
    assert ctypes.sizeof(Z.Piece) == 80 == Z.PIECE_DTYPE.itemsize
    assert ctypes.sizeof(Z.Bucket) == 40 == Z.BUCKET_DTYPE.itemsize
    assert ctypes.sizeof(Z.Adam) == 32


def oracle_tuples(lay, rank):
    return [pc.as_tuple() for pc in OL.rank_pieces(lay, rank)]


def plan_tuples(plan):
    out = []
    for p in plan.pieces():
        out.append((int(p["param_index"]), int(p["bucket_index"]), *map(int, p["gbuf_world"]),
                    *map(int, p["gbuf_world_in_bucket"]), *map(int, p["gbuf_local"]), *map(int, p["param"]),
                    int(p["shard_offset"])))
    return out


def compare(sizes, bucket_numel, D, rank):
    lay = OL.build_layout(sizes, bucket_numel, D)
    plan = Z.build_range_map(sizes, bucket_numel, D, rank)
    try:
        assert plan.buffer_numel == lay.buffer_numel
        assert plan.shard_numel == OL.shard_numel(lay, rank)
        assert plan.owned_numel == OL.owned_numel(lay, rank)
        assert plan_tuples(plan) == oracle_tuples(lay, rank)
        bases, _ = OL.shard_bases(lay, rank)
        want = [(b.offset, b.numel, b.padded_numel, b.shard_numel(D), base) for b, base in zip(lay.buckets, bases)]
        got = [tuple(int(x) for x in b) for b in plan.buckets()]
        assert got == want
    finally:
        plan.destroy()


@pytest.mark.parametrize("name", ["tiny", "gpt2_small", "llama3_8b", "llama3_70b", "frag"])
def test_range_map_matches_oracle(name):
    w = W.get(name)
    ranks = range(w.dp_size) if w.dp_size <= 16 else sorted({0, 1, w.dp_size // 2, w.dp_size - 1})
    for r in ranks:
        compare(w.param_numel, w.bucket_numel, w.dp_size, r)


def test_range_map_random_layouts():
    rng = random.Random(77)
    for _ in range(400):
        sizes = [rng.choice([rng.randint(1, 9), rng.randint(1, 300), rng.randint(1, 5000)])
                 for _ in range(rng.randint(1, 30))]
        D = rng.choice([1, 2, 3, 4, 5, 7, 8, 16, 32, 64])
        bucket = rng.randint(1, 20000)
        compare(sizes, bucket, D, rng.randrange(D))


@pytest.mark.parametrize("args,code", [
    (([], 10, 2, 0), Z.EINVAL),
    (([5, 0], 10, 2, 0), Z.EINVAL),
    (([5, -1], 10, 2, 0), Z.EINVAL),
    (([5], 0, 2, 0), Z.EINVAL),
    (([5], 10, 0, 0), Z.EINVAL),
    (([5], 10, 65, 0), Z.EINVAL),
    (([5], 10, 4, 4), Z.EINVAL),
    (([5], 10, 4, -1), Z.EINVAL),
])
def test_build_errors(args, code):
    with pytest.raises(Z.ZdoError) as e:
        Z.build_range_map(*args)
    assert e.value.code == code
    assert str(e.value)


def test_launch_on_host_only_plan_is_an_error():
    # without a device the plan carries no device table: every launch call
    # reports EHIP before it touches any pointer
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    L = Z.require_library()
    plan = Z.build_range_map([10, 20], 16, 2, 0)
    reps = (ctypes.c_void_p * 2)(16, 32)
    hp = Z.adam_hparams(1e-3, 0.9, 0.999, 1e-8, 0.0, 1)
    assert L.reduce_scatter_local(plan.handle, reps, 2, 0, 1.0, 48, 0, None) == Z.EHIP
    assert L.force_all_reduce(plan.handle, reps, 2, 1.0, 48, None) == Z.EHIP
    assert L.sharded_adam_step(plan.handle, reps, 2, 0, 1.0, 64, 80, 96, None, 0, ctypes.byref(hp), None,
                               None) == Z.EHIP
    assert L.writeback_params(plan.handle, 64, 48, 0, None) == Z.EHIP
    assert L.grad_norm_sq(plan.handle, reps, 2, 0, 1.0, None, 0, 64, 128, None) == Z.EHIP
    assert L.reduce_scatter_local_buckets(plan.handle, 0, 1, reps, 2, 0, 1.0, 48, 0, None) == Z.EHIP
    assert L.sharded_adam_step_buckets(plan.handle, 0, 1, reps, 2, 0, 1.0, 64, 80, 96, None, 0, ctypes.byref(hp),
                                       None, None) == Z.EHIP
    assert L.sharded_adam_step_clipped(plan.handle, reps, 2, 0, 1.0, 64, 80, 96, None, 0, ctypes.byref(hp), 112,
                                       None, None) == Z.EHIP
    assert L.sharded_adam_step_instances(plan.handle, reps, 1, 0, 1.0, 64, 80, 96, None, 0, ctypes.byref(hp), None,
                                         None) == Z.EHIP
    assert L.all_gather_params(plan.handle, reps, 2, 48, None) == Z.EHIP
    assert b"device" in L.zdo_last_error()
    assert L.zdo_plan_norm_workspace_bytes(plan.handle) >= 8
    assert L.clip_coefficient(None, 1, 1.0, 64, None, None) == Z.EINVAL
    assert L.clip_coefficient(64, 0, 1.0, 128, None, None) == Z.EINVAL
    assert L.clip_coefficient(68, 1, 1.0, 128, None, None) == Z.EALIGN
    assert L.clip_coefficient(64, 2, 1.0, 72, None, None) == Z.EALIAS
    assert L.zdo_device_copy(16, 48, 15, None) == Z.EINVAL
    assert L.zdo_device_copy(16, 40, 16, None) == Z.EALIGN
    assert L.zdo_device_copy(16, 32, 32, None) == Z.EALIAS
    assert L.reduce_scatter_local(None, reps, 2, 0, 1.0, 48, 0, None) == Z.EINVAL


def test_plan_accessors_on_null():
    L = Z.require_library()
    assert L.zdo_plan_buffer_numel(None) == -1
    assert L.zdo_plan_shard_numel(None) == -1
    n = ctypes.c_int64()
    assert L.zdo_plan_pieces(None, None, 0, ctypes.byref(n)) == Z.EINVAL
    L.zdo_plan_destroy(None)


def test_buffers_reject_host_tensors_and_wrong_dtypes():
    """zdo.Buffers checks its tensors once, as every call checks a list."""
    import torch
    import zero_distributed_optimizer_amd as zdo
    with pytest.raises(ValueError, match="device"):
        zdo.Buffers([torch.zeros(8, dtype=torch.int16)], "replicas")
    with pytest.raises(TypeError, match="torch tensor"):
        zdo.Buffers([np.zeros(8, np.int16)], "replicas")
    empty = zdo.Buffers([], "replicas")
    assert len(empty) == 0 and empty.numel == 0
