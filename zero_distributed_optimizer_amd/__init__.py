"""Python binding of libzdo: one DP rank's share of a distributed-optimizer
(ZeRO-1) step on an AMD Instinct MI355X.

The functions mirror the C-ABI of include/zdo.h one to one and only marshal
arguments: torch tensors in, device pointers and the current HIP stream out.
Every step of the work runs in the library's HIP kernels. If the library is
missing or cannot be loaded, every call raises; nothing falls back to another
implementation.

    plan = build_range_map(param_numel, bucket_numel, dp_size, rank)
    sharded_adam_step(plan, replicas, WORLD, scale, master, exp_avg, exp_avg_sq,
                      param_buffer, WORLD, lr=..., beta1=..., ..., step=t)
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

WORLD = 0
LOCAL = 1
MAX_REPLICAS = 64
# zdo_stream_probe's store modes (include/zdo.h)
PROBE_STORE_ALL, PROBE_STORE_OUT, PROBE_STORE_NONE = 0, 1, 2

OK, EINVAL, EALIGN, EALIAS, EHIP, ENOMEM = 0, -1, -2, -3, -4, -5
_CODES = {EINVAL: "EINVAL", EALIGN: "EALIGN", EALIAS: "EALIAS", EHIP: "EHIP", ENOMEM: "ENOMEM"}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libzdo.so")


class ZdoError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{_CODES.get(code, code)}: {message}")
        self.code = code


class Range(ctypes.Structure):
    _fields_ = [("start", ctypes.c_int64), ("end", ctypes.c_int64)]


class Piece(ctypes.Structure):
    _fields_ = [("param_index", ctypes.c_int32), ("bucket_index", ctypes.c_int32),
                ("gbuf_world", Range), ("gbuf_world_in_bucket", Range), ("gbuf_local", Range),
                ("param", Range), ("shard_offset", ctypes.c_int64)]


class Bucket(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_int64), ("numel", ctypes.c_int64), ("padded_numel", ctypes.c_int64),
                ("shard_numel", ctypes.c_int64), ("shard_base", ctypes.c_int64)]


class Adam(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("reserved", ctypes.c_int32),
                ("step", ctypes.c_int64)]


PIECE_DTYPE = np.dtype([("param_index", "<i4"), ("bucket_index", "<i4"),
                        ("gbuf_world", "<i8", 2), ("gbuf_world_in_bucket", "<i8", 2),
                        ("gbuf_local", "<i8", 2), ("param", "<i8", 2), ("shard_offset", "<i8")])
BUCKET_DTYPE = np.dtype([("offset", "<i8"), ("numel", "<i8"), ("padded_numel", "<i8"),
                         ("shard_numel", "<i8"), ("shard_base", "<i8")])

# Every symbol include/zdo.h declares.
EXPORTS = ("build_range_map", "zdo_plan_destroy", "zdo_plan_buffer_numel", "zdo_plan_shard_numel",
           "zdo_plan_owned_numel", "zdo_plan_dp_size", "zdo_plan_rank", "zdo_plan_buckets",
           "zdo_plan_pieces", "reduce_scatter_local", "force_all_reduce", "sharded_adam_step",
           "writeback_params", "reduce_scatter_local_buckets", "sharded_adam_step_buckets",
           "zdo_plan_norm_workspace_bytes", "grad_norm_sq", "clip_coefficient", "sharded_adam_step_clipped",
           "sharded_adam_step_instances", "all_gather_params", "zdo_device_copy", "zdo_last_error",
           "plan_buckets", "plan_pieces", "plan_buffer_numel", "plan_shard_numel", "plan_destroy",
           "grad_norm_sq_no_alloc", "reduce_scatter_local_bucket_list", "sharded_adam_step_bucket_list",
           "zdo_stream_probe")
NO_ALLOC_SCRATCH_BYTES = 64 << 20

_lib = None


def require_library() -> ctypes.CDLL:
    """Load libzdo.so (built by zero_distributed_optimizer_amd.build); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libzdo.so not found at {LIB_PATH}; build it with "
                          "`python -m zero_distributed_optimizer_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, f32, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
    L.build_range_map.argtypes = [ctypes.POINTER(i64), i32, i64, i32, i32, ctypes.POINTER(vp)]
    L.zdo_plan_destroy.argtypes = [vp]
    L.zdo_plan_destroy.restype = None
    for f in ("zdo_plan_buffer_numel", "zdo_plan_shard_numel", "zdo_plan_owned_numel"):
        getattr(L, f).argtypes = [vp]
        getattr(L, f).restype = i64
    for f in ("zdo_plan_dp_size", "zdo_plan_rank"):
        getattr(L, f).argtypes = [vp]
        getattr(L, f).restype = i32
    L.zdo_plan_buckets.argtypes = [vp, vp, i32, ctypes.POINTER(i32)]
    L.zdo_plan_pieces.argtypes = [vp, vp, i64, ctypes.POINTER(i64)]
    L.plan_buckets.argtypes = [vp, vp, i32, ctypes.POINTER(i32)]
    L.plan_pieces.argtypes = [vp, vp, i64, ctypes.POINTER(i64)]
    for f in ("plan_buffer_numel", "plan_shard_numel"):
        getattr(L, f).argtypes = [vp]
        getattr(L, f).restype = i64
    L.plan_destroy.argtypes = [vp]
    L.plan_destroy.restype = None
    L.reduce_scatter_local.argtypes = [vp, vp, i32, i32, f32, vp, i32, vp]
    L.force_all_reduce.argtypes = [vp, vp, i32, f32, vp, vp]
    L.sharded_adam_step.argtypes = [vp, vp, i32, i32, f32, vp, vp, vp, vp, i32, ctypes.POINTER(Adam), vp, vp]
    L.writeback_params.argtypes = [vp, vp, vp, i32, vp]
    L.reduce_scatter_local_buckets.argtypes = [vp, i32, i32, vp, i32, i32, f32, vp, i32, vp]
    L.reduce_scatter_local_bucket_list.argtypes = [vp, vp, i32, vp, i32, i32, f32, vp, i32, vp]
    L.sharded_adam_step_bucket_list.argtypes = [vp, vp, i32, vp, i32, i32, f32, vp, vp, vp, vp, i32,
                                                ctypes.POINTER(Adam), vp, vp]
    L.sharded_adam_step_buckets.argtypes = [vp, i32, i32, vp, i32, i32, f32, vp, vp, vp, vp, i32,
                                            ctypes.POINTER(Adam), vp, vp]
    L.zdo_plan_norm_workspace_bytes.argtypes = [vp]
    L.zdo_plan_norm_workspace_bytes.restype = i64
    L.grad_norm_sq.argtypes = [vp, vp, i32, i32, f32, vp, i32, vp, vp, vp]
    L.grad_norm_sq_no_alloc.argtypes = [vp, vp, i32, i32, f32, vp, i32, vp, vp]
    L.clip_coefficient.argtypes = [vp, i32, f32, vp, vp, vp]
    L.sharded_adam_step_clipped.argtypes = [vp, vp, i32, i32, f32, vp, vp, vp, vp, i32, ctypes.POINTER(Adam),
                                            vp, vp, vp]
    L.sharded_adam_step_instances.argtypes = [vp, vp, i32, i32, f32, vp, vp, vp, vp, i32, ctypes.POINTER(Adam), vp,
                                              vp]
    L.all_gather_params.argtypes = [vp, vp, i32, vp, vp]
    L.zdo_device_copy.argtypes = [vp, vp, i64, vp]
    L.zdo_stream_probe.argtypes = [vp, i32, vp, vp, vp, vp, i64, i32, i32, vp]
    L.zdo_last_error.argtypes = []
    L.zdo_last_error.restype = ctypes.c_char_p
    for f in ("build_range_map", "zdo_plan_buckets", "zdo_plan_pieces", "plan_buckets", "plan_pieces",
              "reduce_scatter_local",
              "force_all_reduce", "sharded_adam_step", "writeback_params", "grad_norm_sq", "grad_norm_sq_no_alloc",
              "clip_coefficient",
              "sharded_adam_step_clipped", "reduce_scatter_local_buckets", "sharded_adam_step_buckets",
              "sharded_adam_step_instances", "all_gather_params", "zdo_device_copy",
              "reduce_scatter_local_bucket_list", "sharded_adam_step_bucket_list", "zdo_stream_probe"):
        getattr(L, f).restype = ctypes.c_int
    _lib = L
    return L


class use_library:
    """Within the block, every call goes to the libzdo build at `path` (for
    example one compiled with different launch caps); the previous library
    is restored on exit. Plans made inside belong to that build and must be
    destroyed inside the block."""

    def __init__(self, path: str):
        self.path = os.path.abspath(path)

    def __enter__(self):
        global _lib, LIB_PATH
        self._saved = (_lib, LIB_PATH)
        _lib, LIB_PATH = None, self.path
        return require_library()

    def __exit__(self, *exc):
        global _lib, LIB_PATH
        _lib, LIB_PATH = self._saved
        return False


def _check(rc: int) -> None:
    if rc != OK:
        raise ZdoError(rc, require_library().zdo_last_error().decode(errors="replace"))


class Plan:
    """A rank's layout and range map (owns the library's zdo_plan)."""

    def __init__(self, param_numel, bucket_numel: int, dp_size: int, rank: int):
        L = require_library()
        sizes = np.ascontiguousarray(np.asarray(param_numel, dtype=np.int64))
        h = ctypes.c_void_p()
        _check(L.build_range_map(sizes.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), int(sizes.size),
                                 int(bucket_numel), int(dp_size), int(rank), ctypes.byref(h)))
        self._h = h
        self.dp_size = int(L.zdo_plan_dp_size(h))
        self.rank = int(L.zdo_plan_rank(h))
        self.buffer_numel = int(L.zdo_plan_buffer_numel(h))
        self.shard_numel = int(L.zdo_plan_shard_numel(h))
        self.owned_numel = int(L.zdo_plan_owned_numel(h))

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._h is None:
            raise ValueError("plan destroyed")
        return self._h

    def buckets(self) -> np.ndarray:
        L = require_library()
        n = ctypes.c_int32()
        _check(L.zdo_plan_buckets(self.handle, None, 0, ctypes.byref(n)))
        out = np.zeros(n.value, dtype=BUCKET_DTYPE)
        _check(L.zdo_plan_buckets(self.handle, out.ctypes.data, n.value, ctypes.byref(n)))
        return out

    def pieces(self) -> np.ndarray:
        L = require_library()
        n = ctypes.c_int64()
        _check(L.zdo_plan_pieces(self.handle, None, 0, ctypes.byref(n)))
        out = np.zeros(n.value, dtype=PIECE_DTYPE)
        _check(L.zdo_plan_pieces(self.handle, out.ctypes.data, n.value, ctypes.byref(n)))
        return out

    @property
    def norm_workspace_bytes(self) -> int:
        return int(require_library().zdo_plan_norm_workspace_bytes(self.handle))

    def extent(self, coords: int) -> int:
        return self.buffer_numel if coords == WORLD else self.shard_numel

    def destroy(self) -> None:
        if getattr(self, "_h", None) is not None:
            require_library().zdo_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def build_range_map(param_numel, bucket_numel: int, dp_size: int, rank: int) -> Plan:
    return Plan(param_numel, bucket_numel, dp_size, rank)


# ---- marshalling -------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dev_ptr(t, what: str, kind: str, numel: int | None) -> int:
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{what}: must be a device (cuda) tensor")
    ok = {"bf16": (torch.bfloat16, torch.int16, torch.uint16), "f32": (torch.float32,),
          "f64": (torch.float64,), "bytes": (torch.uint8, torch.int8)}[kind]
    if t.dtype not in ok:
        raise TypeError(f"{what}: dtype {t.dtype} is not {kind}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: must be contiguous")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{what}: needs at least {numel} elements, has {t.numel()}")
    return t.data_ptr()


class Buffers:
    """bf16 device buffers (the D contributions, or the ranks' parameter
    buffers) checked and marshalled once, for calls repeated on the same
    tensors: pass it wherever a call takes a list of them. Checking D
    tensors costs a few microseconds of Python each; a bucket-by-bucket step
    pays that on every launch otherwise. It holds references to the tensors,
    which must keep their storage (no resize) while it is in use."""

    def __init__(self, tensors, what: str = "buffers"):
        self.tensors = tuple(tensors)
        self.array = (ctypes.c_void_p * len(self.tensors))(
            *[_dev_ptr(t, f"{what}[{j}]", "bf16", None) for j, t in enumerate(self.tensors)])
        self.numel = min((int(t.numel()) for t in self.tensors), default=0)

    def __len__(self) -> int:
        return len(self.tensors)

    def __iter__(self):
        return iter(self.tensors)

    def __getitem__(self, j):
        return self.tensors[j]


def _ptr_list(ts, what: str, numel: int):
    if isinstance(ts, Buffers):
        if ts.numel < numel:
            raise ValueError(f"{what}: needs at least {numel} elements per buffer, has {ts.numel}")
        return ts.array
    arr = (ctypes.c_void_p * len(ts))()
    for j, t in enumerate(ts):
        arr[j] = _dev_ptr(t, f"{what}[{j}]", "bf16", numel)
    return arr


def _stream(stream, device) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _bucket_list(buckets):
    """A list of (begin, end) pairs as the C-ABI's int32 pair array, or None
    for a single (begin, end) pair."""
    if len(buckets) == 2 and all(isinstance(b, (int, np.integer)) for b in buckets):
        return None
    arr = np.ascontiguousarray(np.asarray([[int(b), int(e)] for b, e in buckets], dtype=np.int32).reshape(-1))
    return arr


def reduce_scatter_local(plan: Plan, replicas, replica_coords: int, scale: float, out, out_coords: int,
                         stream=None, buckets=None) -> None:
    """buckets=(begin, end): only those buckets (reduce_scatter_local_buckets);
    buckets=[(begin, end), ...]: those ranges in one launch
    (reduce_scatter_local_bucket_list)."""
    reps = _ptr_list(replicas, "replicas", plan.extent(replica_coords))
    o = _dev_ptr(out, "out", "bf16", plan.extent(out_coords))
    L, st = require_library(), _stream(stream, out.device)
    if buckets is None:
        _check(L.reduce_scatter_local(plan.handle, reps, len(replicas), replica_coords, scale, o, out_coords, st))
        return
    lst = _bucket_list(buckets)
    if lst is None:
        _check(L.reduce_scatter_local_buckets(plan.handle, int(buckets[0]), int(buckets[1]), reps, len(replicas),
                                              replica_coords, scale, o, out_coords, st))
    else:
        _check(L.reduce_scatter_local_bucket_list(plan.handle, lst.ctypes.data, lst.size // 2, reps, len(replicas),
                                                  replica_coords, scale, o, out_coords, st))


def force_all_reduce(plan: Plan, replicas, scale: float, out_full, stream=None) -> None:
    reps = _ptr_list(replicas, "replicas", plan.buffer_numel)
    o = _dev_ptr(out_full, "out_full", "bf16", plan.buffer_numel)
    _check(require_library().force_all_reduce(plan.handle, reps, len(replicas), scale, o,
                                              _stream(stream, out_full.device)))


def adam_hparams(lr: float, beta1: float, beta2: float, eps: float, weight_decay: float, step: int) -> Adam:
    return Adam(lr, beta1, beta2, eps, weight_decay, 0, step)


def sharded_adam_step(plan: Plan, grads, grad_coords: int, scale: float, master, exp_avg, exp_avg_sq,
                      param_out=None, param_coords: int = WORLD, *, lr: float, beta1: float, beta2: float,
                      eps: float, weight_decay: float, step: int, main_grad_out=None, stream=None,
                      buckets=None) -> None:
    """buckets=(begin, end): only those buckets (sharded_adam_step_buckets);
    buckets=[(begin, end), ...]: those ranges in one launch
    (sharded_adam_step_bucket_list)."""
    L = plan.shard_numel
    g = _ptr_list(grads, "grads", plan.extent(grad_coords))
    m = _dev_ptr(master, "master", "f32", L)
    a = _dev_ptr(exp_avg, "exp_avg", "f32", L)
    s = _dev_ptr(exp_avg_sq, "exp_avg_sq", "f32", L)
    p = None if param_out is None else _dev_ptr(param_out, "param_out", "bf16", plan.extent(param_coords))
    mg = None if main_grad_out is None else _dev_ptr(main_grad_out, "main_grad_out", "f32", L)
    hp = adam_hparams(lr, beta1, beta2, eps, weight_decay, step)
    L, st = require_library(), _stream(stream, master.device)
    if buckets is None:
        _check(L.sharded_adam_step(plan.handle, g, len(grads), grad_coords, scale, m, a, s, p, param_coords,
                                   ctypes.byref(hp), mg, st))
        return
    lst = _bucket_list(buckets)
    if lst is None:
        _check(L.sharded_adam_step_buckets(plan.handle, int(buckets[0]), int(buckets[1]), g, len(grads),
                                           grad_coords, scale, m, a, s, p, param_coords, ctypes.byref(hp), mg, st))
    else:
        _check(L.sharded_adam_step_bucket_list(plan.handle, lst.ctypes.data, lst.size // 2, g, len(grads),
                                               grad_coords, scale, m, a, s, p, param_coords, ctypes.byref(hp), mg,
                                               st))


def sharded_adam_step_clipped(plan: Plan, grads, grad_coords: int, scale: float, master, exp_avg, exp_avg_sq,
                              param_out=None, param_coords: int = WORLD, *, grad_coeff, lr: float, beta1: float,
                              beta2: float, eps: float, weight_decay: float, step: int, main_grad_out=None,
                              stream=None) -> None:
    """sharded_adam_step with the fp32 main grad multiplied by grad_coeff (a
    one-element float32 device tensor; NaN skips the step)."""
    L = plan.shard_numel
    g = _ptr_list(grads, "grads", plan.extent(grad_coords))
    m = _dev_ptr(master, "master", "f32", L)
    a = _dev_ptr(exp_avg, "exp_avg", "f32", L)
    s = _dev_ptr(exp_avg_sq, "exp_avg_sq", "f32", L)
    p = None if param_out is None else _dev_ptr(param_out, "param_out", "bf16", plan.extent(param_coords))
    mg = None if main_grad_out is None else _dev_ptr(main_grad_out, "main_grad_out", "f32", L)
    c = _dev_ptr(grad_coeff, "grad_coeff", "f32", 1)
    hp = adam_hparams(lr, beta1, beta2, eps, weight_decay, step)
    _check(require_library().sharded_adam_step_clipped(plan.handle, g, len(grads), grad_coords, scale, m, a, s, p,
                                                       param_coords, ctypes.byref(hp), c, mg,
                                                       _stream(stream, master.device)))


def sharded_adam_step_instances(plan: Plan, instances, grad_coords: int, scale: float, master, exp_avg,
                                exp_avg_sq, param_out=None, param_coords: int = WORLD, *, lr: float, beta1: float,
                                beta2: float, eps: float, weight_decay: float, step: int, main_grad_out=None,
                                stream=None) -> None:
    """The step for several optimizer instances in one pass: instances is a
    sequence of n_instances sequences of D gradient tensors each."""
    flat = []
    for i, inst in enumerate(instances):
        if len(inst) != plan.dp_size:
            raise ValueError(f"instance {i} has {len(inst)} gradients, the plan's D is {plan.dp_size}")
        flat.extend(inst)
    L = plan.shard_numel
    g = _ptr_list(flat, "grads", plan.extent(grad_coords))
    m = _dev_ptr(master, "master", "f32", L)
    a = _dev_ptr(exp_avg, "exp_avg", "f32", L)
    s = _dev_ptr(exp_avg_sq, "exp_avg_sq", "f32", L)
    p = None if param_out is None else _dev_ptr(param_out, "param_out", "bf16", plan.extent(param_coords))
    mg = None if main_grad_out is None else _dev_ptr(main_grad_out, "main_grad_out", "f32", L)
    hp = adam_hparams(lr, beta1, beta2, eps, weight_decay, step)
    _check(require_library().sharded_adam_step_instances(plan.handle, g, len(instances), grad_coords, scale, m, a, s,
                                                         p, param_coords, ctypes.byref(hp), mg,
                                                         _stream(stream, master.device)))


def all_gather_params(plan: Plan, params, out, stream=None) -> None:
    """Rank j's range of every padded bucket from params[j] (D bf16 buffers
    of N elements, WORLD coordinates) into out; out may be one of them."""
    p = _ptr_list(params, "params", plan.buffer_numel)
    o = _dev_ptr(out, "out", "bf16", plan.buffer_numel)
    _check(require_library().all_gather_params(plan.handle, p, len(params), o, _stream(stream, out.device)))


def grad_norm_sq(plan: Plan, replicas, replica_coords: int, scale: float, workspace, norm_sq_out,
                 reduced_out=None, out_coords: int = WORLD, stream=None) -> None:
    """The rank's squared gradient norm into norm_sq_out (one-element float64
    device tensor); workspace: uint8 device tensor of plan.norm_workspace_bytes."""
    reps = _ptr_list(replicas, "replicas", plan.extent(replica_coords))
    ws = _dev_ptr(workspace, "workspace", "bytes", plan.norm_workspace_bytes)
    ns = _dev_ptr(norm_sq_out, "norm_sq_out", "f64", 1)
    ro = None if reduced_out is None else _dev_ptr(reduced_out, "reduced_out", "bf16", plan.extent(out_coords))
    _check(require_library().grad_norm_sq(plan.handle, reps, len(replicas), replica_coords, scale, ro, out_coords,
                                          ws, ns, _stream(stream, norm_sq_out.device)))


def grad_norm_sq_no_alloc(plan: Plan, replicas, replica_coords: int, scale: float, norm_sq_out,
                          reduced_out=None, out_coords: int = WORLD, stream=None) -> None:
    """grad_norm_sq with the library's static scratch array instead of a
    workspace (for callers that cannot allocate); calls that overlap in time
    on one GPU race."""
    reps = _ptr_list(replicas, "replicas", plan.extent(replica_coords))
    ns = _dev_ptr(norm_sq_out, "norm_sq_out", "f64", 1)
    ro = None if reduced_out is None else _dev_ptr(reduced_out, "reduced_out", "bf16", plan.extent(out_coords))
    _check(require_library().grad_norm_sq_no_alloc(plan.handle, reps, len(replicas), replica_coords, scale, ro,
                                                   out_coords, ns, _stream(stream, norm_sq_out.device)))


def clip_coefficient(norm_sq_parts, max_norm: float, coeff_out, norm_out=None, stream=None) -> None:
    """Global norm from the ranks' squared norms (float64 device tensor) and the
    clipping coefficient into coeff_out (one-element float32 device tensor)."""
    parts = _dev_ptr(norm_sq_parts, "norm_sq_parts", "f64", 1)
    c = _dev_ptr(coeff_out, "coeff_out", "f32", 1)
    n = None if norm_out is None else _dev_ptr(norm_out, "norm_out", "f64", 1)
    _check(require_library().clip_coefficient(parts, norm_sq_parts.numel(), max_norm, c, n,
                                              _stream(stream, coeff_out.device)))


def writeback_params(plan: Plan, master, param_out, param_coords: int, stream=None) -> None:
    m = _dev_ptr(master, "master", "f32", plan.shard_numel)
    p = _dev_ptr(param_out, "param_out", "bf16", plan.extent(param_coords))
    _check(require_library().writeback_params(plan.handle, m, p, param_coords, _stream(stream, master.device)))


def device_copy(dst, src, stream=None) -> None:
    """Plain device copy (the bandwidth reference); both tensors contiguous, same byte size."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("device_copy: dst too small")
    if not (dst.is_cuda and src.is_cuda and dst.is_contiguous() and src.is_contiguous()):
        raise ValueError("device_copy: contiguous device tensors required")
    _check(require_library().zdo_device_copy(dst.data_ptr(), src.data_ptr(), nbytes, _stream(stream, src.device)))


def stream_probe(reads, state, out, n: int, waves_per_cu: int = 0, stream=None, stores: int = PROBE_STORE_ALL) -> None:
    """The step's stream shape with trivial arithmetic (zdo_stream_probe): the
    bf16 tensors `reads` and the three float32 tensors `state` are read over
    n elements (a multiple of 512); `stores` selects what is then stored:
    the state rewritten and `out` (bf16) written (PROBE_STORE_ALL), `out`
    only (PROBE_STORE_OUT), or one word per tile of `out` (PROBE_STORE_NONE)."""
    r = _ptr_list(reads, "reads", n)
    s0, s1, s2 = (_dev_ptr(x, "state", "f32", n) for x in state)
    o = _dev_ptr(out, "out", "bf16", n)
    _check(require_library().zdo_stream_probe(r, len(reads), s0, s1, s2, o, n, stores, waves_per_cu,
                                              _stream(stream, out.device)))
