"""CPU oracle: one DP rank's share of a distributed-optimizer step, composed
from the range map (oracle.layout) and the element arithmetic (oracle/step.c).

TEST INFRASTRUCTURE; see oracle/__init__.py.

Coordinates of a buffer: WORLD = index into the whole padded flat buffer
[0, N); LOCAL = index into the rank's shard [0, L) (oracle.layout places the
per-bucket local views in the shard).

Page "04 · 分布式优化器":
  * §4.2: reduce-scatter of each bucket's grads, the rank keeping its 1/D range.
  * §4.3: copy of the rank's slice into the fp32 main grads, sliced per
    parameter through the "param" range (split parameters included), Adam on
    the shard only, and write-back of the updated master into the owned range.
  * §5: force_all_reduce produces the full reduced buffer instead.
"""

from __future__ import annotations

import numpy as np

from . import layout as L
from . import numerics as N

WORLD, LOCAL = 0, 1


def _span(coords, world: L.Range, local_start: int):
    if coords == WORLD:
        return world.start, world.end
    return local_start, local_start + world.size


def rank_step(layout: L.Layout, rank: int, grads, grad_coords: int, scale: float,
              master: np.ndarray, m: np.ndarray, v: np.ndarray, hp_arr: np.ndarray,
              param_out: np.ndarray | None = None, param_coords: int = WORLD,
              main_grad_out: np.ndarray | None = None, grad_coeff: float = 1.0,
              buckets: tuple | None = None) -> None:
    """Rank `rank`'s step, in place on master/m/v ([L] fp32) and param_out.
    grad_coeff multiplies the fp32 main grad (global-norm clipping); a NaN
    coefficient means a skipped step: nothing changes. buckets=(begin, end)
    restricts the step to those buckets' pieces."""
    if np.isnan(grad_coeff):
        return
    for pc in L.rank_pieces(layout, rank):
        if buckets is not None and not buckets[0] <= pc.bucket_index < buckets[1]:
            continue
        k0 = pc.shard_offset
        k1 = k0 + pc.gbuf_world.size
        g0, g1 = _span(grad_coords, pc.gbuf_world, k0)
        reps = [g[g0:g1] for g in grads]
        po = None
        if param_out is not None:
            p0, p1 = _span(param_coords, pc.gbuf_world, k0)
            po = param_out[p0:p1]
        mg = None if main_grad_out is None else main_grad_out[k0:k1]
        N.step(reps, scale, master[k0:k1], m[k0:k1], v[k0:k1], hp_arr, po, mg, grad_coeff)


def rank_norm_sq(layout: L.Layout, rank: int, grads, grad_coords: int, scale: float) -> float:
    """The rank's squared gradient norm: squares of the reduced gradient over
    its owned elements, summed in fp64 in shard order (pieces in order, the
    elements of each in order)."""
    total = 0.0
    for pc in L.rank_pieces(layout, rank):
        g0, g1 = _span(grad_coords, pc.gbuf_world, pc.shard_offset)
        total = total + N.norm_sq([g[g0:g1] for g in grads], scale)
    return total


def reduce_scatter(layout: L.Layout, rank: int, grads, grad_coords: int, scale: float,
                   out: np.ndarray, out_coords: int, buckets: tuple | None = None) -> None:
    """The rank's whole range of every bucket (padding included), reduced into
    `out`; buckets=(begin, end) restricts it to those buckets."""
    for b, (world, base) in enumerate(L.rank_ranges(layout, rank)):
        if buckets is not None and not buckets[0] <= b < buckets[1]:
            continue
        g0, g1 = _span(grad_coords, world, base)
        o0, o1 = _span(out_coords, world, base)
        N.reduce([g[g0:g1] for g in grads], scale, out=out[o0:o1])


def all_reduce(grads, scale: float) -> np.ndarray:
    """Every element of the padded buffer reduced (force_all_reduce)."""
    return N.reduce(list(grads), scale)


def all_gather(layout: L.Layout, params, out: np.ndarray) -> None:
    """Page 1, §4.4: after the step every bucket's parameter buffer is
    all-gathered, so that every rank holds the whole updated parameters: rank
    j's range of each bucket (padding included) is taken from params[j], the
    buffer rank j wrote back into (WORLD coordinates)."""
    for b in layout.buckets:
        for j in range(layout.dp_size):
            r = L.rank_range(b, layout.dp_size, j)
            out[r.start:r.end] = params[j][r.start:r.end]


def writeback(layout: L.Layout, rank: int, master: np.ndarray, param_out: np.ndarray,
              param_coords: int) -> None:
    """bf16(master) into the owned pieces of param_out (page 1, §4.3)."""
    for pc in L.rank_pieces(layout, rank):
        k0 = pc.shard_offset
        k1 = k0 + pc.gbuf_world.size
        p0, p1 = _span(param_coords, pc.gbuf_world, k0)
        param_out[p0:p1] = N.narrow(master[k0:k1])


def unsharded_step(layout: L.Layout, grads, scale: float, master_w: np.ndarray, m_w: np.ndarray,
                   v_w: np.ndarray, hp_arr: np.ndarray, param_out: np.ndarray) -> None:
    """The unsharded step: every parameter whole, with flat master/m/v indexed
    by world position (what every rank would compute without the optimizer
    sharding; page 1, §2)."""
    for r in layout.param_world:
        s, e = r.start, r.end
        N.step([g[s:e] for g in grads], scale, master_w[s:e], m_w[s:e], v_w[s:e], hp_arr,
               param_out[s:e])


def gather_shard(layout: L.Layout, rank: int, flat: np.ndarray, fill=0) -> np.ndarray:
    """The rank's shard view ([L]) of a world-indexed array; slots outside the
    owned pieces hold `fill`."""
    out = np.full(L.shard_numel(layout, rank), fill, dtype=flat.dtype)
    for pc in L.rank_pieces(layout, rank):
        k0 = pc.shard_offset
        out[k0:k0 + pc.gbuf_world.size] = flat[pc.gbuf_world.start:pc.gbuf_world.end]
    return out


def scatter_shard(layout: L.Layout, rank: int, shard: np.ndarray, flat: np.ndarray) -> None:
    for pc in L.rank_pieces(layout, rank):
        k0 = pc.shard_offset
        flat[pc.gbuf_world.start:pc.gbuf_world.end] = shard[k0:k0 + pc.gbuf_world.size]


def local_slices(layout: L.Layout, rank: int, world_buf: np.ndarray, fill=0) -> np.ndarray:
    """The rank's LOCAL-coordinate view of a world buffer (whole ranges, padding included)."""
    out = np.full(L.shard_numel(layout, rank), fill, dtype=world_buf.dtype)
    for world, base in L.rank_ranges(layout, rank):
        out[base:base + world.size] = world_buf[world.start:world.end]
    return out
