// Device kernels for gfx950 (CDNA4): the fused sharded Adam step, the
// reduce-scatter / all-reduce of the D contributions, the squared gradient
// norm and clipping coefficient, the parameter write-back, the parameter
// all-gather, and two measurement references (a plain copy and the step's
// stream shape with trivial arithmetic).
//
// Every kernel is a stream: the step moves (2D + 26) bytes per element
// against a few dozen VALU operations, so it is bound by HBM bandwidth, not
// by the matrix cores. A LOCAL index is congruent to its WORLD index modulo
// 64, and a segment's tiles start at a multiple of 64 WORLD elements, so
// with 128-byte-aligned buffers every stream crosses cache lines at tile
// boundaries only (no line is fetched by two workgroups). A workgroup is a
// single wave and takes a tile of 512 consecutive elements of one segment:
// 1 KiB of every bf16 stream and 2 KiB of every fp32 stream, contiguously.
// In the reduce, norm and write-back kernels lane l takes the 8-element
// chunk [8l, 8l + 8) of the tile (one 16-byte load per bf16 stream); the
// step takes two quads per lane (at 32 contributions it reduces whole tiles
// by 8-element chunks and moves the results to the quads across lanes) and
// the all-gather 2048-element tiles (see there). Chunks or quads cut by a
// segment's ends take a per-element path. A launch walks one run of tiles,
// or up to 16 runs (a list of bucket ranges) through tile_at; a short launch
// hands each XCD 8 consecutive tiles at a time (launch_index).
//
// HBM serves this mix of many read streams and some write streams best when
// few requestors share it: one-wave workgroups, a number per compute unit
// capped by the kernel and the launch's length (see lds_reserve; kernels
// that move only a few KiB per tile take more waves or none), non-temporal
// loads of what is read once.
//
// Arithmetic is fixed (contraction off, IEEE division and square root,
// fp32 subnormals kept) so that results match a sequential CPU evaluation bit
// for bit; the order of operations is the one stated in include/zdo.h.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <mutex>

#include "kernels.h"

#pragma clang fp contract(off)

// Scratch memory of grad_norm_sq_no_alloc: the squared norm's per-tile
// partials and level sums for callers that cannot allocate. One copy per GPU
// the library runs on, held until the process ends; every call on a GPU
// shares it (calls that overlap in time on one GPU race). Host code never
// names it: it takes the device address from hipGetSymbolAddress, per device
// (zdo::no_alloc_scratch below).
static __device__ __align__(256) unsigned char scratch[ZDO_NO_ALLOC_SCRATCH_BYTES];

namespace zdo {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---- bf16 ----------------------------------------------------------------------
// A bf16 is the top half of an fp32: widening is a shift or a mask.
__device__ __forceinline__ float lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float h_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Two fp32 to their nearest bf16 (ties to even), packed a | b << 16: one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t to_bf16x2(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// ---- memory ------------------------------------------------------------------------
// The replicas are read exactly once per launch: their loads carry the
// non-temporal hint, which keeps them from displacing the fp32 state in the
// caches (measured: +2% on a 42 GB step, +18% when the state fits the
// 256 MB Infinity Cache between steps). The write-only outputs (parameters,
// reduced gradient, main grad) are non-temporal stores too (Llama-3-8B-shaped
// step: 6.83 ms in every run against 6.83-7.48 ms with plain stores;
// Llama-3-70B-shaped reduce-scatter 7% faster). The fp32 state is read and
// then rewritten. While it is at most a few times the 256 MB Infinity
// Cache, plain loads and stores serve it best (GPT-2-shaped step, 187 MB of
// state, back to back: 97.5 us against 109.8 us with non-temporal state
// accesses). Beyond 1 GiB (see launch_step) the step loads and stores it
// non-temporally as well (Llama-3-8B-shaped step: 6.92-6.98 -> 6.75-6.77
// ms); non-temporal stores after plain loads of the same lines are far
// slower than either (3.4-3.6 TB/s).
__device__ __forceinline__ u32x4 ld_rep(const uint16_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ f32x4 ldf4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ void st16_out(uint16_t *p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}
__device__ __forceinline__ void stf4(float *p, f32x4 v) { *reinterpret_cast<f32x4 *>(p) = v; }
__device__ __forceinline__ void stf4_out(float *p, f32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(p));
}
template <bool kNT>
__device__ __forceinline__ f32x4 ld_state(const float *p) {
    if constexpr (kNT)
        return __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
    else
        return ldf4(p);
}
template <bool kNT>
__device__ __forceinline__ void st_state(float *p, f32x4 v) {
    if constexpr (kNT)
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(p));
    else
        stf4(p, v);
}

// ---- walking the segments -------------------------------------------------------------
struct ChunkPos {
    int64_t w0;     // WORLD index of the chunk's first slot (a multiple of 8)
    int64_t k0;     // LOCAL index of the same slot
    int lo, hi;     // the chunk's slots [lo, hi) that belong to the segment
};

// The plan's tables are read-only for the life of the plan: read through the
// constant address space, the compiler fetches them with scalar loads (one
// per wave, into scalar registers) instead of 64-lane vector loads of one
// address.
template <typename T>
using ro_ptr = const __attribute__((address_space(4))) T *;
template <typename T>
__device__ __forceinline__ ro_ptr<T> ro(const T *p) {
    return (ro_ptr<T>)(p);
}
__device__ __forceinline__ Seg ld_seg(ro_ptr<Seg> p) {
    Seg s;
    s.wbeg = p->wbeg;
    s.lbeg = p->lbeg;
    s.len = p->len;
    s.tile0 = p->tile0;
    return s;
}

// The segment holding `tile` (a table walk): its group's entry, which holds
// the segment itself unless the tile lies past a later segment's start in
// the group; then those segments by their first tile.
__device__ __forceinline__ Seg seg_of(const Walk &wk, int64_t tile) {
    const ro_ptr<GroupSeg> g = ro(wk.group) + tile / kTileGroup;
    if (tile < g->next_tile0)
        return ld_seg(&g->seg);
    int64_t si = g->index + 1;
    Seg cur = ld_seg(ro(wk.segs) + si);
    while (si + 1 < wk.nseg) {
        const Seg nxt = ld_seg(ro(wk.segs) + si + 1);
        if (nxt.tile0 > tile)
            break;
        cur = nxt;
        ++si;
    }
    return cur;
}

// Launches of fewer tiles than this are short: one workgroup per tile (the
// grid cap is far above it), a few rounds of waves over the chip.
constexpr int64_t kShortLaunchTiles = int64_t(1) << 17;

// The launch index that launch slot i (a workgroup's blockIdx.x, plus the
// grid stride when the grid is capped) takes. The dispatcher hands
// workgroups to the 8 XCDs in turn, workgroup i to XCD i mod 8. In a short
// launch each XCD takes 8 consecutive launch indices out of every 64 instead
// of every 8th: within each block of 64 slots the 8 x 8 order is transposed,
// a bijection; the slots after the last whole block keep their index. Short
// launches ran faster so (fragmentation workload, rank 0: step 48.2 -> 45.0
// us back to back, 53.6 -> 51.0 us with cold caches; GPT-2 shape within 1%),
// long ones slower (Llama-3-70B shape 33.4 -> 34.6 ms, Llama-3-8B 6.87 ->
// 7.12 ms), so long launches keep the dispatch order. Kernels that
// store per-index results (the squared norm's tile partials) store them at
// the launch index, so their order does not change.
constexpr int64_t kXcds = 8, kXcdRun = 8, kXcdBlock = kXcds * kXcdRun;
__device__ __forceinline__ int64_t launch_index(const Walk &wk, int64_t i) {
    if (wk.ntiles >= kShortLaunchTiles || i >= wk.ntiles / kXcdBlock * kXcdBlock)
        return i;
    const int64_t r = i % kXcdBlock;
    return i - r + (r % kXcds) * kXcdRun + r / kXcds;
}

// The tile at launch index i (wave-uniform). With several runs the run table
// is read where the launch put it, at the start of the kernel arguments
// (every walking kernel takes its Walk first), by a scan whose index the
// compiler cannot hoist out of the tile loop: hoisted, the 32 table entries
// would stay in scalar registers for the whole kernel.
static_assert(offsetof(ReduceArgs, walk) == 0 && offsetof(StepArgs, walk) == 0 && offsetof(NormArgs, walk) == 0 &&
                  offsetof(WritebackArgs, walk) == 0,
              "tile_at reads the Walk at the start of the kernel arguments");
__device__ __forceinline__ int64_t tile_at(const Walk &wk, int64_t i) {
    if (wk.nruns <= 1)
        return wk.run_begin[0] + i;
    const ro_ptr<Walk> kw = (ro_ptr<Walk>)(__builtin_amdgcn_kernarg_segment_ptr());
    int r = 0;
    while (r + 1 < wk.nruns && i >= kw->run_start[r + 1])
        ++r;
    return kw->run_begin[r] + (i - kw->run_start[r]);
}

// The chunk this thread takes in `tile`; false if it holds no element of the
// segment.
__device__ __forceinline__ bool chunk_of(const Walk &wk, int64_t tile, ChunkPos &c) {
    int64_t wbeg, lbeg, len, tile0;
    if (wk.segs) {
        const Seg s = seg_of(wk, tile);
        wbeg = s.wbeg;
        lbeg = s.lbeg;
        len = s.len;
        tile0 = s.tile0;
    } else {
        wbeg = 0;
        lbeg = 0;
        len = wk.flat_numel;
        tile0 = 0;
    }
    const int64_t w0 = tile_origin(wbeg) + (tile - tile0) * kTileElems + int64_t(threadIdx.x) * kChunk;
    const int64_t wend = wbeg + len;
    if (w0 >= wend || w0 + kChunk <= wbeg)
        return false;
    c.w0 = w0;
    c.k0 = lbeg + (w0 - wbeg);
    c.lo = w0 < wbeg ? int(wbeg - w0) : 0;
    c.hi = w0 + kChunk > wend ? int(wend - w0) : kChunk;
    return true;
}

// ---- the reduction ------------------------------------------------------------------------
// s_j = bf16(g_j * scale); acc = s_0 + s_1 + ... in rank order (fp32).
__device__ __forceinline__ void first_term(float acc[8], u32x4 r, float scale) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t s = to_bf16x2(lo_f32(r[k]) * scale, hi_f32(r[k]) * scale);
        acc[2 * k] = lo_f32(s);
        acc[2 * k + 1] = hi_f32(s);
    }
}
__device__ __forceinline__ void add_term(float acc[8], u32x4 r, float scale) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t s = to_bf16x2(lo_f32(r[k]) * scale, hi_f32(r[k]) * scale);
        acc[2 * k] = acc[2 * k] + lo_f32(s);
        acc[2 * k + 1] = acc[2 * k + 1] + hi_f32(s);
    }
}

// Sum of the contributions over one full chunk at index `gi` of every replica.
template <int D>
__device__ __forceinline__ void reduce_chunk(const uint16_t *const *rep, int nrep, int64_t gi, float scale,
                                             float acc[8]) {
    if constexpr (D > 0) {
        u32x4 r[D];
#pragma unroll
        for (int j = 0; j < D; ++j)
            r[j] = ld_rep(rep[j] + gi);
        first_term(acc, r[0], scale);
#pragma unroll
        for (int j = 1; j < D; ++j)
            add_term(acc, r[j], scale);
    } else {
        first_term(acc, ld_rep(rep[0] + gi), scale);
        for (int j = 1; j < nrep; ++j)
            add_term(acc, ld_rep(rep[j] + gi), scale);
    }
}

// The same for one element.
template <int D>
__device__ __forceinline__ float reduce_one(const uint16_t *const *rep, int nrep, int64_t i, float scale) {
    const int n = D > 0 ? D : nrep;
    float acc = lo_f32(to_bf16x2(h_f32(rep[0][i]) * scale, 0.0f));
    for (int j = 1; j < n; ++j)
        acc = acc + lo_f32(to_bf16x2(h_f32(rep[j][i]) * scale, 0.0f));
    return acc;
}

// Several optimizer instances, one element: instance k's contributions
// rep[k*d .. k*d+d) reduced as above and rounded to bf16 (what the instance's
// reduce-scatter leaves in its grad buffer), then those bf16 results added
// in fp32 in instance order (the all-reduce across instances).
template <int D>
__device__ __forceinline__ float reduce_one_instances(const uint16_t *const *rep, int d, int ninst, int64_t i,
                                                      float scale) {
    float acc = lo_f32(to_bf16x2(reduce_one<D>(rep, d, i, scale), 0.0f));
    for (int k = 1; k < ninst; ++k)
        acc = acc + lo_f32(to_bf16x2(reduce_one<D>(rep + k * d, d, i, scale), 0.0f));
    return acc;
}

// ---- Adam --------------------------------------------------------------------------------------
__device__ __forceinline__ void adam(const AdamConst &c, float g, float &p, float &m, float &v) {
    const float m1 = c.b1 * m;
    const float m2 = c.omb1 * g;
    const float mn = m1 + m2;
    const float gg = g * g;
    const float v1 = c.b2 * v;
    const float v2 = c.omb2 * gg;
    const float vn = v1 + v2;
    const float mh = mn / c.bc1;
    const float vh = vn / c.bc2;
    const float den = __builtin_sqrtf(vh) + c.eps;
    const float u = mh / den;
    const float wdp = c.wd * p;
    const float u2 = u + wdp;
    const float st = c.lr * u2;
    p = p - st;
    m = mn;
    v = vn;
}

// ---- kernels -------------------------------------------------------------------------------------

template <int D>
__global__ __launch_bounds__(kBlock) void reduce_kernel(ReduceArgs a) {
    for (int64_t i = blockIdx.x; i < a.walk.ntiles; i += gridDim.x) {
        const int64_t j = launch_index(a.walk, i);
        const int64_t tile = tile_at(a.walk, j);
        ChunkPos c;
        if (!chunk_of(a.walk, tile, c))
            continue;
        const int64_t gi = a.in_local ? c.k0 : c.w0;
        const int64_t oi = a.out_local ? c.k0 : c.w0;
        if (c.lo == 0 && c.hi == kChunk) {
            float acc[8];
            reduce_chunk<D>(a.rep, a.nrep, gi, a.scale, acc);
            u32x4 o;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                o[k] = to_bf16x2(acc[2 * k], acc[2 * k + 1]);
            st16_out(a.out + oi, o);
        } else {
            for (int e = c.lo; e < c.hi; ++e) {
                const float acc = reduce_one<D>(a.rep, a.nrep, gi + e, a.scale);
                a.out[oi + e] = uint16_t(to_bf16x2(acc, 0.0f));
            }
        }
    }
}

// ---- the step ------------------------------------------------------------------------------
// The step's lanes go by quads: lane l takes slots [4l, 4l + 4) and
// [256 + 4l, 256 + 4l + 4) of its 512-element tile, so that every load and
// store instruction of the wave covers one contiguous run (512 bytes of a
// bf16 stream, 1 KiB of an fp32 stream). With 8 consecutive slots per lane
// (as the other kernels take them), a 16-byte fp32 access covers every other
// 16 bytes of a 2 KiB run; by quads the step measured 2-4% faster on large
// shards. A lane whose two quads both lie inside the segment issues every
// load of the tile before any arithmetic; at a segment's edges a full quad
// goes alone and a partial one slot by slot.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x2 ld_rep2(const uint16_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
}
__device__ __forceinline__ void st8_out(uint16_t *p, u32x2 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(p));
}

struct Quad {
    int64_t w0, k0;  // WORLD and LOCAL index of slot 0 (w0 a multiple of 4)
    int lo, hi;      // slots [lo, hi) belong to the segment; none if lo >= hi
};

// The segment walk's view of `tile`: its segment, or the flat run.
struct SegView {
    int64_t wbeg, lbeg, len, tile0;
};
__device__ __forceinline__ SegView seg_view(const Walk &wk, int64_t tile) {
    if (wk.segs) {
        const Seg s = seg_of(wk, tile);
        return {s.wbeg, s.lbeg, s.len, s.tile0};
    }
    return {0, 0, wk.flat_numel, 0};
}

// The lane's two quads of the tile starting at WORLD index tw.
__device__ __forceinline__ void quads_in(const SegView &s, int64_t tw, Quad q[2]) {
    const int64_t wend = s.wbeg + s.len;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t w0 = tw + h * (kTileElems / 2) + 4 * int64_t(threadIdx.x);
        q[h].w0 = w0;
        q[h].k0 = s.lbeg + (w0 - s.wbeg);
        q[h].lo = w0 < s.wbeg ? (s.wbeg - w0 < 4 ? int(s.wbeg - w0) : 4) : 0;
        q[h].hi = w0 + 4 > wend ? (wend > w0 ? int(wend - w0) : 0) : 4;
    }
}

__device__ __forceinline__ bool full(const Quad &q) { return q.lo == 0 && q.hi == 4; }

__device__ __forceinline__ void first_term2(float acc[4], u32x2 r, float scale) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const uint32_t s = to_bf16x2(lo_f32(r[k]) * scale, hi_f32(r[k]) * scale);
        acc[2 * k] = lo_f32(s);
        acc[2 * k + 1] = hi_f32(s);
    }
}
__device__ __forceinline__ void add_term2(float acc[4], u32x2 r, float scale) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const uint32_t s = to_bf16x2(lo_f32(r[k]) * scale, hi_f32(r[k]) * scale);
        acc[2 * k] = acc[2 * k] + lo_f32(s);
        acc[2 * k + 1] = acc[2 * k + 1] + hi_f32(s);
    }
}

// The reduced gradient (fp32, before its bf16 rounding) of Q full quads at
// contribution indices gi[0..Q), slots 4q..4q+3 of acc. Plain: the a.nrep
// contributions in rank order. kInst: a.ninst instances of D (D = 0: a.dinst)
// contributions; each instance's sum rounded to bf16, those added in fp32 in
// instance order. With D fixed, every load of an instance is issued before
// its arithmetic.
template <int D, bool kInst, int Q>
__device__ __forceinline__ void reduce_quads(const StepArgs &a, const int64_t *gi, float *acc) {
    const int d = kInst ? a.dinst : a.nrep;
    const int ni = kInst ? a.ninst : 1;
    for (int i = 0; i < ni; ++i) {
        const uint16_t *const *rep = a.rep + i * d;
        float part[4 * Q];
        if constexpr (D > 0) {
            u32x2 r[Q][D];
#pragma unroll
            for (int j = 0; j < D; ++j)
#pragma unroll
                for (int h = 0; h < Q; ++h)
                    r[h][j] = ld_rep2(rep[j] + gi[h]);
#pragma unroll
            for (int h = 0; h < Q; ++h) {
                first_term2(part + 4 * h, r[h][0], a.scale);
#pragma unroll
                for (int j = 1; j < D; ++j)
                    add_term2(part + 4 * h, r[h][j], a.scale);
            }
        } else {
#pragma unroll
            for (int h = 0; h < Q; ++h)
                first_term2(part + 4 * h, ld_rep2(rep[0] + gi[h]), a.scale);
            for (int j = 1; j < d; ++j)
#pragma unroll
                for (int h = 0; h < Q; ++h)
                    add_term2(part + 4 * h, ld_rep2(rep[j] + gi[h]), a.scale);
        }
        if constexpr (!kInst) {
#pragma unroll
            for (int e = 0; e < 4 * Q; ++e)
                acc[e] = part[e];
        } else {
#pragma unroll
            for (int k = 0; k < 2 * Q; ++k) {
                const uint32_t r = to_bf16x2(part[2 * k], part[2 * k + 1]);
                acc[2 * k] = i == 0 ? lo_f32(r) : acc[2 * k] + lo_f32(r);
                acc[2 * k + 1] = i == 0 ? hi_f32(r) : acc[2 * k + 1] + hi_f32(r);
            }
        }
    }
}

// Adam and the stores for Q full quads at LOCAL k0[h] / WORLD w0[h], from
// their state and their reduced gradient (bf16 pairs, red[2h], red[2h + 1]).
template <int Q, bool kNT>
__device__ __forceinline__ void finish_quads(const StepArgs &a, const int64_t *k0, const int64_t *w0,
                                             const f32x4 *pv, const f32x4 *mv, const f32x4 *vv,
                                             const uint32_t *red, bool clip, float cf) {
    float g[4 * Q];
#pragma unroll
    for (int k = 0; k < 2 * Q; ++k) {
        g[2 * k] = lo_f32(red[k]);
        g[2 * k + 1] = hi_f32(red[k]);
    }
    if (clip) {
#pragma unroll
        for (int e = 0; e < 4 * Q; ++e)
            g[e] = g[e] * cf;
    }
#pragma unroll
    for (int h = 0; h < Q; ++h) {
        float p[4], m[4], v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            p[e] = pv[h][e];
            m[e] = mv[h][e];
            v[e] = vv[h][e];
            adam(a.c, g[4 * h + e], p[e], m[e], v[e]);
        }
        st_state<kNT>(a.master + k0[h], f32x4{p[0], p[1], p[2], p[3]});
        st_state<kNT>(a.m + k0[h], f32x4{m[0], m[1], m[2], m[3]});
        st_state<kNT>(a.v + k0[h], f32x4{v[0], v[1], v[2], v[3]});
        if (a.main_grad)
            stf4_out(a.main_grad + k0[h], f32x4{g[4 * h], g[4 * h + 1], g[4 * h + 2], g[4 * h + 3]});
        if (a.param)
            st8_out(a.param + (a.param_local ? k0[h] : w0[h]),
                    u32x2{to_bf16x2(p[0], p[1]), to_bf16x2(p[2], p[3])});
    }
}

// A whole tile inside its segment, D contributions by 16-byte loads: lane l
// reduces the tile's slots [8l, 8l + 8) (one load per contribution, 1 KiB
// per load instruction), then takes its two quads' reduced values, slots
// [4l, 4l + 4) and [256 + 4l, 256 + 4l + 4), from lanes l/2 and 32 + l/2
// through the cross-lane permute; the state stays in the quad layout. Half
// the load instructions of the quad path, so every load of the tile is in
// flight at once up to 32 contributions. tw: WORLD index of the tile's first
// slot; kb: its LOCAL index.
template <int D, bool kNT>
__device__ __forceinline__ void step_tile_wide(const StepArgs &a, int64_t tw, int64_t kb, bool clip, float cf) {
    const int lane = int(threadIdx.x);
    int64_t k0[2], w0[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        k0[h] = kb + h * (kTileElems / 2) + 4 * lane;
        w0[h] = tw + h * (kTileElems / 2) + 4 * lane;
    }
    f32x4 pv[2], mv[2], vv[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        pv[h] = ld_state<kNT>(a.master + k0[h]);
        mv[h] = ld_state<kNT>(a.m + k0[h]);
        vv[h] = ld_state<kNT>(a.v + k0[h]);
    }
    const int64_t gi = (a.in_local ? kb : tw) + int64_t(kChunk) * lane;
    u32x4 r[D];
#pragma unroll
    for (int j = 0; j < D; ++j)
        r[j] = ld_rep(a.rep[j] + gi);
    float acc[8];
    first_term(acc, r[0], a.scale);
#pragma unroll
    for (int j = 1; j < D; ++j)
        add_term(acc, r[j], a.scale);
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        w[k] = to_bf16x2(acc[2 * k], acc[2 * k + 1]);
    // quad 0 of lane l: words 2(l&1), 2(l&1)+1 of lane l/2; quad 1: the same
    // words of lane 32 + l/2
    const int src0 = (lane >> 1) << 2, src1 = (32 + (lane >> 1)) << 2;
    const bool odd = lane & 1;
    uint32_t red[4];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const uint32_t a0 = uint32_t(__builtin_amdgcn_ds_bpermute(src0, int(w[k])));
        const uint32_t a1 = uint32_t(__builtin_amdgcn_ds_bpermute(src0, int(w[k + 2])));
        const uint32_t b0 = uint32_t(__builtin_amdgcn_ds_bpermute(src1, int(w[k])));
        const uint32_t b1 = uint32_t(__builtin_amdgcn_ds_bpermute(src1, int(w[k + 2])));
        red[k] = odd ? a1 : a0;
        red[2 + k] = odd ? b1 : b0;
    }
    finish_quads<2, kNT>(a, k0, w0, pv, mv, vv, red, clip, cf);
}

// The whole step for Q full quads: reduce, Adam, write-back. The state loads
// come first, so that they are in flight together with the contributions'
// loads rather than after the reduction.
template <int D, bool kInst, int Q, bool kNT>
__device__ __forceinline__ void step_quads(const StepArgs &a, const Quad *q, bool clip, float cf) {
    int64_t gi[Q];
#pragma unroll
    for (int h = 0; h < Q; ++h)
        gi[h] = a.in_local ? q[h].k0 : q[h].w0;
    f32x4 pv[Q], mv[Q], vv[Q];
#pragma unroll
    for (int h = 0; h < Q; ++h) {
        pv[h] = ld_state<kNT>(a.master + q[h].k0);
        mv[h] = ld_state<kNT>(a.m + q[h].k0);
        vv[h] = ld_state<kNT>(a.v + q[h].k0);
    }
    float acc[4 * Q];
    reduce_quads<D, kInst, Q>(a, gi, acc);
    uint32_t red[2 * Q];
#pragma unroll
    for (int k = 0; k < 2 * Q; ++k)
        red[k] = to_bf16x2(acc[2 * k], acc[2 * k + 1]);
    int64_t k0[Q], w0[Q];
#pragma unroll
    for (int h = 0; h < Q; ++h) {
        k0[h] = q[h].k0;
        w0[h] = q[h].w0;
    }
    finish_quads<Q, kNT>(a, k0, w0, pv, mv, vv, red, clip, cf);
}

// The step for the slots [lo, hi) of a partial quad, one at a time.
template <int D, bool kInst>
__device__ __forceinline__ void step_slots(const StepArgs &a, const Quad &q, bool clip, float cf) {
    const int64_t gi = a.in_local ? q.k0 : q.w0;
    const int64_t pi = a.param_local ? q.k0 : q.w0;
    for (int e = q.lo; e < q.hi; ++e) {
        const float acc = kInst ? reduce_one_instances<D>(a.rep, a.dinst, a.ninst, gi + e, a.scale)
                                : reduce_one<D>(a.rep, a.nrep, gi + e, a.scale);
        float g = lo_f32(to_bf16x2(acc, 0.0f));
        if (clip)
            g = g * cf;
        float p = a.master[q.k0 + e], m = a.m[q.k0 + e], v = a.v[q.k0 + e];
        adam(a.c, g, p, m, v);
        a.master[q.k0 + e] = p;
        a.m[q.k0 + e] = m;
        a.v[q.k0 + e] = v;
        if (a.main_grad)
            a.main_grad[q.k0 + e] = g;
        if (a.param)
            a.param[pi + e] = uint16_t(to_bf16x2(p, 0.0f));
    }
}

// Whole tiles of a fixed number of contributions, at least ZDO_WIDE_STEP_MIN_D,
// take step_tile_wide; edge tiles (a quad at a time) and the other forms
// take the quads. Measured against the quad path in alternating runs on one
// box: Llama-3-70B shape (32 contributions) 33.87 -> 33.65 ms and 33.68 ->
// 33.55 ms; fragmentation (16) 48.5 -> 48.7 us; Llama-3-8B (8) 6.84 -> 6.95
// ms. So only 32 contributions take it.
#ifndef ZDO_WIDE_STEP_MIN_D
#define ZDO_WIDE_STEP_MIN_D 32
#endif
template <int D, bool kInst>
constexpr bool kWideStep = !kInst && D >= 1 && D >= ZDO_WIDE_STEP_MIN_D;

// kInst: a.rep holds a.ninst instances of D (or, for D = 0, a.dinst)
// contributions each; otherwise a.nrep contributions of one instance.
//
// kNT: the fp32 state is loaded and stored non-temporally (it exceeds
// 1 GiB; see launch_step).
//
// The occupancy bounds tell the compiler how many waves can share a SIMD,
// which the launches cap anyway (lds_reserve): with at most 4 (2 for 32
// contributions, whose long launches run 6 waves per compute unit: 1.5 per
// SIMD), it keeps every load of a tile in flight before the first wait
// instead of interleaving waits to save registers.
template <int D, bool kInst, bool kNT>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(D >= 32 && !kInst ? 2 : 1, D < 32 ? 4 : 3)))
void step_kernel(StepArgs a) {
    // Global-norm clipping: the main grad is multiplied by the coefficient; a
    // NaN coefficient (found-inf) leaves everything unchanged.
    // The coefficient load goes out with the walk's arguments, and a NaN
    // empties the tile range instead of branching: a test inside the tile
    // body would split the block that issues all of a tile's loads at once.
    const bool clip = a.coeff != nullptr;
    const float cf = clip ? *ro(a.coeff) : 1.0f;
    const int64_t iend = clip && cf != cf ? 0 : a.walk.ntiles;
    for (int64_t i = blockIdx.x; i < iend; i += gridDim.x) {
        const int64_t j = launch_index(a.walk, i);
        const int64_t tile = tile_at(a.walk, j);
        const SegView sv = seg_view(a.walk, tile);
        const int64_t tw = tile_origin(sv.wbeg) + (tile - sv.tile0) * kTileElems;
        if constexpr (kWideStep<D, kInst>) {
            // wave-uniform: the whole tile lies inside the segment
            if (tw >= sv.wbeg && tw + kTileElems <= sv.wbeg + sv.len) {
                step_tile_wide<D, kNT>(a, tw, sv.lbeg + (tw - sv.wbeg), clip, cf);
                continue;
            }
        }
        Quad q[2];
        quads_in(sv, tw, q);
        if (!kWideStep<D, kInst> && full(q[0]) && full(q[1])) {
            step_quads<D, kInst, 2, kNT>(a, q, clip, cf);
        } else {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (full(q[h]))
                    step_quads<D, kInst, 1, kNT>(a, q + h, clip, cf);
                else
                    step_slots<D, kInst>(a, q[h], clip, cf);
            }
        }
    }
}

// ---- squared gradient norm -----------------------------------------------------------------
// Per tile: each lane sums the squares of its chunk's elements in order (each
// square is exact in fp64: a bf16 has an 8-bit significand), then a fixed
// butterfly over the wave's 64 lanes gives every lane the same tile total.
static_assert(kBlock == 64, "the tile reduction below assumes one wave per workgroup");

template <int D>
__global__ __launch_bounds__(kBlock) void norm_kernel(NormArgs a) {
    for (int64_t i = blockIdx.x; i < a.walk.ntiles; i += gridDim.x) {
        const int64_t j = launch_index(a.walk, i);
        const int64_t tile = tile_at(a.walk, j);
        ChunkPos c;
        double s = 0.0;
        if (chunk_of(a.walk, tile, c)) {
            const int64_t gi = a.in_local ? c.k0 : c.w0;
            const int64_t oi = a.out_local ? c.k0 : c.w0;
            if (c.lo == 0 && c.hi == kChunk) {
                float acc[8];
                reduce_chunk<D>(a.rep, a.nrep, gi, a.scale, acc);
                u32x4 o;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    o[k] = to_bf16x2(acc[2 * k], acc[2 * k + 1]);
                    const double g0 = double(lo_f32(o[k])), g1 = double(hi_f32(o[k]));
                    s = s + g0 * g0;
                    s = s + g1 * g1;
                }
                if (a.out)
                    st16_out(a.out + oi, o);
            } else {
                for (int e = c.lo; e < c.hi; ++e) {
                    const uint32_t r = to_bf16x2(reduce_one<D>(a.rep, a.nrep, gi + e, a.scale), 0.0f);
                    const double g = double(lo_f32(r));
                    s = s + g * g;
                    if (a.out)
                        a.out[oi + e] = uint16_t(r);
                }
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
            s = s + __shfl_xor(s, off, 64);
        if (threadIdx.x == 0)
            a.partial[j] = s;
    }
}

// Sum of n tile partials in two fixed-order levels: workgroup b of G adds
// the contiguous run [b*chunk, min(n, (b+1)*chunk)) (work-item t takes
// indices t, t + 1024, ... of the run in order, then a fixed tree over the
// 1024 work-items) into level[b]; one workgroup then adds level[0..G) by the
// same scheme into *out. The order depends on n only.
constexpr int kSumThreads = 1024;
constexpr int kSumGroups = 1024;

__device__ __forceinline__ double block_sum(const double *x, int64_t n) {
    __shared__ double sh[kSumThreads];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += kSumThreads)
        s = s + x[i];
    sh[threadIdx.x] = s;
    __syncthreads();
    for (int w = kSumThreads / 2; w > 0; w >>= 1) {
        if (int(threadIdx.x) < w)
            sh[threadIdx.x] = sh[threadIdx.x] + sh[threadIdx.x + w];
        __syncthreads();
    }
    return sh[0];
}

__global__ __launch_bounds__(kSumThreads) void tile_sum_kernel(const double *partial, int64_t n, int64_t chunk,
                                                               double *level) {
    const int64_t b0 = int64_t(blockIdx.x) * chunk;
    const int64_t len = n - b0 < chunk ? n - b0 : chunk;
    const double s = block_sum(partial + b0, len > 0 ? len : 0);
    if (threadIdx.x == 0)
        level[blockIdx.x] = s;
}

__global__ __launch_bounds__(kSumThreads) void level_sum_kernel(const double *level, int64_t g, double *out) {
    const double s = block_sum(level, g);
    if (threadIdx.x == 0)
        *out = s;
}

// The clipping coefficient from n squared norms, summed in index order.
__global__ __launch_bounds__(64) void clip_kernel(const double *parts, int32_t n, float max_norm, float *coeff,
                                                  double *norm_out) {
    if (threadIdx.x != 0)
        return;
    double total = 0.0;
    for (int32_t i = 0; i < n; ++i)
        total = total + parts[i];
    const double norm = __builtin_sqrt(total);
    if (norm_out)
        *norm_out = norm;
    if (!__builtin_isfinite(norm)) {
        *coeff = __builtin_nanf("");
        return;
    }
    const double q = double(max_norm) / (norm + 1e-6);
    *coeff = float(q < 1.0 ? q : 1.0);
}

// kNT: master is loaded non-temporally (the state exceeds 1 GiB), as in
// the step.
template <bool kNT>
__global__ __launch_bounds__(kBlock) void writeback_kernel(WritebackArgs a) {
    for (int64_t i = blockIdx.x; i < a.walk.ntiles; i += gridDim.x) {
        const int64_t j = launch_index(a.walk, i);
        const int64_t tile = tile_at(a.walk, j);
        ChunkPos c;
        if (!chunk_of(a.walk, tile, c))
            continue;
        const int64_t pi = a.param_local ? c.k0 : c.w0;
        if (c.lo == 0 && c.hi == kChunk) {
            const f32x4 x0 = ld_state<kNT>(a.master + c.k0), x1 = ld_state<kNT>(a.master + c.k0 + 4);
            u32x4 o = {to_bf16x2(x0[0], x0[1]), to_bf16x2(x0[2], x0[3]), to_bf16x2(x1[0], x1[1]),
                       to_bf16x2(x1[2], x1[3])};
            st16_out(a.param + pi, o);
        } else {
            for (int e = c.lo; e < c.hi; ++e)
                a.param[pi + e] = uint16_t(to_bf16x2(a.master[c.k0 + e], 0.0f));
        }
    }
}

// ---- parameter all-gather ---------------------------------------------------------------------
// One tile space over every rank range of every padded bucket, with no empty
// tiles: tile -> range through the kTileGroup index, then the range's own
// entry. A tile is kGatherTile elements from the range's start rounded down
// to 64; lane l takes the chunks l, l + 64, l + 128, l + 192 (8 elements
// each), so each load instruction covers 1 KiB and the tile's four loads
// are in flight together. A range whose source is `out` itself is already
// in place and is skipped. Every byte is read once and written once:
// non-temporal loads and stores, as in the copy.
constexpr int kGatherChunks = int(kGatherTile / kTileElems);   // chunks per lane

__global__ __launch_bounds__(kBlock) void gather_kernel(GatherArgs a) {
    for (int64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
        int64_t y = ro(a.group)[tile / kTileGroup];
        while (y + 1 < a.nranges && ro(a.ranges)[y + 1].tile0 <= tile)
            ++y;
        const ro_ptr<RangeSpan> rp = ro(a.ranges) + y;
        const RangeSpan r = {rp->rb, rp->re, rp->tile0, rp->src};
        const uint16_t *src = a.src[r.src];
        if (src == a.out)
            continue;
        const int64_t base = tile_origin(r.rb) + (tile - r.tile0) * kGatherTile;
        u32x4 v[kGatherChunks];
        bool whole[kGatherChunks];
#pragma unroll
        for (int c = 0; c < kGatherChunks; ++c) {
            const int64_t w0 = base + (int64_t(c) * kBlock + threadIdx.x) * kChunk;
            whole[c] = w0 >= r.rb && w0 + kChunk <= r.re;
            if (whole[c])
                v[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src + w0));
        }
#pragma unroll
        for (int c = 0; c < kGatherChunks; ++c) {
            const int64_t w0 = base + (int64_t(c) * kBlock + threadIdx.x) * kChunk;
            if (whole[c]) {
                __builtin_nontemporal_store(v[c], reinterpret_cast<u32x4 *>(a.out + w0));
            } else {
                for (int64_t w = w0 > r.rb ? w0 : r.rb; w < w0 + kChunk && w < r.re; ++w)
                    a.out[w] = src[w];
            }
        }
    }
}

// The step's stream shape with trivial arithmetic (a measurement reference):
// per 512-element tile, D bf16 streams read by 16-byte chunks, three fp32
// streams read by two quads per lane, every access non-temporal as in the
// step on a large shard. kStores selects what is stored (include/zdo.h,
// ZDO_PROBE_STORE_*): the step's stores (the state rewritten, gaining the
// exponent bits of the lane's XOR of its chunks, and the bf16 stream
// written), the bf16 stream only, or one word per tile. Every loaded byte
// feeds a stored one, so no load can be dropped or narrowed. The occupancy
// bounds are the step's, so that the compiler likewise issues every load of
// a tile before the first wait.
template <int D, int kStores>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(D >= 32 ? 2 : 1, D < 32 ? 4 : 3)))
void probe_kernel(ProbeArgs a) {
    const int lane = int(threadIdx.x);
    for (int64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
        const int64_t kb = tile * kTileElems;
        f32x4 s[2][3];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 3; ++i)
                s[h][i] = ld_state<true>(a.state[i] + kb + h * (kTileElems / 2) + 4 * lane);
        u32x4 r[D];
#pragma unroll
        for (int j = 0; j < D; ++j)
            r[j] = ld_rep(a.rep[j] + kb + int64_t(kChunk) * lane);
        u32x4 x = r[0];
#pragma unroll
        for (int j = 1; j < D; ++j)
            x ^= r[j];
        if constexpr (kStores == ZDO_PROBE_STORE_ALL) {
            const float f = __uint_as_float((x[0] ^ x[1] ^ x[2] ^ x[3]) & 0x3f000000u);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int i = 0; i < 3; ++i)
                    st_state<true>(a.state[i] + kb + h * (kTileElems / 2) + 4 * lane, s[h][i] + f);
                st8_out(a.out + kb + h * (kTileElems / 2) + 4 * lane,
                        u32x2{__float_as_uint(s[h][0][0]) ^ x[2 * h], __float_as_uint(s[h][1][1]) ^ x[2 * h + 1]});
            }
        } else {
            uint32_t sx[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                sx[h] = 0;
#pragma unroll
                for (int i = 0; i < 3; ++i)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        sx[h] ^= __float_as_uint(s[h][i][c]);
            }
            if constexpr (kStores == ZDO_PROBE_STORE_OUT) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    st8_out(a.out + kb + h * (kTileElems / 2) + 4 * lane, u32x2{x[2 * h] ^ sx[h], x[2 * h + 1] ^ sx[h]});
            } else {
                uint32_t v = x[0] ^ x[1] ^ x[2] ^ x[3] ^ sx[0] ^ sx[1];
#pragma unroll
                for (int off = 32; off > 0; off >>= 1)
                    v ^= uint32_t(__shfl_xor(int(v), off, 64));
                if (lane == 0)
                    *reinterpret_cast<uint32_t *>(a.out + 2 * tile) = v;
            }
        }
    }
}

__global__ __launch_bounds__(kBlock) void copy_kernel(u32x4 *dst, const u32x4 *src, int64_t n16) {
    for (int64_t i = int64_t(blockIdx.x) * kBlock + threadIdx.x; i < n16; i += int64_t(gridDim.x) * kBlock)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Enough blocks to cover every tile once, up to a cap that keeps the grid's
// work-item count in range; larger launches loop over tiles (every kernel's
// tile loop steps by gridDim.x). A build with a small cap makes every
// launch take that loop.
#ifndef ZDO_MAX_GRID
#define ZDO_MAX_GRID (int64_t(1) << 24)
#endif
constexpr int64_t kMaxGrid = ZDO_MAX_GRID;
static_assert(kMaxGrid >= 1 && kMaxGrid <= (int64_t(1) << 24), "grid cap out of range");

unsigned grid_for(int64_t ntiles) {
    return unsigned(ntiles < kMaxGrid ? ntiles : kMaxGrid);
}

// HBM serves a long stream of many read and write streams at a higher rate
// when fewer waves share a compute unit (measured on the 42 GB
// Llama-3-8B-shaped step: 5.32 TB/s uncapped, 5.69 TB/s at 10 waves per
// compute unit, 5.66 at 8, 5.55 at 14), while a short launch, a few dozen
// rounds of workgroups over the chip, finishes sooner with more waves in
// flight (GPT-2-shaped step, 30k tiles: 106 us at 10 waves per compute unit,
// 102 us at 16; its clipped step 92 us at 10, 78 us at 16). The launch
// reserves LDS it never uses so that at most `long_waves` waves (by default
// ZDO_WAVES_PER_CU), or ZDO_WAVES_PER_CU_SHORT for launches of fewer than
// kShortLaunchTiles tiles, fit on one compute unit. A step with a fixed
// number (2 to 32) of contributions has every load of a tile in flight at
// once and needs fewer waves to cover the latency: its long launches take
// ZDO_STEP_WAVES_PER_CU.
#ifndef ZDO_WAVES_PER_CU
#define ZDO_WAVES_PER_CU 10
#endif
#ifndef ZDO_WAVES_PER_CU_SHORT
#define ZDO_WAVES_PER_CU_SHORT 16
#endif
#ifndef ZDO_STEP_WAVES_PER_CU
#define ZDO_STEP_WAVES_PER_CU 6
#endif
// force_all_reduce walks the whole buffer flat. Its long launches do best
// with 8 waves per compute unit at 8 contributions (GPT-2-shaped buffer:
// 344-345 us at 10, 335-338 at 8, 358-362 at 7) and with 7 at 16
// (fragmentation workload: 414-415 us at 10, 413-414 at 8, 394-395 at 7).
constexpr int flat_waves(int nrep) { return nrep >= 16 ? 7 : 8; }

// LDS per workgroup that lets at most `waves` waves share a compute unit.
unsigned lds_for_waves(int lds_per_cu, int waves) {
    if (waves <= 0 || lds_per_cu <= 0)
        return 0;
    const int waves_per_group = kBlock / 64;
    int groups = waves / waves_per_group;
    if (groups < 4 / waves_per_group + (waves_per_group > 4))
        groups = 4 / waves_per_group + (waves_per_group > 4);
    return unsigned(lds_per_cu / groups) & ~127u;
}

unsigned lds_reserve(int lds_per_cu, int64_t ntiles, int long_waves = ZDO_WAVES_PER_CU) {
    return lds_for_waves(lds_per_cu, ntiles < kShortLaunchTiles ? ZDO_WAVES_PER_CU_SHORT : long_waves);
}

// The all-gather's tiles read 4 KiB each. With at most 12 waves per compute
// unit, short launches and long ones alike ran as fast as uncapped or
// faster (fragmentation workload 51.3-51.6 -> 49.1-49.8 us, Llama-3-8B
// shape 4.56-4.62 -> 4.45-4.47 ms, GPT-2 shape 70.1-70.6 -> 70.3-70.5 us;
// 8 waves: 5-10% slower, 16 and 24: between the two).
constexpr int kGatherWaves = 12;

}  // namespace

hipError_t launch_reduce(const ReduceArgs &a, int lds_per_cu, hipStream_t stream) {
    if (a.walk.ntiles <= 0)
        return hipSuccess;
    const dim3 grid(grid_for(a.walk.ntiles)), block(kBlock);
    const unsigned lds =
        lds_reserve(lds_per_cu, a.walk.ntiles, a.walk.segs ? ZDO_WAVES_PER_CU : flat_waves(a.nrep));
    switch (a.nrep) {
    case 1: hipLaunchKernelGGL(reduce_kernel<1>, grid, block, lds, stream, a); break;
    case 2: hipLaunchKernelGGL(reduce_kernel<2>, grid, block, lds, stream, a); break;
    case 4: hipLaunchKernelGGL(reduce_kernel<4>, grid, block, lds, stream, a); break;
    case 8: hipLaunchKernelGGL(reduce_kernel<8>, grid, block, lds, stream, a); break;
    case 16: hipLaunchKernelGGL(reduce_kernel<16>, grid, block, lds, stream, a); break;
    case 32: hipLaunchKernelGGL(reduce_kernel<32>, grid, block, lds, stream, a); break;
    default: hipLaunchKernelGGL(reduce_kernel<0>, grid, block, lds, stream, a); break;
    }
    return hipGetLastError();
}

// The fp32 state goes non-temporal above 1 GiB (12 bytes per shard slot).
// Measured on one box, plain -> non-temporal state, step time with cold
// caches (back to back in brackets): 187 MB 102 -> 112 us (97 -> 109),
// 299 MB 148 -> 159 us (150 -> 155), 498 MB 209 -> 218 us (235 -> 216),
// 747 MB 296 -> 308 us (323 -> 307), 1.49 GB 582 -> 562 us (603 -> 565),
// 3.0 GB 4.09 -> 3.99 ms, 6.0 GB 4.91 -> 4.73 ms, 12 GB 6.96 -> 6.76 ms.
// Between steps of a training run the caches are cold, and there
// non-temporal accesses pay off once the state is well beyond the 256 MB
// Infinity Cache.
#ifndef ZDO_STATE_CACHE_BYTES
#define ZDO_STATE_CACHE_BYTES (int64_t(1) << 30)
#endif

template <bool kNT>
void launch_step_as(const StepArgs &a, dim3 grid, dim3 block, unsigned lds, hipStream_t stream) {
    // One contribution per instance is the plain sum over the instances: the
    // inner rounding of a single bf16 term changes nothing.
    if (a.ninst > 1 && a.dinst > 1) {
        switch (a.dinst) {
        case 2: hipLaunchKernelGGL((step_kernel<2, true, kNT>), grid, block, lds, stream, a); break;
        case 4: hipLaunchKernelGGL((step_kernel<4, true, kNT>), grid, block, lds, stream, a); break;
        case 8: hipLaunchKernelGGL((step_kernel<8, true, kNT>), grid, block, lds, stream, a); break;
        case 16: hipLaunchKernelGGL((step_kernel<16, true, kNT>), grid, block, lds, stream, a); break;
        case 32: hipLaunchKernelGGL((step_kernel<32, true, kNT>), grid, block, lds, stream, a); break;
        default: hipLaunchKernelGGL((step_kernel<0, true, kNT>), grid, block, lds, stream, a); break;
        }
        return;
    }
    switch (a.nrep) {
    case 1: hipLaunchKernelGGL((step_kernel<1, false, kNT>), grid, block, lds, stream, a); break;
    case 2: hipLaunchKernelGGL((step_kernel<2, false, kNT>), grid, block, lds, stream, a); break;
    case 4: hipLaunchKernelGGL((step_kernel<4, false, kNT>), grid, block, lds, stream, a); break;
    case 8: hipLaunchKernelGGL((step_kernel<8, false, kNT>), grid, block, lds, stream, a); break;
    case 16: hipLaunchKernelGGL((step_kernel<16, false, kNT>), grid, block, lds, stream, a); break;
    case 32: hipLaunchKernelGGL((step_kernel<32, false, kNT>), grid, block, lds, stream, a); break;
    default: hipLaunchKernelGGL((step_kernel<0, false, kNT>), grid, block, lds, stream, a); break;
    }
}

hipError_t launch_step(const StepArgs &a, int lds_per_cu, hipStream_t stream) {
    if (a.walk.ntiles <= 0)
        return hipSuccess;
    const dim3 grid(grid_for(a.walk.ntiles)), block(kBlock);
    const int d = a.ninst > 1 && a.dinst > 1 ? a.dinst : a.nrep;   // the template's D
    const bool fixed = d == 2 || d == 4 || d == 8 || d == 16 || d == 32;
    const unsigned lds = lds_reserve(lds_per_cu, a.walk.ntiles, fixed ? ZDO_STEP_WAVES_PER_CU : ZDO_WAVES_PER_CU);
    if (a.state_numel * int64_t(3 * sizeof(float)) > ZDO_STATE_CACHE_BYTES)
        launch_step_as<true>(a, grid, block, lds, stream);
    else
        launch_step_as<false>(a, grid, block, lds, stream);
    return hipGetLastError();
}

hipError_t launch_writeback(const WritebackArgs &a, hipStream_t stream) {
    if (a.walk.ntiles <= 0)
        return hipSuccess;
    // A tile moves 3 KiB: no occupancy cap, so that enough bytes are in
    // flight (Llama-3-8B shape, non-temporal master: 1150 us at 16 waves
    // per compute unit, 966 at 24, 964-967 uncapped; GPT-2 shape, plain
    // loads: 17.2 us at 16, 15.5 uncapped). The master array goes
    // non-temporal on the step's rule (Llama-3-8B uncapped: 1004-1007 us
    // with plain loads; GPT-2: 16.2 us with non-temporal ones).
    const dim3 grid(grid_for(a.walk.ntiles)), block(kBlock);
    if (a.state_numel * int64_t(3 * sizeof(float)) > ZDO_STATE_CACHE_BYTES)
        hipLaunchKernelGGL(writeback_kernel<true>, grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL(writeback_kernel<false>, grid, block, 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_norm(const NormArgs &a, double *norm_sq, int lds_per_cu, hipStream_t stream) {
    if (a.walk.ntiles > 0) {
        const dim3 grid(grid_for(a.walk.ntiles)), block(kBlock);
        const unsigned lds = lds_reserve(lds_per_cu, a.walk.ntiles);
        switch (a.nrep) {
        case 1: hipLaunchKernelGGL(norm_kernel<1>, grid, block, lds, stream, a); break;
        case 2: hipLaunchKernelGGL(norm_kernel<2>, grid, block, lds, stream, a); break;
        case 4: hipLaunchKernelGGL(norm_kernel<4>, grid, block, lds, stream, a); break;
        case 8: hipLaunchKernelGGL(norm_kernel<8>, grid, block, lds, stream, a); break;
        case 16: hipLaunchKernelGGL(norm_kernel<16>, grid, block, lds, stream, a); break;
        case 32: hipLaunchKernelGGL(norm_kernel<32>, grid, block, lds, stream, a); break;
        default: hipLaunchKernelGGL(norm_kernel<0>, grid, block, lds, stream, a); break;
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    // level 1: G <= kSumGroups runs of `chunk` partials; level 2: one workgroup
    const int64_t n = a.walk.ntiles;
    int64_t g = (n + kSumThreads - 1) / kSumThreads;
    if (g > kSumGroups)
        g = kSumGroups;
    if (g < 1)
        g = 1;
    const int64_t chunk = n > 0 ? (n + g - 1) / g : 1;
    double *level = a.partial + (n > 0 ? n : 0);
    hipLaunchKernelGGL(tile_sum_kernel, dim3(unsigned(g)), dim3(kSumThreads), 0, stream, a.partial, n, chunk, level);
    hipLaunchKernelGGL(level_sum_kernel, dim3(1), dim3(kSumThreads), 0, stream, level, g, norm_sq);
    return hipGetLastError();
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device, once looked up
}  // namespace

hipError_t no_alloc_scratch(void **out) {
    *out = nullptr;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_clip(const double *parts, int32_t n, float max_norm, float *coeff, double *norm_out,
                       hipStream_t stream) {
    hipLaunchKernelGGL(clip_kernel, dim3(1), dim3(64), 0, stream, parts, n, max_norm, coeff, norm_out);
    return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs &a, int lds_per_cu, hipStream_t stream) {
    if (a.ntiles <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(gather_kernel, dim3(grid_for(a.ntiles)), dim3(kBlock), lds_for_waves(lds_per_cu, kGatherWaves),
                       stream, a);
    return hipGetLastError();
}

hipError_t launch_probe(const ProbeArgs &a, int waves_per_cu, int lds_per_cu, hipStream_t stream) {
    if (a.ntiles <= 0)
        return hipSuccess;
    const dim3 grid(grid_for(a.ntiles)), block(kBlock);
    const unsigned lds = lds_for_waves(lds_per_cu, waves_per_cu);
    switch (a.nrep * 4 + a.stores) {
    case 8 * 4 + ZDO_PROBE_STORE_ALL: hipLaunchKernelGGL((probe_kernel<8, ZDO_PROBE_STORE_ALL>), grid, block, lds, stream, a); break;
    case 8 * 4 + ZDO_PROBE_STORE_OUT: hipLaunchKernelGGL((probe_kernel<8, ZDO_PROBE_STORE_OUT>), grid, block, lds, stream, a); break;
    case 8 * 4 + ZDO_PROBE_STORE_NONE: hipLaunchKernelGGL((probe_kernel<8, ZDO_PROBE_STORE_NONE>), grid, block, lds, stream, a); break;
    case 16 * 4 + ZDO_PROBE_STORE_ALL: hipLaunchKernelGGL((probe_kernel<16, ZDO_PROBE_STORE_ALL>), grid, block, lds, stream, a); break;
    case 16 * 4 + ZDO_PROBE_STORE_OUT: hipLaunchKernelGGL((probe_kernel<16, ZDO_PROBE_STORE_OUT>), grid, block, lds, stream, a); break;
    case 16 * 4 + ZDO_PROBE_STORE_NONE: hipLaunchKernelGGL((probe_kernel<16, ZDO_PROBE_STORE_NONE>), grid, block, lds, stream, a); break;
    case 32 * 4 + ZDO_PROBE_STORE_ALL: hipLaunchKernelGGL((probe_kernel<32, ZDO_PROBE_STORE_ALL>), grid, block, lds, stream, a); break;
    case 32 * 4 + ZDO_PROBE_STORE_OUT: hipLaunchKernelGGL((probe_kernel<32, ZDO_PROBE_STORE_OUT>), grid, block, lds, stream, a); break;
    case 32 * 4 + ZDO_PROBE_STORE_NONE: hipLaunchKernelGGL((probe_kernel<32, ZDO_PROBE_STORE_NONE>), grid, block, lds, stream, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_copy(void *dst, const void *src, int64_t n16, hipStream_t stream) {
    if (n16 <= 0)
        return hipSuccess;
    const int64_t blocks = (n16 + kBlock - 1) / kBlock;
    hipLaunchKernelGGL(copy_kernel, dim3(grid_for(blocks)), dim3(kBlock), 0, stream, static_cast<u32x4 *>(dst),
                       static_cast<const u32x4 *>(src), n16);
    return hipGetLastError();
}

}  // namespace zdo
