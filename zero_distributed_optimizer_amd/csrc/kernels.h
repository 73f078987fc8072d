// Launch arguments and launchers of the device kernels (kernels.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "zdo_internal.h"

namespace zdo {

// Adam constants of one step, formed on the host (see abi.cpp).
struct AdamConst {
    float lr, b1, b2, omb1, omb2, eps, wd, bc1, bc2;
};

// Disjoint runs of tiles one launch may walk (a list of bucket ranges ready
// together).
constexpr int kMaxTileRuns = 16;

// Segments walked by a launch: either a table (nseg segments and their
// kTileGroup index) or, when segs is NULL, the single run [0, flat_numel).
// The launch takes ntiles tiles of that tile space: launch index i in
// [run_start[r], run_start[r + 1]) is tile run_begin[r] + (i - run_start[r]),
// for the nruns runs (run_start[0] = 0; one run: tiles [run_begin[0],
// run_begin[0] + ntiles)).
struct Walk {
    const Seg *segs;
    const GroupSeg *group;
    int64_t nseg;
    int64_t ntiles;      // tiles in this launch
    int64_t flat_numel;
    int32_t nruns;
    int64_t run_begin[kMaxTileRuns];
    int64_t run_start[kMaxTileRuns];
};

// A walk over the one run [first, first + count) of a tile space.
inline Walk one_run(const Seg *segs, const GroupSeg *group, int64_t nseg, int64_t first, int64_t count,
                    int64_t flat_numel = 0) {
    Walk w{};
    w.segs = segs;
    w.group = group;
    w.nseg = nseg;
    w.ntiles = count;
    w.flat_numel = flat_numel;
    w.nruns = 1;
    w.run_begin[0] = first;
    w.run_start[0] = 0;
    return w;
}

struct ReduceArgs {
    Walk walk;
    const uint16_t *rep[ZDO_MAX_REPLICAS];
    int32_t nrep;
    int32_t in_local;    // replicas indexed by LOCAL (1) or WORLD (0) position
    int32_t out_local;
    float scale;
    uint16_t *out;
};

struct StepArgs {
    Walk walk;
    const uint16_t *rep[ZDO_MAX_REPLICAS];
    int32_t nrep;
    // Several optimizer instances: rep holds ninst groups of dinst
    // contributions (nrep = ninst * dinst), reduced within each group first.
    // ninst = 1, dinst = nrep for the plain step.
    int32_t ninst;
    int32_t dinst;
    int32_t in_local;
    int32_t param_local;
    float scale;
    float *master, *m, *v;
    uint16_t *param;     // may be NULL
    float *main_grad;    // may be NULL
    const float *coeff;  // device clipping coefficient, or NULL for none
    int64_t state_numel; // L: the master/m/v arrays' length (selects their cache policy)
    AdamConst c;
};

struct NormArgs {
    Walk walk;
    const uint16_t *rep[ZDO_MAX_REPLICAS];
    int32_t nrep;
    int32_t in_local;
    int32_t out_local;
    float scale;
    uint16_t *out;       // reduced gradient at the owned elements, or NULL
    double *partial;     // one per tile of walk
};

// The all-gather of the parameter buffers: every rank range of every padded
// bucket copied from its rank's buffer into out, except ranges whose source
// is out itself.
struct GatherArgs {
    const RangeSpan *ranges;
    const uint32_t *group;   // range at the first tile of every kTileGroup tiles
    int64_t nranges;         // buckets x D
    int64_t ntiles;
    const uint16_t *src[ZDO_MAX_REPLICAS];
    uint16_t *out;
};

struct WritebackArgs {
    Walk walk;
    int32_t param_local;
    const float *master;
    uint16_t *param;
    int64_t state_numel;  // L: the master array's length (selects its cache policy)
};

// The step's stream shape with trivial arithmetic (zdo_stream_probe): ntiles
// tiles of 512 elements of nrep bf16 streams (read), three fp32 streams (read,
// and rewritten with ZDO_PROBE_STORE_ALL) and one bf16 stream (written with
// ZDO_PROBE_STORE_ALL or _OUT; one word per tile with _NONE).
struct ProbeArgs {
    const uint16_t *rep[ZDO_MAX_REPLICAS];
    int32_t nrep;
    int32_t stores;      // ZDO_PROBE_STORE_*
    float *state[3];
    uint16_t *out;
    int64_t ntiles;
};

// lds_per_cu: LDS bytes per compute unit of the launch device (0 if unknown),
// used to cap how many workgroups share a compute unit.
hipError_t launch_reduce(const ReduceArgs &a, int lds_per_cu, hipStream_t stream);
hipError_t launch_step(const StepArgs &a, int lds_per_cu, hipStream_t stream);
hipError_t launch_writeback(const WritebackArgs &a, hipStream_t stream);
hipError_t launch_copy(void *dst, const void *src, int64_t n16, hipStream_t stream);
// waves_per_cu: occupancy cap (0: none).
hipError_t launch_probe(const ProbeArgs &a, int waves_per_cu, int lds_per_cu, hipStream_t stream);
hipError_t launch_gather(const GatherArgs &a, int lds_per_cu, hipStream_t stream);
// Squared norm: per-tile partials into a.partial, then their fixed-order sum
// into *norm_sq (0 when a.walk has no tiles).
hipError_t launch_norm(const NormArgs &a, double *norm_sq, int lds_per_cu, hipStream_t stream);
hipError_t launch_clip(const double *parts, int32_t n, float max_norm, float *coeff, double *norm_out,
                       hipStream_t stream);
// Device address of the library's static scratch array on the current
// device (ZDO_NO_ALLOC_SCRATCH_BYTES bytes), looked up once per device.
hipError_t no_alloc_scratch(void **out);

}  // namespace zdo
