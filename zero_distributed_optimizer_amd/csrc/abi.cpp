// The C-ABI of libzdo: argument checks, the host-side Adam constants and the
// launches. Declared and documented in include/zdo.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "kernels.h"
#include "zdo_internal.h"

namespace zdo {

int build_plan(const int64_t *param_numel, int32_t n_params, int64_t bucket_numel, int32_t dp_size,
               int32_t rank, zdo_plan &p);
int upload_plan(zdo_plan &p);

namespace {

thread_local std::string g_error;

struct Span {
    uintptr_t lo, hi;
};

Span span_of(const void *p, int64_t elems, int64_t elem_bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return {lo, lo + uintptr_t(elems) * uintptr_t(elem_bytes)};
}

bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi && a.lo < a.hi && b.lo < b.hi; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool aligned_to(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int fail(int code, const std::string &msg) {
    g_error = msg;
    return code;
}

// The plan must be device-ready, and on the current device.
int check_plan(const zdo_plan *plan, const char *fn) {
    if (!plan)
        return fail(ZDO_EINVAL, std::string(fn) + ": plan is NULL");
    if (!plan->d_table)
        return fail(ZDO_EHIP, std::string(fn) + ": the plan has no device table (no HIP device when it was built)");
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess)
        return fail(ZDO_EHIP, std::string(fn) + ": hipGetDevice failed");
    if (dev != plan->device)
        return fail(ZDO_EINVAL, std::string(fn) + ": the plan was built on device " + std::to_string(plan->device) +
                                    " but device " + std::to_string(dev) + " is current");
    return ZDO_OK;
}

int check_coords(int32_t c, const char *fn, const char *what) {
    if (c != ZDO_WORLD && c != ZDO_LOCAL)
        return fail(ZDO_EINVAL, std::string(fn) + ": " + what + " must be ZDO_WORLD or ZDO_LOCAL");
    return ZDO_OK;
}

int check_ptr(const void *p, const char *fn, const char *what) {
    if (!p)
        return fail(ZDO_EINVAL, std::string(fn) + ": " + what + " is NULL");
    if (!aligned16(p))
        return fail(ZDO_EALIGN, std::string(fn) + ": " + what + " is not 16-byte aligned");
    return ZDO_OK;
}

int64_t extent(const zdo_plan *p, int32_t coords) { return coords == ZDO_WORLD ? p->buffer_numel : p->shard_numel; }

int launch_result(hipError_t e, const char *fn) {
    if (e != hipSuccess)
        return fail(ZDO_EHIP, std::string(fn) + ": launch failed: " + hipGetErrorString(e));
    return ZDO_OK;
}

// Checks the replica list; fills `rep`.
int take_replicas(const zdo_plan *p, const uint16_t *const *replicas, int32_t n, int32_t coords, const char *fn,
                  const uint16_t *rep[ZDO_MAX_REPLICAS], Span spans[ZDO_MAX_REPLICAS]) {
    if (!replicas)
        return fail(ZDO_EINVAL, std::string(fn) + ": replica list is NULL");
    for (int32_t j = 0; j < n; ++j) {
        const std::string what = "replica " + std::to_string(j);
        if (int rc = check_ptr(replicas[j], fn, what.c_str()))
            return rc;
        rep[j] = replicas[j];
        spans[j] = span_of(replicas[j], extent(p, coords), 2);
    }
    return ZDO_OK;
}

// 1 - beta^t: the double 1.0 multiplied t times by (double)beta, rounded once
// to fp32 (beta in [0, 1)). Once beta^t < 2^-60, 1 - beta^t is 1.0 in double
// and stays so for every larger t, so the products stop there. The last
// (beta, t, product) of a few betas is kept per thread, so that consecutive
// steps cost O(1).
float bias_correction(float beta, int64_t t) {
    struct Entry {
        float beta;
        int64_t t;
        double pw;
    };
    thread_local Entry cache[4] = {{-1.0f, 0, 1.0}, {-1.0f, 0, 1.0}, {-1.0f, 0, 1.0}, {-1.0f, 0, 1.0}};
    thread_local unsigned next = 0;
    Entry *e = nullptr;
    for (auto &c : cache)
        if (c.beta == beta && c.t <= t)
            e = &c;
    double pw = 1.0;
    int64_t i = 0;
    if (e) {
        pw = e->pw;
        i = e->t;
    } else {
        e = &cache[next++ % 4];
    }
    for (; i < t && pw >= 0x1p-60; ++i)
        pw *= double(beta);
    *e = {beta, t, pw};
    return float(1.0 - pw);
}

// Tiles [first, first + count) of a launch space that cover buckets [b0, b1):
// segs are in bucket order, seg_bucket[i] is segment i's bucket (NULL: i).
void bucket_tiles(const std::vector<Seg> &segs, const int32_t *seg_bucket, int64_t total_tiles, int32_t b0,
                  int32_t b1, int64_t &first, int64_t &count) {
    const int64_t n = int64_t(segs.size());
    auto first_seg_at = [&](int32_t b) {
        int64_t lo = 0, hi = n;   // first i with bucket(i) >= b
        while (lo < hi) {
            const int64_t mid = (lo + hi) / 2;
            if ((seg_bucket ? seg_bucket[mid] : int32_t(mid)) < b)
                lo = mid + 1;
            else
                hi = mid;
        }
        return lo < n ? segs[size_t(lo)].tile0 : total_tiles;
    };
    first = first_seg_at(b0);
    count = first_seg_at(b1) - first;
}

int check_buckets(const zdo_plan *plan, int32_t b0, int32_t b1, const char *fn) {
    if (b0 < 0 || b1 < b0 || b1 > int32_t(plan->buckets.size()))
        return fail(ZDO_EINVAL, std::string(fn) + ": need 0 <= bucket_begin <= bucket_end <= " +
                                    std::to_string(plan->buckets.size()));
    return ZDO_OK;
}

typedef std::pair<int32_t, int32_t> BucketRange;

// n (begin, end) pairs: each within [0, number of buckets], pairwise
// disjoint; sorted by begin into `out`, empty ranges dropped.
int check_bucket_list(const zdo_plan *plan, const int32_t *pairs, int32_t n, const char *fn,
                      std::vector<BucketRange> &out) {
    if (n < 0 || (n > 0 && !pairs))
        return fail(ZDO_EINVAL, std::string(fn) + ": need n_ranges >= 0 and a range array");
    out.clear();
    for (int64_t i = 0; i < n; ++i) {
        const int32_t b0 = pairs[2 * i], b1 = pairs[2 * i + 1];
        if (int rc = check_buckets(plan, b0, b1, fn))
            return rc;
        if (b0 < b1)
            out.emplace_back(b0, b1);
    }
    std::sort(out.begin(), out.end());
    for (size_t i = 1; i < out.size(); ++i)
        if (out[i].first < out[i - 1].second)
            return fail(ZDO_EINVAL, std::string(fn) + ": bucket ranges [" + std::to_string(out[i - 1].first) + ", " +
                                        std::to_string(out[i - 1].second) + ") and [" +
                                        std::to_string(out[i].first) + ", " + std::to_string(out[i].second) +
                                        ") overlap");
    return ZDO_OK;
}

struct TileRun {
    int64_t first, count;
};

// The tile runs of a launch space that cover sorted, disjoint bucket ranges;
// runs that touch are merged and empty ones dropped.
std::vector<TileRun> tile_runs(const std::vector<Seg> &segs, const int32_t *seg_bucket, int64_t total_tiles,
                               const std::vector<BucketRange> &ranges) {
    std::vector<TileRun> runs;
    for (const BucketRange &b : ranges) {
        int64_t first = 0, count = 0;
        bucket_tiles(segs, seg_bucket, total_tiles, b.first, b.second, first, count);
        if (count <= 0)
            continue;
        if (!runs.empty() && runs.back().first + runs.back().count == first)
            runs.back().count += count;
        else
            runs.push_back({first, count});
    }
    return runs;
}

// Launch walks over the runs, up to kMaxTileRuns runs each; `launch` takes a
// Walk and returns the launch's hipError_t.
template <typename F>
int launch_runs(const std::vector<TileRun> &runs, const Seg *segs, const GroupSeg *group, int64_t nseg,
                const char *fn, F launch) {
    for (size_t c = 0; c < runs.size(); c += kMaxTileRuns) {
        Walk w{};
        w.segs = segs;
        w.group = group;
        w.nseg = nseg;
        const size_t n = std::min(runs.size() - c, size_t(kMaxTileRuns));
        w.nruns = int32_t(n);
        int64_t start = 0;
        for (size_t r = 0; r < n; ++r) {
            w.run_begin[r] = runs[c + r].first;
            w.run_start[r] = start;
            start += runs[c + r].count;
        }
        w.ntiles = start;
        if (int rc = launch_result(launch(w), fn))
            return rc;
    }
    return ZDO_OK;
}

}  // namespace

void set_error(const std::string &msg) { g_error = msg; }

}  // namespace zdo

using namespace zdo;

extern "C" {

const char *zdo_last_error(void) { return g_error.c_str(); }

int build_range_map(const int64_t *param_numel, int32_t n_params, int64_t bucket_numel, int32_t dp_size,
                    int32_t rank, zdo_plan **out) {
    if (!out)
        return fail(ZDO_EINVAL, "build_range_map: out is NULL");
    *out = nullptr;
    zdo_plan *p = new (std::nothrow) zdo_plan();
    if (!p)
        return fail(ZDO_ENOMEM, "build_range_map: out of host memory");
    int rc;
    try {
        rc = build_plan(param_numel, n_params, bucket_numel, dp_size, rank, *p);
        if (rc == ZDO_OK)
            rc = upload_plan(*p);
    } catch (const std::bad_alloc &) {
        rc = fail(ZDO_ENOMEM, "build_range_map: out of host memory");
    }
    if (rc != ZDO_OK) {
        zdo_plan_destroy(p);
        return rc;
    }
    *out = p;
    return ZDO_OK;
}

void zdo_plan_destroy(zdo_plan *plan) {
    if (!plan)
        return;
    if (plan->d_table)
        (void)hipFree(plan->d_table);
    delete plan;
}

int64_t zdo_plan_buffer_numel(const zdo_plan *p) { return p ? p->buffer_numel : -1; }
int64_t zdo_plan_shard_numel(const zdo_plan *p) { return p ? p->shard_numel : -1; }
int64_t zdo_plan_owned_numel(const zdo_plan *p) { return p ? p->owned_numel : -1; }
int32_t zdo_plan_dp_size(const zdo_plan *p) { return p ? p->dp_size : -1; }
int32_t zdo_plan_rank(const zdo_plan *p) { return p ? p->rank : -1; }

int zdo_plan_buckets(const zdo_plan *p, zdo_bucket *out, int32_t cap, int32_t *n) {
    if (!p || !n)
        return fail(ZDO_EINVAL, "zdo_plan_buckets: plan or n is NULL");
    *n = int32_t(p->buckets.size());
    if (out && cap >= *n)
        for (int32_t i = 0; i < *n; ++i)
            out[i] = p->buckets[size_t(i)];
    return ZDO_OK;
}

int zdo_plan_pieces(const zdo_plan *p, zdo_piece *out, int64_t cap, int64_t *n) {
    if (!p || !n)
        return fail(ZDO_EINVAL, "zdo_plan_pieces: plan or n is NULL");
    *n = int64_t(p->pieces.size());
    if (out && cap >= *n)
        for (int64_t i = 0; i < *n; ++i)
            out[i] = p->pieces[size_t(i)];
    return ZDO_OK;
}

int plan_buckets(const zdo_plan *p, zdo_bucket *out, int32_t cap, int32_t *n) {
    return zdo_plan_buckets(p, out, cap, n);
}
int plan_pieces(const zdo_plan *p, zdo_piece *out, int64_t cap, int64_t *n) {
    return zdo_plan_pieces(p, out, cap, n);
}
int64_t plan_buffer_numel(const zdo_plan *p) { return zdo_plan_buffer_numel(p); }
int64_t plan_shard_numel(const zdo_plan *p) { return zdo_plan_shard_numel(p); }
void plan_destroy(zdo_plan *p) { zdo_plan_destroy(p); }

static int reduce_scatter_impl(const char *fn, const zdo_plan *plan, const std::vector<BucketRange> &ranges,
                               const uint16_t *const *replicas, int32_t n_replicas, int32_t replica_coords,
                               float scale, uint16_t *out, int32_t out_coords, void *stream) {
    if (n_replicas < 1 || n_replicas > ZDO_MAX_REPLICAS)
        return fail(ZDO_EINVAL, std::string(fn) + ": n_replicas must be in [1, " + std::to_string(ZDO_MAX_REPLICAS) +
                                    "]");
    if (int rc = check_coords(replica_coords, fn, "replica_coords"))
        return rc;
    if (int rc = check_coords(out_coords, fn, "out_coords"))
        return rc;
    ReduceArgs a{};
    Span spans[ZDO_MAX_REPLICAS];
    if (int rc = take_replicas(plan, replicas, n_replicas, replica_coords, fn, a.rep, spans))
        return rc;
    if (int rc = check_ptr(out, fn, "out"))
        return rc;
    const Span so = span_of(out, extent(plan, out_coords), 2);
    for (int32_t j = 0; j < n_replicas; ++j)
        if (overlap(so, spans[j]) && !(out == replicas[j] && out_coords == replica_coords))
            return fail(ZDO_EALIAS, std::string(fn) + ": out overlaps replica " + std::to_string(j) +
                                        " without coinciding with it");
    a.nrep = n_replicas;
    a.in_local = replica_coords == ZDO_LOCAL;
    a.out_local = out_coords == ZDO_LOCAL;
    a.scale = scale;
    a.out = out;
    const std::vector<TileRun> runs = tile_runs(plan->range_segs, nullptr, plan->range_tiles, ranges);
    return launch_runs(runs, plan->d_range_segs, plan->d_range_group, int64_t(plan->range_segs.size()), fn,
                       [&](const Walk &w) {
                           a.walk = w;
                           return launch_reduce(a, plan->lds_per_cu, static_cast<hipStream_t>(stream));
                       });
}

static std::vector<BucketRange> all_buckets(const zdo_plan *plan) {
    return {BucketRange(0, int32_t(plan->buckets.size()))};
}

int reduce_scatter_local(const zdo_plan *plan, const uint16_t *const *replicas, int32_t n_replicas,
                         int32_t replica_coords, float scale, uint16_t *out, int32_t out_coords, void *stream) {
    const char *fn = "reduce_scatter_local";
    if (int rc = check_plan(plan, fn))
        return rc;
    return reduce_scatter_impl(fn, plan, all_buckets(plan), replicas, n_replicas, replica_coords, scale, out,
                               out_coords, stream);
}

int reduce_scatter_local_buckets(const zdo_plan *plan, int32_t bucket_begin, int32_t bucket_end,
                                 const uint16_t *const *replicas, int32_t n_replicas, int32_t replica_coords,
                                 float scale, uint16_t *out, int32_t out_coords, void *stream) {
    const char *fn = "reduce_scatter_local_buckets";
    if (int rc = check_plan(plan, fn))
        return rc;
    if (int rc = check_buckets(plan, bucket_begin, bucket_end, fn))
        return rc;
    return reduce_scatter_impl(fn, plan, {BucketRange(bucket_begin, bucket_end)}, replicas, n_replicas,
                               replica_coords, scale, out, out_coords, stream);
}

int reduce_scatter_local_bucket_list(const zdo_plan *plan, const int32_t *bucket_ranges, int32_t n_ranges,
                                     const uint16_t *const *replicas, int32_t n_replicas, int32_t replica_coords,
                                     float scale, uint16_t *out, int32_t out_coords, void *stream) {
    const char *fn = "reduce_scatter_local_bucket_list";
    if (int rc = check_plan(plan, fn))
        return rc;
    std::vector<BucketRange> ranges;
    if (int rc = check_bucket_list(plan, bucket_ranges, n_ranges, fn, ranges))
        return rc;
    return reduce_scatter_impl(fn, plan, ranges, replicas, n_replicas, replica_coords, scale, out, out_coords,
                               stream);
}

int force_all_reduce(const zdo_plan *plan, const uint16_t *const *replicas, int32_t n_replicas, float scale,
                     uint16_t *out_full, void *stream) {
    const char *fn = "force_all_reduce";
    if (int rc = check_plan(plan, fn))
        return rc;
    if (n_replicas < 1 || n_replicas > ZDO_MAX_REPLICAS)
        return fail(ZDO_EINVAL, std::string(fn) + ": n_replicas must be in [1, " + std::to_string(ZDO_MAX_REPLICAS) +
                                    "]");
    ReduceArgs a{};
    Span spans[ZDO_MAX_REPLICAS];
    if (int rc = take_replicas(plan, replicas, n_replicas, ZDO_WORLD, fn, a.rep, spans))
        return rc;
    if (int rc = check_ptr(out_full, fn, "out_full"))
        return rc;
    const Span so = span_of(out_full, plan->buffer_numel, 2);
    for (int32_t j = 0; j < n_replicas; ++j)
        if (overlap(so, spans[j]) && out_full != replicas[j])
            return fail(ZDO_EALIAS, std::string(fn) + ": out_full overlaps replica " + std::to_string(j) +
                                        " without coinciding with it");
    a.walk = one_run(nullptr, nullptr, 0, 0, seg_tiles(0, plan->buffer_numel), plan->buffer_numel);
    a.nrep = n_replicas;
    a.in_local = 0;
    a.out_local = 0;
    a.scale = scale;
    a.out = out_full;
    return launch_result(launch_reduce(a, plan->lds_per_cu, static_cast<hipStream_t>(stream)), fn);
}

// n_instances groups of n_grads / n_instances contributions (1 for the plain
// step).
static int adam_step(const char *fn, const zdo_plan *plan, const std::vector<BucketRange> &ranges,
                     const uint16_t *const *grads, int32_t n_grads, int32_t n_instances, int32_t grad_coords,
                     float scale, float *master, float *exp_avg, float *exp_avg_sq, uint16_t *param_out,
                     int32_t param_coords, const zdo_adam *hp, const float *coeff, float *main_grad_out,
                     void *stream) {
    if (n_grads < 1 || n_grads > ZDO_MAX_REPLICAS)
        return fail(ZDO_EINVAL, std::string(fn) + ": n_grads must be in [1, " + std::to_string(ZDO_MAX_REPLICAS) +
                                    "]");
    if (int rc = check_coords(grad_coords, fn, "grad_coords"))
        return rc;
    if (param_out)
        if (int rc = check_coords(param_coords, fn, "param_coords"))
            return rc;
    if (!hp)
        return fail(ZDO_EINVAL, std::string(fn) + ": hp is NULL");
    if (hp->step < 1 || hp->reserved != 0)
        return fail(ZDO_EINVAL, std::string(fn) + ": hp->step must be >= 1 and hp->reserved 0");
    if (!(hp->beta1 >= 0.0f && hp->beta1 < 1.0f && hp->beta2 >= 0.0f && hp->beta2 < 1.0f))
        return fail(ZDO_EINVAL, std::string(fn) + ": beta1 and beta2 must be in [0, 1)");
    StepArgs a{};
    Span gs[ZDO_MAX_REPLICAS];
    if (int rc = take_replicas(plan, grads, n_grads, grad_coords, fn, a.rep, gs))
        return rc;
    if (int rc = check_ptr(master, fn, "master"))
        return rc;
    if (int rc = check_ptr(exp_avg, fn, "exp_avg"))
        return rc;
    if (int rc = check_ptr(exp_avg_sq, fn, "exp_avg_sq"))
        return rc;
    if (param_out)
        if (int rc = check_ptr(param_out, fn, "param_out"))
            return rc;
    if (main_grad_out)
        if (int rc = check_ptr(main_grad_out, fn, "main_grad_out"))
            return rc;
    if (coeff && !aligned_to(coeff, 4))
        return fail(ZDO_EALIGN, std::string(fn) + ": grad_coeff is not 4-byte aligned");
    const int64_t L = plan->shard_numel;
    // Every written buffer must be disjoint from every other buffer.
    struct Named {
        Span s;
        const char *name;
    };
    Named written[5];
    int nw = 0;
    written[nw++] = {span_of(master, L, 4), "master"};
    written[nw++] = {span_of(exp_avg, L, 4), "exp_avg"};
    written[nw++] = {span_of(exp_avg_sq, L, 4), "exp_avg_sq"};
    if (param_out)
        written[nw++] = {span_of(param_out, extent(plan, param_coords), 2), "param_out"};
    if (main_grad_out)
        written[nw++] = {span_of(main_grad_out, L, 4), "main_grad_out"};
    for (int i = 0; i < nw; ++i) {
        for (int k = i + 1; k < nw; ++k)
            if (overlap(written[i].s, written[k].s))
                return fail(ZDO_EALIAS, std::string(fn) + ": " + written[i].name + " overlaps " + written[k].name);
        for (int32_t j = 0; j < n_grads; ++j)
            if (overlap(written[i].s, gs[j]))
                return fail(ZDO_EALIAS, std::string(fn) + ": " + written[i].name + " overlaps grad " +
                                            std::to_string(j));
        if (coeff && overlap(written[i].s, span_of(coeff, 1, 4)))
            return fail(ZDO_EALIAS, std::string(fn) + ": " + written[i].name + " overlaps grad_coeff");
    }
    a.nrep = n_grads;
    a.ninst = n_instances;
    a.dinst = n_grads / n_instances;
    a.in_local = grad_coords == ZDO_LOCAL;
    a.param_local = param_coords == ZDO_LOCAL;
    a.scale = scale;
    a.master = master;
    a.m = exp_avg;
    a.v = exp_avg_sq;
    a.param = param_out;
    a.main_grad = main_grad_out;
    a.coeff = coeff;
    a.state_numel = L;
    a.c.lr = hp->lr;
    a.c.b1 = hp->beta1;
    a.c.b2 = hp->beta2;
    a.c.omb1 = 1.0f - hp->beta1;
    a.c.omb2 = 1.0f - hp->beta2;
    a.c.eps = hp->eps;
    a.c.wd = hp->weight_decay;
    a.c.bc1 = bias_correction(hp->beta1, hp->step);
    a.c.bc2 = bias_correction(hp->beta2, hp->step);
    const std::vector<TileRun> runs = tile_runs(plan->param_segs, plan->param_seg_bucket.data(), plan->param_tiles,
                                                ranges);
    return launch_runs(runs, plan->d_param_segs, plan->d_param_group, int64_t(plan->param_segs.size()), fn,
                       [&](const Walk &w) {
                           a.walk = w;
                           return launch_step(a, plan->lds_per_cu, static_cast<hipStream_t>(stream));
                       });
}

int sharded_adam_step(const zdo_plan *plan, const uint16_t *const *grads, int32_t n_grads, int32_t grad_coords,
                      float scale, float *master, float *exp_avg, float *exp_avg_sq, uint16_t *param_out,
                      int32_t param_coords, const zdo_adam *hp, float *main_grad_out, void *stream) {
    const char *fn = "sharded_adam_step";
    if (int rc = check_plan(plan, fn))
        return rc;
    return adam_step(fn, plan, all_buckets(plan), grads, n_grads, 1, grad_coords, scale, master, exp_avg, exp_avg_sq,
                     param_out, param_coords, hp, nullptr, main_grad_out, stream);
}

int sharded_adam_step_buckets(const zdo_plan *plan, int32_t bucket_begin, int32_t bucket_end,
                              const uint16_t *const *grads, int32_t n_grads, int32_t grad_coords, float scale,
                              float *master, float *exp_avg, float *exp_avg_sq, uint16_t *param_out,
                              int32_t param_coords, const zdo_adam *hp, float *main_grad_out, void *stream) {
    const char *fn = "sharded_adam_step_buckets";
    if (int rc = check_plan(plan, fn))
        return rc;
    if (int rc = check_buckets(plan, bucket_begin, bucket_end, fn))
        return rc;
    return adam_step(fn, plan, {BucketRange(bucket_begin, bucket_end)}, grads, n_grads, 1, grad_coords, scale, master,
                     exp_avg, exp_avg_sq, param_out, param_coords, hp, nullptr, main_grad_out, stream);
}

int sharded_adam_step_bucket_list(const zdo_plan *plan, const int32_t *bucket_ranges, int32_t n_ranges,
                                  const uint16_t *const *grads, int32_t n_grads, int32_t grad_coords, float scale,
                                  float *master, float *exp_avg, float *exp_avg_sq, uint16_t *param_out,
                                  int32_t param_coords, const zdo_adam *hp, float *main_grad_out, void *stream) {
    const char *fn = "sharded_adam_step_bucket_list";
    if (int rc = check_plan(plan, fn))
        return rc;
    std::vector<BucketRange> ranges;
    if (int rc = check_bucket_list(plan, bucket_ranges, n_ranges, fn, ranges))
        return rc;
    return adam_step(fn, plan, ranges, grads, n_grads, 1, grad_coords, scale, master, exp_avg, exp_avg_sq, param_out,
                     param_coords, hp, nullptr, main_grad_out, stream);
}

int sharded_adam_step_clipped(const zdo_plan *plan, const uint16_t *const *grads, int32_t n_grads,
                              int32_t grad_coords, float scale, float *master, float *exp_avg, float *exp_avg_sq,
                              uint16_t *param_out, int32_t param_coords, const zdo_adam *hp,
                              const float *grad_coeff, float *main_grad_out, void *stream) {
    const char *fn = "sharded_adam_step_clipped";
    if (int rc = check_plan(plan, fn))
        return rc;
    if (!grad_coeff)
        return fail(ZDO_EINVAL, "sharded_adam_step_clipped: grad_coeff is NULL");
    return adam_step(fn, plan, all_buckets(plan), grads, n_grads, 1, grad_coords, scale, master, exp_avg, exp_avg_sq,
                     param_out, param_coords, hp, grad_coeff, main_grad_out, stream);
}

int sharded_adam_step_instances(const zdo_plan *plan, const uint16_t *const *grads, int32_t n_instances,
                                int32_t grad_coords, float scale, float *master, float *exp_avg, float *exp_avg_sq,
                                uint16_t *param_out, int32_t param_coords, const zdo_adam *hp, float *main_grad_out,
                                void *stream) {
    const char *fn = "sharded_adam_step_instances";
    if (int rc = check_plan(plan, fn))
        return rc;
    if (n_instances < 1 || int64_t(n_instances) * plan->dp_size > ZDO_MAX_REPLICAS)
        return fail(ZDO_EINVAL, std::string(fn) + ": n_instances must be >= 1 with n_instances * D <= " +
                                    std::to_string(ZDO_MAX_REPLICAS));
    return adam_step(fn, plan, all_buckets(plan), grads, n_instances * plan->dp_size, n_instances, grad_coords,
                     scale, master, exp_avg, exp_avg_sq, param_out, param_coords, hp, nullptr, main_grad_out, stream);
}

int64_t zdo_plan_norm_workspace_bytes(const zdo_plan *p) {
    if (!p)
        return -1;
    // one partial per tile, then up to 1024 second-level sums
    return (p->param_tiles + 1024) * int64_t(sizeof(double));
}

static int norm_sq_impl(const char *fn, const zdo_plan *plan, const uint16_t *const *replicas, int32_t n_replicas,
                        int32_t replica_coords, float scale, uint16_t *reduced_out, int32_t out_coords,
                        void *workspace, double *norm_sq_out, void *stream) {
    if (n_replicas < 1 || n_replicas > ZDO_MAX_REPLICAS)
        return fail(ZDO_EINVAL, std::string(fn) + ": n_replicas must be in [1, " + std::to_string(ZDO_MAX_REPLICAS) +
                                    "]");
    if (int rc = check_coords(replica_coords, fn, "replica_coords"))
        return rc;
    if (reduced_out)
        if (int rc = check_coords(out_coords, fn, "out_coords"))
            return rc;
    NormArgs a{};
    Span spans[ZDO_MAX_REPLICAS];
    if (int rc = take_replicas(plan, replicas, n_replicas, replica_coords, fn, a.rep, spans))
        return rc;
    if (reduced_out)
        if (int rc = check_ptr(reduced_out, fn, "reduced_out"))
            return rc;
    if (int rc = check_ptr(workspace, fn, "workspace"))
        return rc;
    if (!norm_sq_out)
        return fail(ZDO_EINVAL, std::string(fn) + ": norm_sq_out is NULL");
    if (!aligned_to(norm_sq_out, 8))
        return fail(ZDO_EALIGN, std::string(fn) + ": norm_sq_out is not 8-byte aligned");
    const Span ws = span_of(workspace, zdo_plan_norm_workspace_bytes(plan), 1);
    const Span ns = span_of(norm_sq_out, 1, 8);
    if (overlap(ws, ns))
        return fail(ZDO_EALIAS, std::string(fn) + ": workspace overlaps norm_sq_out");
    for (int32_t j = 0; j < n_replicas; ++j)
        if (overlap(ws, spans[j]) || overlap(ns, spans[j]))
            return fail(ZDO_EALIAS, std::string(fn) + ": workspace or norm_sq_out overlaps replica " +
                                        std::to_string(j));
    if (reduced_out) {
        const Span so = span_of(reduced_out, extent(plan, out_coords), 2);
        if (overlap(so, ws) || overlap(so, ns))
            return fail(ZDO_EALIAS, std::string(fn) + ": reduced_out overlaps workspace or norm_sq_out");
        for (int32_t j = 0; j < n_replicas; ++j)
            if (overlap(so, spans[j]) && !(reduced_out == replicas[j] && out_coords == replica_coords))
                return fail(ZDO_EALIAS, std::string(fn) + ": reduced_out overlaps replica " + std::to_string(j) +
                                            " without coinciding with it");
    }
    a.walk = one_run(plan->d_param_segs, plan->d_param_group, int64_t(plan->param_segs.size()), 0, plan->param_tiles);
    a.nrep = n_replicas;
    a.in_local = replica_coords == ZDO_LOCAL;
    a.out_local = out_coords == ZDO_LOCAL;
    a.scale = scale;
    a.out = reduced_out;
    a.partial = static_cast<double *>(workspace);
    return launch_result(launch_norm(a, norm_sq_out, plan->lds_per_cu, static_cast<hipStream_t>(stream)), fn);
}

int grad_norm_sq(const zdo_plan *plan, const uint16_t *const *replicas, int32_t n_replicas, int32_t replica_coords,
                 float scale, uint16_t *reduced_out, int32_t out_coords, void *workspace, double *norm_sq_out,
                 void *stream) {
    const char *fn = "grad_norm_sq";
    if (int rc = check_plan(plan, fn))
        return rc;
    return norm_sq_impl(fn, plan, replicas, n_replicas, replica_coords, scale, reduced_out, out_coords, workspace,
                        norm_sq_out, stream);
}

int grad_norm_sq_no_alloc(const zdo_plan *plan, const uint16_t *const *replicas, int32_t n_replicas,
                          int32_t replica_coords, float scale, uint16_t *reduced_out, int32_t out_coords,
                          double *norm_sq_out, void *stream) {
    const char *fn = "grad_norm_sq_no_alloc";
    if (!plan)
        return fail(ZDO_EINVAL, std::string(fn) + ": plan is NULL");
    // the size limit first: it needs only the plan's host tables
    const int64_t need = zdo_plan_norm_workspace_bytes(plan);
    if (need > int64_t(ZDO_NO_ALLOC_SCRATCH_BYTES))
        return fail(ZDO_EINVAL, std::string(fn) + ": the plan needs " + std::to_string(need) +
                                    " bytes of scratch, more than the library's static " +
                                    std::to_string(ZDO_NO_ALLOC_SCRATCH_BYTES) +
                                    " (use grad_norm_sq with a workspace of zdo_plan_norm_workspace_bytes)");
    if (int rc = check_plan(plan, fn))
        return rc;
    void *scratch = nullptr;
    const hipError_t e = no_alloc_scratch(&scratch);
    if (e != hipSuccess)
        return fail(ZDO_EHIP, std::string(fn) + ": the static scratch array's address: " + hipGetErrorString(e));
    return norm_sq_impl(fn, plan, replicas, n_replicas, replica_coords, scale, reduced_out, out_coords, scratch,
                        norm_sq_out, stream);
}

int clip_coefficient(const double *norm_sq_parts, int32_t n_parts, float max_norm, float *coeff_out,
                     double *norm_out, void *stream) {
    const char *fn = "clip_coefficient";
    if (!norm_sq_parts || n_parts < 1)
        return fail(ZDO_EINVAL, std::string(fn) + ": need at least one squared norm");
    if (!coeff_out)
        return fail(ZDO_EINVAL, std::string(fn) + ": coeff_out is NULL");
    if (!aligned_to(norm_sq_parts, 8) || !aligned_to(coeff_out, 4) || (norm_out && !aligned_to(norm_out, 8)))
        return fail(ZDO_EALIGN, std::string(fn) + ": a pointer is not naturally aligned");
    const Span ps = span_of(norm_sq_parts, n_parts, 8), cs = span_of(coeff_out, 1, 4);
    if (overlap(ps, cs) || (norm_out && (overlap(ps, span_of(norm_out, 1, 8)) ||
                                         overlap(cs, span_of(norm_out, 1, 8)))))
        return fail(ZDO_EALIAS, std::string(fn) + ": outputs overlap each other or the squared norms");
    return launch_result(launch_clip(norm_sq_parts, n_parts, max_norm, coeff_out, norm_out,
                                     static_cast<hipStream_t>(stream)), fn);
}

int writeback_params(const zdo_plan *plan, const float *master, uint16_t *param_out, int32_t param_coords,
                     void *stream) {
    const char *fn = "writeback_params";
    if (int rc = check_plan(plan, fn))
        return rc;
    if (int rc = check_coords(param_coords, fn, "param_coords"))
        return rc;
    if (int rc = check_ptr(master, fn, "master"))
        return rc;
    if (int rc = check_ptr(param_out, fn, "param_out"))
        return rc;
    if (overlap(span_of(master, plan->shard_numel, 4), span_of(param_out, extent(plan, param_coords), 2)))
        return fail(ZDO_EALIAS, std::string(fn) + ": param_out overlaps master");
    WritebackArgs a{};
    a.walk = one_run(plan->d_param_segs, plan->d_param_group, int64_t(plan->param_segs.size()), 0, plan->param_tiles);
    a.param_local = param_coords == ZDO_LOCAL;
    a.master = master;
    a.param = param_out;
    a.state_numel = plan->shard_numel;
    return launch_result(launch_writeback(a, static_cast<hipStream_t>(stream)), fn);
}

int all_gather_params(const zdo_plan *plan, const uint16_t *const *params, int32_t n_params, uint16_t *out,
                      void *stream) {
    const char *fn = "all_gather_params";
    if (int rc = check_plan(plan, fn))
        return rc;
    if (n_params != plan->dp_size)
        return fail(ZDO_EINVAL, std::string(fn) + ": n_params must equal the DP size " +
                                    std::to_string(plan->dp_size));
    GatherArgs a{};
    Span spans[ZDO_MAX_REPLICAS];
    if (int rc = take_replicas(plan, params, n_params, ZDO_WORLD, fn, a.src, spans))
        return rc;
    if (int rc = check_ptr(out, fn, "out"))
        return rc;
    const Span so = span_of(out, plan->buffer_numel, 2);
    for (int32_t j = 0; j < n_params; ++j)
        if (overlap(so, spans[j]) && out != params[j])
            return fail(ZDO_EALIAS, std::string(fn) + ": out overlaps params[" + std::to_string(j) +
                                        "] without coinciding with it");
    a.ranges = plan->d_gather_ranges;
    a.group = plan->d_gather_group;
    a.nranges = int64_t(plan->gather_ranges.size());
    a.ntiles = plan->gather_tiles;
    a.out = out;
    return launch_result(launch_gather(a, plan->lds_per_cu, static_cast<hipStream_t>(stream)), fn);
}

int zdo_device_copy(void *dst, const void *src, int64_t bytes, void *stream) {
    const char *fn = "zdo_device_copy";
    if (bytes < 0 || bytes % 16 != 0)
        return fail(ZDO_EINVAL, std::string(fn) + ": bytes must be a non-negative multiple of 16");
    if (int rc = check_ptr(dst, fn, "dst"))
        return rc;
    if (int rc = check_ptr(src, fn, "src"))
        return rc;
    if (overlap(span_of(dst, bytes, 1), span_of(src, bytes, 1)))
        return fail(ZDO_EALIAS, std::string(fn) + ": dst overlaps src");
    return launch_result(launch_copy(dst, src, bytes / 16, static_cast<hipStream_t>(stream)), fn);
}

int zdo_stream_probe(const uint16_t *const *reads, int32_t n_reads, float *state0, float *state1, float *state2,
                     uint16_t *out, int64_t n, int32_t stores, int32_t waves_per_cu, void *stream) {
    const char *fn = "zdo_stream_probe";
    if (n_reads != 8 && n_reads != 16 && n_reads != 32)
        return fail(ZDO_EINVAL, std::string(fn) + ": n_reads must be 8, 16 or 32");
    if (stores != ZDO_PROBE_STORE_ALL && stores != ZDO_PROBE_STORE_OUT && stores != ZDO_PROBE_STORE_NONE)
        return fail(ZDO_EINVAL, std::string(fn) + ": stores must be ZDO_PROBE_STORE_ALL, _OUT or _NONE");
    if (n < 0 || n % kTileElems != 0)
        return fail(ZDO_EINVAL, std::string(fn) + ": n must be a non-negative multiple of 512");
    if (waves_per_cu < 0)
        return fail(ZDO_EINVAL, std::string(fn) + ": waves_per_cu must be >= 0");
    if (!reads)
        return fail(ZDO_EINVAL, std::string(fn) + ": reads is NULL");
    ProbeArgs a{};
    Span spans[ZDO_MAX_REPLICAS + 4];
    for (int32_t j = 0; j < n_reads; ++j) {
        if (int rc = check_ptr(reads[j], fn, "reads[j]"))
            return rc;
        a.rep[j] = reads[j];
        spans[j] = span_of(reads[j], n, 2);
    }
    float *st[3] = {state0, state1, state2};
    for (int i = 0; i < 3; ++i) {
        if (int rc = check_ptr(st[i], fn, "state"))
            return rc;
        a.state[i] = st[i];
        spans[n_reads + i] = span_of(st[i], n, 4);
    }
    if (int rc = check_ptr(out, fn, "out"))
        return rc;
    spans[n_reads + 3] = span_of(out, n, 2);
    for (int32_t i = 0; i < n_reads + 4; ++i)
        for (int32_t k = i + 1; k < n_reads + 4; ++k)
            if (overlap(spans[i], spans[k]))
                return fail(ZDO_EALIAS, std::string(fn) + ": buffers overlap");
    int dev = 0, lds = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess)
        return fail(ZDO_EHIP, std::string(fn) + ": no HIP device");
    a.nrep = n_reads;
    a.stores = stores;
    a.out = out;
    a.ntiles = n / kTileElems;
    return launch_result(launch_probe(a, waves_per_cu, lds, static_cast<hipStream_t>(stream)), fn);
}

}  // extern "C"
