// Host-only exercise of the plan builder and the ABI's argument checks, for a
// build with AddressSanitizer and UndefinedBehaviorSanitizer on the host code
// (tests/test_host_sanitizers.py). The kernel launchers are stubs: without a
// device the plan has no device table and no launch is reached.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>
#include "zdo.h"
#include "kernels.h"

namespace zdo {
hipError_t launch_reduce(const ReduceArgs &, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_step(const StepArgs &, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_writeback(const WritebackArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_copy(void *, const void *, int64_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_norm(const NormArgs &, double *, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_clip(const double *, int32_t, float, float *, double *, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_gather(const GatherArgs &, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t no_alloc_scratch(void **out) { *out = nullptr; return hipErrorNoDevice; }
hipError_t launch_probe(const ProbeArgs &, int, int, hipStream_t) { return hipErrorNoDevice; }
}

int main() {
    std::mt19937_64 rng(7);
    long checked = 0;
    for (int trial = 0; trial < 3000; ++trial) {
        const int np = 1 + int(rng() % 40);
        std::vector<int64_t> sizes(np);
        for (auto &x : sizes) x = 1 + int64_t(rng() % (rng() % 2 ? 30 : 20000));
        const int32_t D = 1 + int32_t(rng() % 64);
        const int64_t bucket = 1 + int64_t(rng() % 50000);
        const int32_t rank = int32_t(rng() % D);
        zdo_plan *p = nullptr;
        if (build_range_map(sizes.data(), np, bucket, D, rank, &p) != ZDO_OK) { std::printf("build failed\n"); return 1; }
        int32_t nb = 0;
        zdo_plan_buckets(p, nullptr, 0, &nb);
        std::vector<zdo_bucket> b(nb);
        if (zdo_plan_buckets(p, b.data(), nb, &nb) != ZDO_OK) return 2;
        int64_t npc = 0;
        zdo_plan_pieces(p, nullptr, 0, &npc);
        std::vector<zdo_piece> pc(static_cast<size_t>(npc));
        if (zdo_plan_pieces(p, pc.data(), npc, &npc) != ZDO_OK) return 3;
        // every piece inside the shard and the buffer; pieces do not overlap
        // in the shard
        const int64_t L = zdo_plan_shard_numel(p), N = zdo_plan_buffer_numel(p);
        std::vector<char> used(size_t(L), 0);
        for (const auto &q : pc) {
            const int64_t n = q.gbuf_world.end - q.gbuf_world.start;
            if (q.gbuf_world.start < 0 || q.gbuf_world.end > N || q.shard_offset < 0 || q.shard_offset + n > L) return 4;
            for (int64_t k = q.shard_offset; k < q.shard_offset + n; ++k) { if (used[size_t(k)]) return 5; used[size_t(k)] = 1; }
            ++checked;
        }
        // launch calls on a host-only plan: errors, no crash
        const uint16_t *reps[64] = {};
        zdo_adam hp{1e-3f, 0.9f, 0.999f, 1e-8f, 0.0f, 0, 1};
        if (reduce_scatter_local(p, reps, D, ZDO_WORLD, 1.0f, nullptr, ZDO_WORLD, nullptr) == ZDO_OK) return 6;
        if (sharded_adam_step(p, reps, D, ZDO_WORLD, 1.0f, nullptr, nullptr, nullptr, nullptr, 0, &hp, nullptr, nullptr) == ZDO_OK) return 7;
        if (all_gather_params(p, reps, D, nullptr, nullptr) == ZDO_OK) return 8;
        const int32_t ranges[4] = {0, nb, nb, nb};
        if (sharded_adam_step_bucket_list(p, ranges, 2, reps, D, ZDO_WORLD, 1.0f, nullptr, nullptr, nullptr, nullptr, 0,
                                          &hp, nullptr, nullptr) == ZDO_OK) return 13;
        if (reduce_scatter_local_bucket_list(p, ranges, 2, reps, D, ZDO_WORLD, 1.0f, nullptr, ZDO_WORLD, nullptr) == ZDO_OK)
            return 14;
        double nsq = 0.0;
        if (grad_norm_sq_no_alloc(p, reps, D, ZDO_WORLD, 1.0f, nullptr, ZDO_WORLD, &nsq, nullptr) == ZDO_OK) return 15;
        (void)zdo_last_error();
        zdo_plan_destroy(p);
    }
    // argument errors
    zdo_plan *p = nullptr;
    int64_t s[2] = {5, -1};
    if (build_range_map(s, 2, 10, 2, 0, &p) == ZDO_OK) return 9;
    if (build_range_map(nullptr, 0, 10, 2, 0, &p) == ZDO_OK) return 10;
    if (build_range_map(s, 1, 10, 65, 0, &p) == ZDO_OK) return 11;
    if (zdo_device_copy(nullptr, nullptr, 15, nullptr) == ZDO_OK) return 12;
    // the stream probe's argument checks come before any device call
    const uint16_t *rr[8] = {};
    if (zdo_stream_probe(rr, 8, nullptr, nullptr, nullptr, nullptr, 512, 3, 0, nullptr) == ZDO_OK) return 16;
    if (zdo_stream_probe(rr, 7, nullptr, nullptr, nullptr, nullptr, 512, ZDO_PROBE_STORE_ALL, 0, nullptr) == ZDO_OK)
        return 17;
    if (zdo_stream_probe(rr, 8, nullptr, nullptr, nullptr, nullptr, 500, ZDO_PROBE_STORE_NONE, 0, nullptr) == ZDO_OK)
        return 18;
    std::printf("ok: 3000 plans, %ld pieces checked\n", checked);
    return 0;
}
