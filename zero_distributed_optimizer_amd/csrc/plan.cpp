// Host side of the plan: bucket layout, rank ranges, the four-way range map
// and the segment table the kernels walk.
//
// Page "04 · 分布式优化器": one flat buffer cut into buckets by size (§2), each
// padded to a multiple of the DP size by the layout (§5) and split into D
// equal contiguous ranges, rank r owning range r (§2, §3); per parameter
// piece, the four ranges gbuf_world, gbuf_world_in_bucket, gbuf_local and
// param, translations of one another (§4.1).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <limits>
#include <new>

#include "zdo_internal.h"

namespace {

constexpr int64_t kMaxNumel = int64_t(1) << 56;

int64_t floor_mod(int64_t a, int64_t m) {
    int64_t r = a % m;
    return r < 0 ? r + m : r;
}

}  // namespace

namespace zdo {

int build_plan(const int64_t *param_numel, int32_t n_params, int64_t bucket_numel, int32_t dp_size,
               int32_t rank, zdo_plan &p) {
    if (!param_numel || n_params < 1) {
        set_error("build_range_map: need at least one parameter");
        return ZDO_EINVAL;
    }
    if (bucket_numel < 1) {
        set_error("build_range_map: bucket_numel must be >= 1");
        return ZDO_EINVAL;
    }
    if (dp_size < 1 || dp_size > ZDO_MAX_REPLICAS) {
        set_error("build_range_map: dp_size must be in [1, " + std::to_string(ZDO_MAX_REPLICAS) + "]");
        return ZDO_EINVAL;
    }
    if (rank < 0 || rank >= dp_size) {
        set_error("build_range_map: rank must be in [0, dp_size)");
        return ZDO_EINVAL;
    }
    p.dp_size = dp_size;
    p.rank = rank;
    p.bucket_numel = bucket_numel;
    p.param_numel.assign(param_numel, param_numel + n_params);

    // Buckets: parameters in order, packed; a bucket closes right after the
    // parameter that brings it to bucket_numel elements or after the last one,
    // and is padded at its tail to a multiple of D.
    std::vector<int64_t> param_start(n_params);
    std::vector<int32_t> param_bucket(n_params);
    int64_t offset = 0, filled = 0;
    for (int32_t i = 0; i < n_params; ++i) {
        const int64_t n = param_numel[i];
        if (n < 1 || n > kMaxNumel) {
            set_error("build_range_map: parameter " + std::to_string(i) + " has a bad element count");
            return ZDO_EINVAL;
        }
        param_start[i] = offset + filled;
        param_bucket[i] = int32_t(p.buckets.size());
        filled += n;
        if (offset + filled > kMaxNumel) {
            set_error("build_range_map: buffer too large");
            return ZDO_EINVAL;
        }
        if (filled >= bucket_numel || i == n_params - 1) {
            zdo_bucket b{};
            b.offset = offset;
            b.numel = filled;
            b.padded_numel = (filled + dp_size - 1) / dp_size * dp_size;
            b.shard_numel = b.padded_numel / dp_size;
            p.buckets.push_back(b);
            offset += b.padded_numel;
            filled = 0;
        }
    }
    p.buffer_numel = offset;

    // The rank's shard: per bucket, the local view starts at the first slot
    // at or after the previous view's end that has the WORLD start's phase
    // modulo kAnchor (64).
    int64_t end = 0;
    for (auto &b : p.buckets) {
        const int64_t rstart = b.offset + int64_t(rank) * b.shard_numel;
        b.shard_base = end + floor_mod(rstart - end, kAnchor);
        end = b.shard_base + b.shard_numel;
    }
    p.shard_numel = end;

    // Pieces: every parameter's overlap with the rank's range of its bucket.
    int32_t i = 0;
    for (int32_t bi = 0; bi < int32_t(p.buckets.size()); ++bi) {
        const zdo_bucket &b = p.buckets[bi];
        const int64_t rs = b.offset + int64_t(rank) * b.shard_numel;
        const int64_t re = rs + b.shard_numel;
        for (; i < n_params && param_bucket[i] == bi; ++i) {
            const int64_t ps = param_start[i], pe = ps + param_numel[i];
            const int64_t lo = std::max(ps, rs), hi = std::min(pe, re);
            if (lo >= hi)
                continue;
            zdo_piece pc{};
            pc.param_index = i;
            pc.bucket_index = bi;
            pc.gbuf_world = {lo, hi};
            pc.gbuf_world_in_bucket = {lo - b.offset, hi - b.offset};
            pc.gbuf_local = {lo - rs, hi - rs};
            pc.param = {lo - ps, hi - ps};
            pc.shard_offset = b.shard_base + (lo - rs);
            p.pieces.push_back(pc);
            p.owned_numel += hi - lo;
        }
        // Owned parameter elements of this bucket form one run (the padding
        // sits at the bucket's tail); the whole range is one run as well.
        const int64_t own_end = std::min(re, b.offset + b.numel);
        if (own_end > rs) {
            p.param_segs.push_back({rs, b.shard_base, own_end - rs, 0});
            p.param_seg_bucket.push_back(bi);
        }
        p.range_segs.push_back({rs, b.shard_base, b.shard_numel, 0});
    }
    for (auto *segs : {&p.param_segs, &p.range_segs}) {
        int64_t t = 0;
        for (auto &s : *segs) {
            s.tile0 = t;
            t += seg_tiles(s.wbeg, s.len);
        }
        (segs == &p.param_segs ? p.param_tiles : p.range_tiles) = t;
    }
    int64_t gt = 0;
    for (const auto &b : p.buckets)
        for (int32_t j = 0; j < dp_size; ++j) {
            const int64_t rb = b.offset + int64_t(j) * b.shard_numel;
            p.gather_ranges.push_back({rb, rb + b.shard_numel, gt, j});
            gt += range_tiles(rb, b.shard_numel);
        }
    p.gather_tiles = gt;
    return ZDO_OK;
}

int upload_plan(zdo_plan &p) {
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count < 1) {
        (void)hipGetLastError();
        return ZDO_OK;   // host-only plan
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        set_error("build_range_map: hipGetDevice failed");
        return ZDO_EHIP;
    }
    // per launch space, the segment holding the first tile of every
    // kTileGroup tiles
    auto group_index = [](int64_t ntiles, size_t n, auto tile0_of) {
        std::vector<uint32_t> g(size_t((ntiles + kTileGroup - 1) / kTileGroup));
        size_t s = 0;
        for (size_t i = 0; i < g.size(); ++i) {
            while (s + 1 < n && tile0_of(s + 1) <= int64_t(i) * kTileGroup)
                ++s;
            g[i] = uint32_t(s);
        }
        return g;
    };
    auto group_segs = [&](const std::vector<Seg> &segs, int64_t ntiles) {
        const auto idx = group_index(ntiles, segs.size(), [&](size_t s) { return segs[s].tile0; });
        std::vector<GroupSeg> g(idx.size());
        for (size_t i = 0; i < idx.size(); ++i) {
            const size_t s = idx[i];
            g[i] = {segs[s], int64_t(s),
                    s + 1 < segs.size() ? segs[s + 1].tile0 : std::numeric_limits<int64_t>::max()};
        }
        return g;
    };
    const auto param_group = group_segs(p.param_segs, p.param_tiles);
    const auto range_group = group_segs(p.range_segs, p.range_tiles);
    const auto gather_group =
        group_index(p.gather_tiles, p.gather_ranges.size(), [&](size_t y) { return p.gather_ranges[y].tile0; });
    // one allocation: segments, the two walks' group entries, the gather
    // ranges, then the gather's group index
    const size_t nseg = p.param_segs.size() + p.range_segs.size();
    const size_t seg_bytes = nseg * sizeof(Seg);
    const size_t gseg_bytes = (param_group.size() + range_group.size()) * sizeof(GroupSeg);
    const size_t span_bytes = p.gather_ranges.size() * sizeof(RangeSpan);
    const size_t bytes = seg_bytes + gseg_bytes + span_bytes + gather_group.size() * sizeof(uint32_t);
    std::vector<char> host(bytes);
    std::copy(p.param_segs.begin(), p.param_segs.end(), reinterpret_cast<Seg *>(host.data()));
    std::copy(p.range_segs.begin(), p.range_segs.end(),
              reinterpret_cast<Seg *>(host.data()) + p.param_segs.size());
    GroupSeg *gs = reinterpret_cast<GroupSeg *>(host.data() + seg_bytes);
    gs = std::copy(param_group.begin(), param_group.end(), gs);
    std::copy(range_group.begin(), range_group.end(), gs);
    std::copy(p.gather_ranges.begin(), p.gather_ranges.end(),
              reinterpret_cast<RangeSpan *>(host.data() + seg_bytes + gseg_bytes));
    std::copy(gather_group.begin(), gather_group.end(),
              reinterpret_cast<uint32_t *>(host.data() + seg_bytes + gseg_bytes + span_bytes));
    void *d = nullptr;
    hipError_t e = hipMalloc(&d, bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        set_error(std::string("build_range_map: hipMalloc of the segment table: ") + hipGetErrorString(e));
        return e == hipErrorOutOfMemory ? ZDO_ENOMEM : ZDO_EHIP;
    }
    e = hipMemcpy(d, host.data(), bytes, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        (void)hipFree(d);
        set_error(std::string("build_range_map: upload of the segment table: ") + hipGetErrorString(e));
        return ZDO_EHIP;
    }
    p.d_table = d;
    p.d_param_segs = static_cast<const Seg *>(d);
    p.d_range_segs = p.d_param_segs + p.param_segs.size();
    p.d_param_group = reinterpret_cast<const GroupSeg *>(static_cast<const char *>(d) + seg_bytes);
    p.d_range_group = p.d_param_group + param_group.size();
    p.d_gather_ranges = reinterpret_cast<const RangeSpan *>(static_cast<const char *>(d) + seg_bytes + gseg_bytes);
    p.d_gather_group =
        reinterpret_cast<const uint32_t *>(static_cast<const char *>(d) + seg_bytes + gseg_bytes + span_bytes);
    p.device = dev;
    if (hipDeviceGetAttribute(&p.lds_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
        hipSuccess) {
        (void)hipGetLastError();
        p.lds_per_cu = 0;
    }
    return ZDO_OK;
}

}  // namespace zdo
