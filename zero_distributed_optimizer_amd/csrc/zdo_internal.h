// Internal declarations shared by the plan builder, the kernels and the C-ABI.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "zdo.h"

namespace zdo {

// Elements per lane per tile: 8 (a 16-byte bf16 chunk, or two 4-element
// quads in the step).
constexpr int kChunk = 8;
// Threads per workgroup; a workgroup takes one tile of kBlock chunks at a time.
#ifndef ZDO_BLOCK
#define ZDO_BLOCK 64
#endif
constexpr int kBlock = ZDO_BLOCK;
constexpr int kTileElems = kChunk * kBlock;

// One contiguous run of the rank's elements, as the kernels walk it.
struct Seg {
    int64_t wbeg;   // WORLD index of the first element
    int64_t lbeg;   // LOCAL (shard) index of the first element; lbeg == wbeg (mod kAnchor)
    int64_t len;    // elements, >= 1
    int64_t tile0;  // index of the segment's first tile in the launch's tile space
};

// A segment's tiles start at its first WORLD index rounded down to a
// multiple of kAnchor (64 elements: one 128-byte cache line of bf16), so
// that, at a given alignment of the buffers, a tile's runs never share a
// cache line with the next tile's.
constexpr int64_t kAnchor = 64;
constexpr int64_t tile_origin(int64_t wbeg) { return wbeg / kAnchor * kAnchor; }
// Tiles a segment needs: kTileElems-element steps from its origin to its end.
inline int64_t seg_tiles(int64_t wbeg, int64_t len) {
    return (wbeg + len - tile_origin(wbeg) + kTileElems - 1) / kTileElems;
}
// Tiles map to their segment (or range) through one entry per kTileGroup
// tiles: the one holding the group's first tile; the few later ones of the
// group follow by their tile0. The index stays small enough to live in the
// L2 cache, so a tile's lookup does not go to HBM.
constexpr int64_t kTileGroup = 64;

// A group entry of the segment walks: a copy of the segment holding the
// group's first tile, with that segment's index and the next segment's first
// tile, so that a workgroup finds its segment in one load unless its tile
// lies past a segment start inside the group.
struct GroupSeg {
    Seg seg;
    int64_t index;
    int64_t next_tile0;  // first tile of segment index + 1, or INT64_MAX
};

// One rank range of one padded bucket, as the all-gather walks it: tiles of
// kGatherTile elements from rb rounded down to kAnchor.
struct RangeSpan {
    int64_t rb, re;  // WORLD range [rb, re)
    int64_t tile0;   // its first tile in the all-gather's tile space
    int64_t src;     // the rank whose buffer holds it
};
// All-gather tiles: 2048 elements, four 16-byte chunks per lane, so that the
// tile's lookups are paid once per 4 KiB read. They map to ranges through a
// kTileGroup index as above.
constexpr int64_t kGatherTile = 2048;
inline int64_t range_tiles(int64_t rb, int64_t len) {
    return (rb + len - tile_origin(rb) + kGatherTile - 1) / kGatherTile;
}

void set_error(const std::string &msg);

}  // namespace zdo

struct zdo_plan {
    int32_t dp_size = 0, rank = 0;
    int64_t bucket_numel = 0;
    std::vector<int64_t> param_numel;
    std::vector<zdo_bucket> buckets;
    std::vector<zdo_piece> pieces;
    int64_t buffer_numel = 0;  // N
    int64_t shard_numel = 0;   // L
    int64_t owned_numel = 0;   // E
    // Owned parameter elements (one run per bucket, padding excluded) and the
    // rank's whole range of every bucket (padding included).
    std::vector<zdo::Seg> param_segs, range_segs;
    std::vector<int32_t> param_seg_bucket;   // bucket of each param seg (range seg i is bucket i)
    int64_t param_tiles = 0, range_tiles = 0;
    // The all-gather's launch space: every rank range of every padded bucket
    // (bucket-major, rank-minor).
    std::vector<zdo::RangeSpan> gather_ranges;
    int64_t gather_tiles = 0;
    // Device copies, in one allocation on `device`: both segment lists, the
    // gather ranges, and the kTileGroup index of each launch space.
    void *d_table = nullptr;
    const zdo::Seg *d_param_segs = nullptr, *d_range_segs = nullptr;
    const zdo::GroupSeg *d_param_group = nullptr, *d_range_group = nullptr;
    const zdo::RangeSpan *d_gather_ranges = nullptr;
    const uint32_t *d_gather_group = nullptr;
    int device = -1;
    int lds_per_cu = 0;   // bytes of LDS per compute unit on `device`
};
