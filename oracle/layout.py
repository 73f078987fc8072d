"""CPU oracle: bucket layout and the four-way range map of one DP rank.

TEST INFRASTRUCTURE. Only the tests, the smoke check and bench.py's CPU
baseline may import this package. The product path (the
zero_distributed_optimizer_amd package and its HIP library) never does,
and the two share no code.

Written from the page "04 · 分布式优化器" (Megatron-LM code-reading guide,
distributed optimizer chapter):
  * §2, decision one: the grads of one dtype form one contiguous 1-D buffer,
    which is cut by size into buckets.
  * §2, decision two, and the demo in §3: every bucket is split into D equal
    contiguous ranges and DP rank r owns range r, however many parameters it
    crosses and even when it cuts a parameter in two.
  * §4.1: Range is a half-open (start, end) with a rebase ("normalize"); each
    parameter piece owned by the rank carries four ranges (gbuf_world,
    gbuf_world_in_bucket, gbuf_local, param) that are translations of one
    another; the bucket size must divide by D; rank r's range starts at
    r * (bucket size / D) within the bucket.
  * §5: padding that makes a bucket divisible by D belongs to the buffer layout.

Readings where the page leaves a step open (each also listed in the design doc):
  * A parameter belongs to exactly one bucket (§4.1 speaks of "its" bucket);
    buckets are filled greedily in parameter order and a bucket closes right
    after the parameter that brings its element count to at least
    bucket_numel, or after the last parameter.
  * A bucket's padding sits at its tail, up to the next multiple of D.
  * The rank's fp32 shard (master, m, v) concatenates the per-bucket local
    views in bucket order, each placed at the first slot >= the previous
    end whose index is congruent to the range's world start modulo 64
    (SHARD_PHASE); so every shard index is congruent to its world index
    modulo 64. The gap slots (< 64 per bucket) and the padding slots are
    never read or written.
"""

from __future__ import annotations

from dataclasses import dataclass

SHARD_PHASE = 64  # elements: one 128-byte line of bf16


@dataclass(frozen=True)
class Range:
    """Half-open interval [start, end) of element indices (page 1, §4.1)."""
    start: int
    end: int

    @property
    def size(self) -> int:
        return self.end - self.start

    def normalize(self, start: int = 0) -> "Range":
        """The same interval shifted so that it begins at `start`."""
        return Range(start, start + self.size)

    def shift(self, delta: int) -> "Range":
        return Range(self.start + delta, self.end + delta)


@dataclass(frozen=True)
class Bucket:
    index: int
    offset: int          # world index of the bucket's first element
    numel: int           # parameter elements (unpadded)
    padded_numel: int    # numel rounded up to a multiple of D
    params: tuple        # parameter indices, in buffer order

    def shard_numel(self, dp_size: int) -> int:
        return self.padded_numel // dp_size


@dataclass(frozen=True)
class Layout:
    param_numel: tuple
    bucket_numel: int
    dp_size: int
    buckets: tuple
    param_world: tuple    # Range of each parameter in the flat buffer

    @property
    def buffer_numel(self) -> int:
        last = self.buckets[-1]
        return last.offset + last.padded_numel


@dataclass(frozen=True)
class Piece:
    """One parameter's intersection with the rank's range in one bucket."""
    param_index: int
    bucket_index: int
    gbuf_world: Range
    gbuf_world_in_bucket: Range
    gbuf_local: Range
    param: Range
    shard_offset: int     # index of gbuf_world.start in the rank's fp32 shard

    def as_tuple(self) -> tuple:
        return (self.param_index, self.bucket_index,
                self.gbuf_world.start, self.gbuf_world.end,
                self.gbuf_world_in_bucket.start, self.gbuf_world_in_bucket.end,
                self.gbuf_local.start, self.gbuf_local.end,
                self.param.start, self.param.end, self.shard_offset)


def build_layout(param_numel, bucket_numel: int, dp_size: int) -> Layout:
    """Place parameters contiguously, cut buckets, pad each bucket to a multiple of D."""
    sizes = tuple(int(n) for n in param_numel)
    if dp_size < 1 or bucket_numel < 1 or not sizes or min(sizes) < 1:
        raise ValueError("bad layout arguments")
    buckets = []
    param_world = []
    offset = 0           # world start of the bucket being filled
    members = []
    filled = 0
    for i, n in enumerate(sizes):
        param_world.append(Range(offset + filled, offset + filled + n))
        members.append(i)
        filled += n
        if filled >= bucket_numel or i == len(sizes) - 1:
            padded = -(-filled // dp_size) * dp_size
            buckets.append(Bucket(len(buckets), offset, filled, padded, tuple(members)))
            offset += padded
            members = []
            filled = 0
    return Layout(sizes, bucket_numel, dp_size, tuple(buckets), tuple(param_world))


def rank_range(bucket: Bucket, dp_size: int, rank: int) -> Range:
    """Rank r's range of a bucket, in world coordinates (page 1, §3 and §4.1)."""
    if bucket.padded_numel % dp_size != 0:
        raise AssertionError("bucket size must divide by the DP size")
    shard = bucket.padded_numel // dp_size
    return Range(bucket.offset + rank * shard, bucket.offset + (rank + 1) * shard)


def shard_bases(layout: Layout, rank: int) -> list:
    """Where each bucket's local view starts in the rank's fp32 shard, and the shard length."""
    bases = []
    end = 0
    for b in layout.buckets:
        start = rank_range(b, layout.dp_size, rank).start
        base = end + (start - end) % SHARD_PHASE
        bases.append(base)
        end = base + b.shard_numel(layout.dp_size)
    return bases, end


def rank_pieces(layout: Layout, rank: int) -> list:
    """All pieces the rank owns, ordered by world position (page 1, §3 and §4.1)."""
    if not 0 <= rank < layout.dp_size:
        raise ValueError("rank out of range")
    bases, _ = shard_bases(layout, rank)
    pieces = []
    for b in layout.buckets:
        mine = rank_range(b, layout.dp_size, rank)
        for p in b.params:
            pr = layout.param_world[p]
            lo, hi = max(pr.start, mine.start), min(pr.end, mine.end)
            if lo >= hi:
                continue
            world = Range(lo, hi)
            local = world.shift(-mine.start)
            pieces.append(Piece(
                param_index=p,
                bucket_index=b.index,
                gbuf_world=world,
                gbuf_world_in_bucket=world.shift(-b.offset),
                gbuf_local=local,
                param=world.shift(-pr.start),
                shard_offset=bases[b.index] + local.start,
            ))
    return pieces


def shard_numel(layout: Layout, rank: int) -> int:
    """Length L of the rank's fp32 shard, gap and padding slots included."""
    return shard_bases(layout, rank)[1]


def owned_numel(layout: Layout, rank: int) -> int:
    """Parameter elements owned by the rank (padding excluded)."""
    return sum(p.gbuf_world.size for p in rank_pieces(layout, rank))


def rank_ranges(layout: Layout, rank: int) -> list:
    """(world Range, shard start) of the rank's whole range in every bucket, padding included."""
    bases, _ = shard_bases(layout, rank)
    return [(rank_range(b, layout.dp_size, rank), bases[b.index]) for b in layout.buckets]
