"""Pins of the oracle's layout and range map (oracle.layout) against what page
"04 · 分布式优化器" fixes: the §3 demo, the §4.1 invariants (divisibility,
translation-only ranges, one bucket per parameter), the §4.3 slicing of split
parameters through the "param" range, and a brute-force owner scan."""

import os
import random

import pytest

import oracle.layout as L
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def test_page_demo_ranges():
    # 1000 elements, dp 4 -> shard 250, rank 1 owns [250, 500)
    lay = L.build_layout([1000], 1000, 4)
    assert lay.buffer_numel == 1000
    b = lay.buckets[0]
    assert b.shard_numel(4) == 250
    assert L.rank_range(b, 4, 1) == L.Range(250, 500)
    assert [L.rank_range(b, 4, r) for r in range(4)] == [L.Range(250 * r, 250 * (r + 1)) for r in range(4)]


def test_tiny_golden_pieces():
    w = W.get("tiny")
    lay = L.build_layout(w.param_numel, w.bucket_numel, w.dp_size)
    want = {}
    for row in _golden_rows("tiny_pieces.txt"):
        r, p, *vals = (int(x) for x in row)
        want.setdefault(r, []).append((p, 0, *vals))
    for r in range(4):
        got = [pc.as_tuple() for pc in L.rank_pieces(lay, r)]
        assert got == want[r], f"rank {r}"
    # the one parameter the demo's rank edge cuts is split 130 / 170
    split = [pc for r in range(4) for pc in L.rank_pieces(lay, r) if pc.param_index == 1]
    assert [(pc.param.start, pc.param.end) for pc in split] == [(0, 130), (130, 300)]


def test_range_normalize():
    r = L.Range(250, 420)
    assert r.size == 170
    assert r.normalize() == L.Range(0, 170)
    assert r.normalize(130) == L.Range(130, 300)


def _check_invariants(lay: L.Layout):
    D = lay.dp_size
    # every bucket divides by D; buckets tile the buffer; params sit in one bucket, in order
    pos = 0
    for b in lay.buckets:
        assert b.padded_numel % D == 0
        assert b.offset == pos
        assert b.numel <= b.padded_numel < b.numel + D
        pos += b.padded_numel
        inner = b.offset
        for p in b.params:
            pr = lay.param_world[p]
            assert pr.start == inner and pr.size == lay.param_numel[p]
            inner = pr.end
        assert inner == b.offset + b.numel
    assert pos == lay.buffer_numel
    assert [p for b in lay.buckets for p in b.params] == list(range(len(lay.param_numel)))
    # greedy closing rule: every bucket but the last reached bucket_numel only with its last param
    for b in lay.buckets[:-1]:
        assert b.numel >= lay.bucket_numel
        assert b.numel - lay.param_numel[b.params[-1]] < lay.bucket_numel
    # ranks' ranges tile every bucket
    for b in lay.buckets:
        rs = [L.rank_range(b, D, r) for r in range(D)]
        assert rs[0].start == b.offset and rs[-1].end == b.offset + b.padded_numel
        assert all(rs[i].end == rs[i + 1].start for i in range(D - 1))
    cover = {i: [] for i in range(len(lay.param_numel))}
    for r in range(D):
        pieces = L.rank_pieces(lay, r)
        bases, Ln = L.shard_bases(lay, r)
        used = []
        for pc in pieces:
            b = lay.buckets[pc.bucket_index]
            mine = L.rank_range(b, D, r)
            n = pc.gbuf_world.size
            assert n > 0
            # four ranges, one size, translations of one another
            for rg in (pc.gbuf_world_in_bucket, pc.gbuf_local, pc.param):
                assert rg.size == n
            assert pc.gbuf_world_in_bucket.start + b.offset == pc.gbuf_world.start
            assert pc.gbuf_local.start + mine.start == pc.gbuf_world.start
            assert pc.param.start + lay.param_world[pc.param_index].start == pc.gbuf_world.start
            assert mine.start <= pc.gbuf_world.start and pc.gbuf_world.end <= mine.end
            assert pc.param_index in b.params
            # shard placement: in bounds, phase-aligned with the world index
            assert pc.shard_offset == bases[pc.bucket_index] + pc.gbuf_local.start
            assert 0 <= pc.shard_offset and pc.shard_offset + n <= Ln
            assert (pc.shard_offset - pc.gbuf_world.start) % L.SHARD_PHASE == 0
            used.append((pc.shard_offset, pc.shard_offset + n))
            cover[pc.param_index].append((pc.param.start, pc.param.end))
        used.sort()
        assert all(used[i][1] <= used[i + 1][0] for i in range(len(used) - 1))
        # shard bases: bucket views in order, gaps < 8
        end = 0
        for b, base in zip(lay.buckets, bases):
            assert end <= base < end + L.SHARD_PHASE
            end = base + b.shard_numel(D)
        assert end == Ln
        # pieces sorted by world position
        assert [pc.gbuf_world.start for pc in pieces] == sorted(pc.gbuf_world.start for pc in pieces)
    # every parameter's pieces tile [0, n) exactly (split parameters included)
    for i, spans in cover.items():
        spans.sort()
        assert spans[0][0] == 0 and spans[-1][1] == lay.param_numel[i]
        assert all(spans[k][1] == spans[k + 1][0] for k in range(len(spans) - 1))


@pytest.mark.parametrize("name", ["tiny", "gpt2_small", "llama3_8b", "llama3_70b", "frag"])
def test_workload_invariants(name):
    w = W.get(name)
    lay = L.build_layout(w.param_numel, w.bucket_numel, w.dp_size)
    _check_invariants(lay)


def test_workload_sizes():
    # closed forms: with no padding the buffer is the parameter total and each
    # rank owns exactly N / D elements
    for name, nb in [("gpt2_small", 4), ("llama3_8b", 66), ("llama3_70b", 242)]:
        w = W.get(name)
        lay = L.build_layout(w.param_numel, w.bucket_numel, w.dp_size)
        assert len(lay.buckets) == nb
        assert lay.buffer_numel == w.total_numel
        for r in w.verify_ranks:
            assert L.owned_numel(lay, r) == w.total_numel // w.dp_size
    assert W.get("gpt2_small").total_numel == 124_439_808
    assert len(W.get("gpt2_small").param_numel) == 148
    assert len(W.get("llama3_8b").param_numel) == 291
    assert len(W.get("llama3_70b").param_numel) == 723
    w = W.get("frag")
    lay = L.build_layout(w.param_numel, w.bucket_numel, w.dp_size)
    assert len(w.param_numel) == 20064
    assert sum(L.owned_numel(lay, r) for r in range(16)) == w.total_numel


def _brute_pieces(sizes, bucket_numel, D, rank):
    """Element-by-element owner scan, independent of the interval arithmetic:
    replay the buffer one slot at a time and group consecutive slots of the
    same (owner rank, parameter)."""
    slots = []                      # (param or None, bucket) for every world slot
    bucket, filled = 0, 0
    for i, n in enumerate(sizes):
        slots += [(i, bucket)] * n
        filled += n
        if filled >= bucket_numel or i == len(sizes) - 1:
            while filled % D:
                slots.append((None, bucket))
                filled += 1
            bucket += 1
            filled = 0
    # bucket offsets and owners
    starts = {}
    for w, (_, b) in enumerate(slots):
        starts.setdefault(b, w)
    size = {b: sum(1 for s in slots if s[1] == b) for b in starts}
    out = []
    for w, (p, b) in enumerate(slots):
        owner = (w - starts[b]) // (size[b] // D)
        if owner != rank or p is None:
            continue
        pstart = next(k for k, s in enumerate(slots) if s[0] == p)
        rstart = starts[b] + rank * (size[b] // D)
        if out and out[-1][0] == p and out[-1][3] == w:
            out[-1][3] = w + 1
        else:
            out.append([p, b, w, w + 1, pstart, starts[b], rstart])
    return [(p, b, s, e, s - bo, e - bo, s - ro, e - ro, s - ps, e - ps)
            for p, b, s, e, ps, bo, ro in out]


def test_brute_force_owner_scan():
    rng = random.Random(1234)
    for _ in range(300):
        P = rng.randint(1, 10)
        sizes = [rng.randint(1, 40) for _ in range(P)]
        D = rng.randint(1, 7)
        bucket_numel = rng.randint(1, 120)
        lay = L.build_layout(sizes, bucket_numel, D)
        _check_invariants(lay)
        for r in range(D):
            got = [pc.as_tuple()[:10] for pc in L.rank_pieces(lay, r)]
            assert got == _brute_pieces(sizes, bucket_numel, D, r), (sizes, bucket_numel, D, r)


def test_padding_and_padding_only_rank():
    # 5 elements in one bucket at D=4 -> padded to 8, shard 2; rank 3 owns only padding
    lay = L.build_layout([3, 2], 100, 4)
    assert lay.buffer_numel == 8 and lay.buckets[0].padded_numel == 8
    assert L.rank_pieces(lay, 3) == []
    assert L.owned_numel(lay, 2) == 1
    assert [pc.param_index for pc in L.rank_pieces(lay, 1)] == [0, 1]


@pytest.mark.parametrize("args", [([], 10, 2), ([0], 10, 2), ([4], 0, 2), ([4], 10, 0)])
def test_bad_arguments(args):
    with pytest.raises(ValueError):
        L.build_layout(*args)
