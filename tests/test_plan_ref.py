"""Pins for the CPU reference planner (the plan-byte specification the GPU planner must match).

The item extents are checked by brute force against the explicit visibility mask of the oracle's
reading of the causal rule, and the ordering and coverage against their definitions.
"""
import numpy as np
import pytest

from oracle import plan_ref
from oracle.mla_oracle import dense_visible
from workloads import cu_from_lens


def _tile(sq, m, bm):
    """Rows of query tile m: tiles are aligned to the sequence end, so row r belongs to tile
    (r + pad) // bm with pad = ceil(sq / bm) * bm - sq."""
    pad = -(-sq // bm) * bm - sq
    r = np.arange(sq)
    return r[(r + pad) // bm == m]


def test_tile_rows_partition_the_sequence():
    for sq, bm in [(1, 128), (127, 128), (128, 128), (129, 128), (1726, 128), (300, 64), (5, 16)]:
        t = -(-sq // bm)
        tiles = [_tile(sq, m, bm) for m in range(t)]
        assert np.array_equal(np.concatenate(tiles), np.arange(sq))
        assert all(len(x) == bm for x in tiles[1:]) and 1 <= len(tiles[0]) <= bm
        assert tiles[-1][-1] == sq - 1
        for m in range(t):
            first, last = plan_ref.tile_rows(sq, m, bm)
            assert (first, last) == (int(tiles[m][0]), int(tiles[m][-1]))


def _brute_kv_end(sq, sk, m, bm, causal):
    rows = _tile(sq, m, bm)
    vis = dense_visible(sq, sk, causal, rows=rows)
    cols = np.nonzero(vis.any(axis=0))[0]
    return 0 if cols.size == 0 else int(cols.max()) + 1


@pytest.mark.parametrize("lens_q,lens_k,causal,bm,bn", [
    ([128], [128], True, 128, 64),
    ([1726, 583, 280, 656, 885, 1680, 959, 246], None, True, 128, 64),
    ([2048] * 4, [16384, 12345, 8191, 4097], True, 128, 64),
    ([0, 5, 129, 1, 300], [7, 0, 129, 4096, 100], True, 64, 32),
    ([0, 5, 129, 1, 300], [7, 0, 129, 4096, 100], False, 256, 64),
    ([1, 129, 1, 129], [128, 512, 8192, 4096], True, 128, 128),
])
def test_plan_items_cover_and_order(lens_q, lens_k, causal, bm, bn):
    lens_k = lens_q if lens_k is None else lens_k
    cu_q, cu_k = cu_from_lens(lens_q), cu_from_lens(lens_k)
    max_q = max(lens_q)
    items = plan_ref.plan_items(cu_q, cu_k, max_q, bm, bn, causal)
    want = {(b, m) for b, sq in enumerate(lens_q) for m in range(-(-sq // bm))}
    got = [(it[0], it[1]) for it in items]
    assert sorted(got) == sorted(want) and len(got) == len(set(got))
    mt = -(-max_q // bm)
    for (b, m, nb, kv_end) in items:
        assert kv_end == _brute_kv_end(lens_q[b], lens_k[b], m, bm, causal)
        assert nb == -(-kv_end // bn)
    # sequence by sequence (more key blocks first, ties by b), each from its last tile to its first
    seq_blocks = [-(-n // bn) for n in lens_k]
    keys = [(-seq_blocks[it[0]], it[0], -it[1]) for it in items]
    assert keys == sorted(keys)


@pytest.mark.parametrize("lens_q,lens_k,causal,window,bm,bn", [
    ([1726, 583, 280], None, True, (256, -1), 128, 64),
    ([300, 5, 129], [700, 7, 129], False, (100, 30), 64, 32),
    ([2048, 100], [4096, 100], False, (0, 0), 128, 64),
    ([513, 64], [513, 1000], False, (-1, 17), 128, 64),
    ([200], [50], True, (10, -1), 64, 64),               # many rows see nothing
])
def test_plan_items_window_extent_brute_force(lens_q, lens_k, causal, window, bm, bn):
    """With a (left, right) window the block range of each item is exactly the span of keys some
    row of its tile can see, by brute force over the oracle's visibility mask (reading R18)."""
    lens_k = lens_q if lens_k is None else lens_k
    cu_q, cu_k = cu_from_lens(lens_q), cu_from_lens(lens_k)
    items = plan_ref.plan_items(cu_q, cu_k, max(lens_q), bm, bn, causal, window)
    assert len(items) == sum(-(-sq // bm) for sq in lens_q)
    for (b, m, nb, kv_end) in items:
        sq, sk = lens_q[b], lens_k[b]
        rows = _tile(sq, m, bm)
        cols = np.nonzero(dense_visible(sq, sk, causal, rows=rows, window=window).any(axis=0))[0]
        if cols.size == 0:
            assert nb == 0
            continue
        lo_blk, hi_blk = int(cols.min()) // bn, -(-(int(cols.max()) + 1) // bn)
        assert kv_end == int(cols.max()) + 1
        assert nb == hi_blk - lo_blk
        left = window[0]
        kv_start = min(max(int(rows[0]) + sk - sq - left, 0), sk) if left >= 0 else 0
        assert kv_start // bn == lo_blk
    mt = -(-max(lens_q) // bm)
    if window[0] >= 0:   # longest first, ties by slot
        keys = [(-it[2], it[0] * mt + it[1]) for it in items]
    else:                # sequence by sequence, each from its last tile
        keys = [(-(-(-lens_k[it[0]] // bn)), it[0], -it[1]) for it in items]
    assert keys == sorted(keys)


def test_plan_buffer_fill_and_capacity():
    cu = cu_from_lens([3, 200])
    buf, n = plan_ref.plan_buffer(cu, cu, 200, 64, 64, True, capacity=10)
    assert n == 5 and buf.shape == (10, 4)
    assert np.all(buf[n:] == -1)
    assert buf[0].tolist() == [1, 3, 4, 200]   # the sequence with more keys first, from its last tile
    assert buf[1:4, 1].tolist() == [2, 1, 0] and buf[4].tolist()[:2] == [0, 0]
    # tiles end at the sequence end: tile 0 of the 200-row sequence holds rows 0..7 (pad 56), so
    # under the causal mask it sees 8 keys in one block; tile 1 holds rows 8..71
    assert buf[3].tolist() == [1, 0, 1, 8] and buf[2].tolist() == [1, 1, 2, 72]
    with pytest.raises(ValueError):
        plan_ref.plan_buffer(cu, cu, 200, 64, 64, True, capacity=4)


def test_plan_unsorted_beyond_sort_capacity():
    lens = [1] * (plan_ref.SORT_CAPACITY + 1)
    lens[-1] = 1
    cu = cu_from_lens(lens)
    items = plan_ref.plan_items(cu, cu, 1, 64, 64, True)
    assert [it[0] for it in items] == list(range(len(lens)))
