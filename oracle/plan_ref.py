"""CPU reference of the varlen tile plan: the specification of the plan bytes.

TEST INFRASTRUCTURE ONLY (imported by ``tests/`` and nowhere in the product path). The GPU
planner must produce exactly these int32 words.

Prior art on the pages: a device-side planner for ragged batches, with a helper that clears its
counters (page "Mojo module mla": ``mla_prefill_plan_kernel``, ``set_buffer_lengths_to_zero``),
and a metadata call run before the attention operator whose int32 output of fixed size holds the
operator's task table (page "SparseFlashMla", Description: ``SparseFlashMlaMetadata``;
Constraints: ``metadata``). Neither page gives a format, so the format below is this library's
own.

Plan format
-----------
Slots: ``slot = b * Mt + m`` for sequence ``b`` in [0, B) and query tile ``m`` in [0, Mt) with
``Mt = ceil(max_seqlen_q / BM)``. A slot is a work item iff ``m < T_b = ceil(Sq_b / BM)``.
Query tiles are aligned to the end of their sequence: tile ``m`` holds the rows
``[m*BM - pad_b, (m+1)*BM - pad_b)`` that exist, with ``pad_b = T_b*BM - Sq_b`` (the leftover
``Sq_b mod BM`` rows form tile 0, where causal rows see the fewest keys); see ``tile_rows``.

For an item: ``kv_end`` is the number of leading keys any row of the tile can see:
``Sk_b`` without a right limit; with the bottom-right causal mask (right window 0) or a right
window ``r >= 0`` it is ``clamp(i_last + Sk_b - Sq_b + r + 1, 0, Sk_b)`` where ``i_last`` is the
tile's last row. With a left window ``l >= 0`` the first key any row can see is
``kv_start = clamp(i_first + Sk_b - Sq_b - l, 0, Sk_b)`` with ``i_first`` the tile's first row
(else 0). ``n_blocks`` counts the key
blocks from ``kv_start // BN`` up to ``ceil(kv_end / BN)``, and is 0 when ``kv_end <= kv_start``;
without a left window it is ``ceil(kv_end / BN)``. The dense kernel recomputes ``kv_start // BN``
from ``(m, Sq_b, Sk_b, l)``.

Each item is four int32 words ``(b, m, n_blocks, kv_end)``. Items are ordered sequence by
sequence, sequences with more key blocks first (``min(ceil(Sk_b / BN), MAX_BLOCKS)`` descending,
ties by ``b`` ascending), and within a sequence from its last query tile to its first (``m``
descending); with a left window (``l >= 0``) they are ordered longest first instead:
``n_blocks`` descending, ties by slot ascending. When there are more than ``SORT_CAPACITY``
slots the items stay in slot order.
Words past the last item, up to ``capacity`` items, are -1.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

SORT_CAPACITY = 16384
MAX_BLOCKS = 0x3FFFE


def tile_rows(sq: int, m: int, bm: int) -> Tuple[int, int]:
    """Rows [first, last] of sequence rows held by query tile m (tiles aligned to the sequence end)."""
    n_tiles = -(-sq // bm)
    row0 = m * bm - (n_tiles * bm - sq)
    return max(row0, 0), row0 + bm - 1


def plan_items(cu_q: Sequence[int], cu_k: Sequence[int], max_seqlen_q: int, bm: int, bn: int,
               causal: bool, window: Tuple[int, int] = (-1, -1)) -> list:
    """The work items as (b, m, n_blocks, kv_end) tuples, in plan order; window = (left, right),
    -1 = unlimited, causal forces right = 0."""
    left, right = int(window[0]), int(window[1])
    if causal:
        right = 0
    b_count = len(cu_q) - 1
    mt = -(-int(max_seqlen_q) // bm) if max_seqlen_q > 0 else 0
    items = []
    for b in range(b_count):
        sq = int(cu_q[b + 1]) - int(cu_q[b])
        sk = int(cu_k[b + 1]) - int(cu_k[b])
        for m in range(-(-sq // bm)):
            i_first, i_last = tile_rows(sq, m, bm)
            if right >= 0:
                kv_end = min(max(i_last + sk - sq + right + 1, 0), sk)
            else:
                kv_end = sk
            kv_start = min(max(i_first + sk - sq - left, 0), sk) if left >= 0 else 0
            n_blocks = 0 if kv_end <= kv_start else -(-kv_end // bn) - kv_start // bn
            if left < 0:
                order = (-min(-(-sk // bn), MAX_BLOCKS), b, -m)
            else:
                order = (-min(n_blocks, MAX_BLOCKS), b * mt + m, 0)
            items.append((order, (b, m, n_blocks, kv_end)))
    if b_count * mt <= SORT_CAPACITY:
        items.sort(key=lambda it: it[0])
    return [it[1] for it in items]


def plan_buffer(cu_q: Sequence[int], cu_k: Sequence[int], max_seqlen_q: int, bm: int, bn: int,
                causal: bool, capacity: int, window: Tuple[int, int] = (-1, -1)) -> Tuple[np.ndarray, int]:
    """The full plan buffer (int32 [capacity, 4]) and the item count."""
    items = plan_items(cu_q, cu_k, max_seqlen_q, bm, bn, causal, window)
    if len(items) > capacity:
        raise ValueError("plan capacity too small")
    buf = np.full((capacity, 4), -1, dtype=np.int32)
    if items:
        buf[: len(items)] = np.asarray(items, dtype=np.int32)
    return buf, len(items)
