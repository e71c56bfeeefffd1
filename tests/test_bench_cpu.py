"""CPU checks of the benchmark's work accounting: the algorithmic FLOP of the dense workloads come
from visible (query, key) pair counts, which must match the oracle's visibility rule."""
import numpy as np
import pytest

import bench
from oracle import mla_oracle as O


@pytest.mark.parametrize("sq,sk,causal,window", [
    (128, 128, True, (-1, -1)), (50, 80, False, (7, 3)), (80, 50, True, (10, -1)),
    (30, 30, False, (-1, -1)), (300, 4096, True, (256, -1)), (5, 0, True, (-1, -1)),
])
def test_pair_counts_match_visibility(sq, sk, causal, window):
    assert bench.dense_pairs([sq], [sk], causal, window) == int(O.dense_visible(sq, sk, causal, window=window).sum())


def test_headline_flops_closed_form():
    lens = [1726, 583, 280, 656, 885, 1680, 959, 246]
    pairs = sum(n * (n + 1) // 2 for n in lens)
    assert bench.dense_flops(lens, lens, 128, True) == 640 * 128 * pairs
