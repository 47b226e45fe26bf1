"""The benchmark's work accounting (CPU): the closed form for the visible
(query, key) pairs that the FLOP counts rest on, against a direct count of
the mask, and the traffic lookup's refusal of unknown parts."""

import numpy as np
import pytest

import bench


@pytest.mark.parametrize("S", [1, 2, 63, 64, 65, 128, 129, 300, 1000])
@pytest.mark.parametrize("W", [0, 1, 2, 64, 127, 128, 129, 5000])
def test_pairs_per_head_matches_a_direct_count(S, W):
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    visible = (j <= i) & ((W == 0) | (i - j < W))
    assert bench.pairs_per_head(S, W) == int(visible.sum())


def test_workload_pair_counts():
    # the B = 4, S = 4096, 64-head step: full-causal and sliding-128 layers
    assert 4 * 64 * bench.pairs_per_head(4096, 0) == 2_148_007_936
    assert bench.pairs_per_head(4096, 128) == 128 * 129 // 2 + (4096 - 128) * 128


def test_traffic_lookup_refuses_unknown_parts():
    assert bench.measured_traffic("no_such_part_full") is None
