"""Offloaded-linear planner on the CPU (dkv_linear_plan_inspect, no HIP call).

Every (output row, k) pair must be covered exactly once, rows [0, floor(r N))
by host items and the rest by HBM items (the oracle's split rule), blocks never
straddle the tiers, and partial slots are unique and used only when a block is
split over K.
"""
import numpy as np
import pytest

import oracle as O

dkv_lib = pytest.importorskip("decode_attention_host_amd._lib")
from decode_attention_host_amd.api import linear_plan_inspect, reset_tuning, set_tuning  # noqa: E402


@pytest.mark.parametrize("N,K", [(1, 8), (100, 64), (1024, 4096), (14336, 4096), (4096, 14336), (333, 2056)])
@pytest.mark.parametrize("ratio", [0.0, 0.3, 0.5, 0.9, 1.0])
def test_linear_plan_covers_rows_and_k(N, K, ratio):
    items, info = linear_plan_inspect(N, K, ratio, 256)
    nh = O.linear_split_rows(ratio, N)
    cover = np.zeros(N, dtype=np.int64)   # total k covered per row
    slots = [int(s) for s in items[:, 5] if s >= 0]
    assert len(slots) == len(set(slots)) == info["num_splits"]
    for pool in (0, 1):   # a tier's items all write partials (K split) or none do
        tier = items[items[:, 0] == pool]
        assert np.all(tier[:, 5] >= 0) or np.all(tier[:, 5] < 0)
    for pool, r0, nr, k0, k1, slot in items:
        assert 1 <= nr <= 64 and 0 <= k0 < k1 <= K and k0 % 32 == 0
        rows = np.arange(r0, r0 + nr)
        assert np.all((rows < nh) == (pool == 0)), "block straddles the tiers"
        cover[rows] += k1 - k0
    assert np.all(cover == K)
    assert info["host_bytes"] == nh * K * 2 and info["dev_bytes"] == (N - nh) * K * 2
    assert (info["host_items"] == 0) == (nh == 0) and (info["dev_items"] == 0) == (nh == N)


def test_linear_plan_k_split_follows_tuning():
    try:
        set_tuning(dev_chunk=512)
        items, info = linear_plan_inspect(128, 4096, 0.0, 256)
    finally:
        reset_tuning()
    assert set(int(k1 - k0) for _, _, _, k0, k1, _ in items) == {512}
    assert info["num_splits"] == len(items) == 2 * 8


def test_linear_validation():
    with pytest.raises(dkv_lib.DkvError):
        linear_plan_inspect(64, 100, 0.5, 256)    # K not a multiple of 8
    with pytest.raises(dkv_lib.DkvError):
        linear_plan_inspect(64, 64, 1.5, 256)     # ratio outside [0, 1]
    with pytest.raises(dkv_lib.DkvError):
        linear_plan_inspect(0, 64, 0.5, 256)
