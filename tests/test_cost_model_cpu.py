"""The alpha-beta cost model against every number the lecture prints for it.

Source: CMU 11-868 lecture 14 notes, "Distributed Training I": section 3.1
(pipelined ring broadcast: about 64 segments, 3.15 ms, vs 17.96 ms
unsegmented at K = 8, 64 MB, 25 GB/s, 5 us), section 3.4 (ring / tree /
naive regimes and the ~235 KB ring-tree crossover at K = 8, 5 us, 25 GB/s),
section 4.4 (6.12x / 2.09x / 0.77x speedups) and the answers to exercises
5, 6, 7, 8 and 11. MB and GB are 1e6 and 1e9 bytes, as the printed numbers
require. Host arithmetic only: runs without a GPU.
"""
import math

import pytest

import gradient_sync_zr_amd as zr

US = 1e-6
MB, GB = 1e6, 1e9


def printed(x, shown, decimals):
    """x rounds to the printed value `shown` at `decimals` places (half up)."""
    return abs(x - shown) <= 0.5 * 10 ** -decimals + 1e-12


def test_pipelined_broadcast_section_3_1():
    K, N, B, a = 8, 64 * MB, 25 * GB, 5 * US
    s, t = zr.zr_cost_best_broadcast_segments(K, N, a, B)
    assert s == 64
    assert printed(t * 1e3, 3.15, 2)
    assert printed(zr.zr_cost_pipelined_broadcast(K, N, 1, a, B) * 1e3, 17.96, 2)
    # without per-message latency the segmented time tends to N / B
    assert zr.zr_cost_pipelined_broadcast(K, N, 1 << 20, 0.0, B) == pytest.approx(N / B, rel=1e-4)


def test_regimes_and_crossover_section_3_4():
    K, a, b = 8, 5 * US, 25 * GB

    def fastest(n):
        t = {"ring": zr.zr_cost_ring_allreduce(K, n, a, b),
             "tree": zr.zr_cost_tree_allreduce(K, n, a, b),
             "naive": zr.zr_cost_naive_allreduce(K, n, a, b)}
        return min(t, key=t.get)

    assert fastest(1e3) == "naive" and fastest(1e4) == "naive"
    assert fastest(1e5) == "tree"
    assert fastest(1e6) == "ring" and fastest(1e9) == "ring"
    x = zr.zr_cost_ring_tree_crossover(K, a, b)
    assert printed(x / 1e3, 235, 0)
    assert zr.zr_cost_ring_allreduce(K, x, a, b) == pytest.approx(
        zr.zr_cost_tree_allreduce(K, x, a, b), rel=1e-12)


def test_exercise_5_ring_time_and_latency_share():
    K, N, b, a = 16, 1 * GB, 25 * GB, 10 * US
    t = zr.zr_cost_ring_allreduce(K, N, a, b)
    assert printed(t * 1e3, 75.3, 1)
    latency = t - zr.zr_cost_ring_allreduce(K, N, 0.0, b)
    assert printed(latency * 1e3, 0.3, 1)


def test_exercise_6_broadcast():
    K, N, B = 4, 100 * MB, 10 * GB
    assert printed(zr.zr_cost_pipelined_broadcast(K, N, 1, 0.0, B) * 1e3, 30.0, 1)
    assert printed(zr.zr_cost_pipelined_broadcast(K, N, 100, 0.0, B) * 1e3, 10.2, 1)
    assert printed(zr.zr_cost_pipelined_broadcast(K, N, 100, 20 * US, B) * 1e3, 12.2, 1)


def test_exercise_7_ring_naive_crossover():
    K, a, b = 8, 5 * US, 25 * GB
    x = zr.zr_cost_ring_naive_crossover(K, a, b)
    assert printed(x / 1e3, 122, 0)
    assert zr.zr_cost_ring_allreduce(K, x, a, b) == pytest.approx(
        zr.zr_cost_naive_allreduce(K, x, a, b), rel=1e-12)


def test_exercise_8_ring_side():
    # 16 devices, 2 GB of parameters, 25 GB/s: each device sends 3.75 GB, 0.15 s
    assert zr.zr_cost_ring_allreduce(16, 2 * GB, 0.0, 25 * GB) == pytest.approx(0.15, rel=1e-12)


def test_exercise_11_speedups():
    got = [zr.zr_cost_dp_speedup(K, 0.1, 1 * GB, 0.0, 25 * GB) for K in (2, 4, 8)]
    assert all(printed(x, w, 2) for x, w in zip(got, [1.11, 1.18, 1.21]))


def test_section_4_4_speedups():
    a, b, t1 = 5 * US, 25 * GB, 20e-3
    assert printed(zr.zr_cost_dp_speedup(8, t1, 10 * MB, a, b), 6.12, 2)
    assert printed(zr.zr_cost_dp_speedup(8, t1, 100 * MB, a, b), 2.09, 2)
    assert printed(zr.zr_cost_dp_speedup(2, t1, 400 * MB, a, b), 0.77, 2)


def test_reduce_scatter_is_half_the_ring_and_send_volume():
    # lecture 14, 3.2: reduce-scatter is the first K-1 of the 2(K-1) rounds
    for K in (2, 3, 8, 64):
        assert zr.zr_cost_ring_reduce_scatter(K, 1e9, 1e-5, 1e10) * 2 == pytest.approx(
            zr.zr_cost_ring_allreduce(K, 1e9, 1e-5, 1e10), rel=1e-12)
    assert zr.zr_cost_ring_allreduce(1, 1e9, 1e-5, 1e10) == 0.0


def test_invalid_arguments_give_nan():
    assert math.isnan(zr.zr_cost_ring_allreduce(0, 1.0, 0.0, 1.0))
    assert math.isnan(zr.zr_cost_tree_allreduce(4, -1.0, 0.0, 1.0))
    assert math.isnan(zr.zr_cost_naive_allreduce(4, 1.0, 0.0, 0.0))
    assert math.isnan(zr.zr_cost_pipelined_broadcast(1, 1.0, 1, 0.0, 1.0))
    assert zr.zr_cost_best_broadcast_segments(4, 1.0, 0.0, 0.0)[0] == -1
