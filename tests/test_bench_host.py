"""Host-side logic of bench.py: path roofline sum and receiver statistics
(small hand-made inputs; no GPU)."""
import types

import pytest
import torch

import bench


def test_path_roofline_sums_the_binding_peak():
    work = {"g": ("flop", 2.5e12), "c": ("byte", 8e9)}  # 1 ms each at the peaks
    kernels = {"g": {"launches_per_step": 1}, "c": {"launches_per_step": 2}}
    r = bench.path_roofline(kernels, work, ms=6.0)
    assert r["ms_at_peaks"] == pytest.approx(3.0)
    assert r["frac"] == pytest.approx(0.5)


def test_path_roofline_ignores_kernels_not_run():
    r = bench.path_roofline({}, {"g": ("flop", 2.5e12)}, ms=1.0)
    assert r["ms_at_peaks"] == 0.0


def _st(counts, cap_recv, R):
    d = types.SimpleNamespace(n_ranks=R, cap_recv=cap_recv)
    return types.SimpleNamespace(d=d, recv_counts=torch.tensor(counts, dtype=torch.int64))


def test_receiver_stats_fixed_capacity():
    # 2 ranks x (2 waves x 2 experts); capacity 5
    st = _st([1, 2, 3, 4, 9, 0, 7, 1], cap_recv=5, R=2)
    pct, hot = bench.receiver_stats(st)
    # dropped: 9 - 5 = 4 and 7 - 5 = 2 of 27
    assert pct == pytest.approx(100.0 * 6 / 27)
    # kept: rank 0 = 10, rank 1 = 5 + 0 + 5 + 1 = 11
    assert hot == 1


def test_receiver_stats_ragged_keeps_everything():
    st = _st([1, 2, 30, 4], cap_recv=0, R=2)
    pct, hot = bench.receiver_stats(st)
    assert pct == 0.0 and hot == 1


def test_step_stats_median_and_mean():
    s = bench.step_stats([3.0, 1.0, 2.0, 10.0])
    assert s["median"] == pytest.approx(2.5) and s["mean"] == pytest.approx(4.0)
    assert s["min"] == 1.0 and s["max"] == 10.0
    assert bench.step_stats([5.0, 1.0, 2.0])["median"] == 2.0


def test_metric_names_tokens_rooflines_and_drops():
    assert bench.METRIC.startswith("routed tokens/s through MoE layer on 1 MI355X")
    assert "roofline" in bench.METRIC and "drop %" in bench.METRIC
