"""Pins for the step-cost identity and KV accounting against the pages' printed figures."""

import json
import math
import os

import pytest

from oracle import accounting as acc

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def test_dropped_fraction_at_1m_matches_printed_99_percent():
    g = GOLD["dropped_entries_at_1m"]
    f = acc.dropped_fraction(g["context"], g["window"])
    assert f == 1.0 - 4096 / 1048576                      # 0.99609375
    assert math.floor(f * 100) / 100 == g["value"]           # "about 99 %": 99.6 %, truncated
    assert acc.dropped_fraction(100, 4096) == 0.0         # short context: nothing dropped


def test_reclaimed_fraction_spans_printed_range():
    # One draft attention layer beside L_attn target attention layers of equal KV
    # size: the native draft pool is 1/(L_attn + 1) of all KV, which is the printed
    # 7.7-11 % for L_attn between 12 and 8.
    g = GOLD["reclaimed_kv_range"]
    T = 1 << 20
    hi = acc.reclaimed_fraction(T, 0, 8, T)
    lo = acc.reclaimed_fraction(T, 0, 12, T)
    assert hi == pytest.approx(1 / 9) and lo == pytest.approx(1 / 13)
    assert round(lo, 3) == g["lo"] and round(hi, 2) == g["hi"]
    # the 8-layer stack workload with a 4096-slot ring after 1M + 10,000 appends
    Tm = 1048576 + 10000
    f = acc.reclaimed_fraction(Tm, 4096, 8, Tm)
    assert f == pytest.approx((Tm - 4096) / (9 * Tm))
    assert g["lo"] <= f <= g["hi"] + 0.001
    assert round(f, 5) == 0.11068


def test_eq1_step_cost_and_hybrid_depth7_figures():
    g = GOLD["hybrid_120b_depth7"]
    # +28.3 % read as t_native / t_window - 1 with a 7.3 ms saving
    t_w = g["saving_ms"] / g["gain"]
    t_n = t_w + g["saving_ms"]
    up, down = acc.cost_reduction(t_n, t_w)
    assert up == pytest.approx(g["gain"])
    assert down == pytest.approx(g["saving_ms"] / t_n)
    assert 25.0 < t_w < 26.5 and 32.5 < t_n < 33.5
    # the 1.2 ms bookkeeping drop is about 16 % of the saving and about 4 % of the step
    d = g["tovh_native_ms"] - g["tovh_window_ms"]
    assert round(d / g["saving_ms"], 2) == g["share_of_saving"]
    assert round(d / t_n, 2) == g["share_of_step"] or round(d / t_w, 2) == 0.05
    # Eq. 1 is additive with gamma draft forwards
    assert acc.step_cost(10.0, 2.0, 1.5, 7) == 10.0 + 2.0 + 7 * 1.5
    with pytest.raises(ValueError):
        acc.step_cost(1, 1, 1, -1)


def test_eq3_latency_ratio():
    g = GOLD["hybrid_120b_depth7"]
    t_w = g["saving_ms"] / g["gain"]
    t_n = t_w + g["saving_ms"]
    r = acc.latency_ratio(t_n, t_w, g["al_native"], g["al_window"])
    assert r == pytest.approx((1 + g["gain"]) * g["al_window"] / g["al_native"])
    assert acc.latency_ratio(2.0, 1.0, 3.0, 3.0) == 2.0        # matched acceptance: cost ratio


def test_both_readings_of_gain_range():
    g = GOLD["per_step_gain_range"]
    for gain in (g["lo"], g["hi"]):
        up, down = acc.cost_reduction(1.0 + gain, 1.0)
        assert up == pytest.approx(gain)
        assert down == pytest.approx(gain / (1 + gain))
    with pytest.raises(ValueError):
        acc.cost_reduction(0.0, 1.0)


def test_kv_bytes_of_workloads():
    assert acc.kv_bytes(1048576, 2, 256) == 2 * 1024 ** 3          # 1M, 2 kv heads, D 256: 2 GiB
    assert acc.kv_bytes(4096, 2, 256) == 8 * 1024 ** 2              # the 4096-slot window: 8 MiB
    assert acc.kv_bytes(8192, 2, 128) == 8 * 1024 ** 2
    assert math.isclose(acc.kv_bytes(1, 4, 128), 2048)
