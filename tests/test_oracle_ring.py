"""Pins for the ring-buffer model (CPU only).

The step-by-step model and the closed form are written independently and checked
against each other, and the window they expose is checked against the set
definition of the sink-plus-recent window: after any number of appends the ring
holds exactly the sink positions and the last ``C - n_sink`` positions, and with
``C = n_sink + n_recent`` that is the window itself.
"""

import pytest
from hypothesis import given, settings, strategies as st

from oracle import attention as A
from oracle import ring as R


def test_logical_pos_small_table():
    # C = 6, n_sink = 2: positions 0,1 stay; 2.. cycle through slots 2..5
    got = [R.logical_pos(p, 2, 6) for p in range(12)]
    assert got == [0, 1, 2, 3, 4, 5, 2, 3, 4, 5, 2, 3]
    assert R.slot(3, 7, 2, 6) == 3 * 6 + 3
    with pytest.raises(ValueError):
        R.logical_pos(-1, 2, 6)
    with pytest.raises(ValueError):
        R.logical_pos(0, 6, 6)


@settings(max_examples=300, deadline=None)
@given(n_sink=st.integers(0, 6), span=st.integers(1, 12), T=st.integers(0, 60))
def test_model_matches_closed_form(n_sink, span, T):
    C = n_sink + span
    m = R.RingModel(1, C, n_sink)
    m.append(0, T)
    assert m.pos[0] == R.expected_pos_after(T, n_sink, C)
    assert m.T[0] == T


@settings(max_examples=300, deadline=None)
@given(n_sink=st.integers(0, 6), n_recent=st.integers(1, 12), T=st.integers(0, 60))
def test_full_ring_without_slack_holds_exactly_the_window(n_sink, n_recent, T):
    C = n_sink + n_recent
    pos = R.expected_pos_after(T, n_sink, C)
    held = sorted(p for p in pos if p >= 0)
    assert held == A.window_positions(T, n_sink, n_recent).tolist()
    valid = R.window_valid(pos, T, n_sink, n_recent)
    assert all(v == (p >= 0) for v, p in zip(valid, pos))


@settings(max_examples=300, deadline=None)
@given(n_sink=st.integers(0, 5), n_recent=st.integers(1, 10), slack=st.integers(0, 6),
       T=st.integers(0, 50), back=st.integers(0, 6))
def test_slack_absorbs_rollback(n_sink, n_recent, slack, T, back):
    # Reading of the "+d slack": with at least `back` spare slots, rolling back
    # `back` speculative positions leaves every position of the new window in the
    # ring, so the windowed read after the rollback is exact.
    C = n_sink + n_recent + slack
    m = R.RingModel(1, C, n_sink)
    m.append(0, T)
    back = min(back, T)
    m.rollback(0, T - back)
    T2 = T - back
    valid = R.window_valid(m.pos[0], T2, n_sink, n_recent)
    read = sorted(p for p, v in zip(m.pos[0], valid) if v)
    want = A.window_positions(T2, n_sink, n_recent).tolist()
    if back <= slack:
        assert read == want
    else:
        assert set(read) <= set(want)


@settings(max_examples=200, deadline=None)
@given(n_sink=st.integers(0, 5), span=st.integers(1, 10), T0=st.integers(0, 40), n=st.integers(0, 40))
def test_bulk_append_equals_one_by_one(n_sink, span, T0, n):
    C = n_sink + span
    a = R.RingModel(1, C, n_sink)
    b = R.RingModel(1, C, n_sink)
    a.append(0, T0)
    b.append(0, T0)
    a.append(0, n)
    for _ in range(n):
        b.append(0)
    assert a.pos == b.pos and a.T == b.T


def test_rebuild_from_kept_positions_equals_incremental():
    # Resume: writing only the positions the ring keeps (sink + last C - n_sink)
    # gives the same contents as appending every position.
    n_sink, C, T = 4, 64, 1000
    inc = R.RingModel(1, C, n_sink)
    inc.append(0, T)
    kept = list(range(min(n_sink, T))) + list(range(max(n_sink, T - (C - n_sink)), T))
    rebuilt = [-1] * C
    for p in kept:
        rebuilt[R.logical_pos(p, n_sink, C)] = p
    assert rebuilt == inc.pos[0]


def test_rings_are_independent_per_request():
    m = R.RingModel(3, 8, 2)
    m.append(0, 5)
    m.append(2, 20)
    assert m.pos[1] == [-1] * 8
    assert m.pos[0] == R.expected_pos_after(5, 2, 8)
    assert m.pos[2] == R.expected_pos_after(20, 2, 8)


def test_large_ring_wrap_after_ten_thousand_appends():
    # The 1M-context stack workload: 4 + 4092 slots after 1,048,576 + 10,000 appends.
    n_sink, C = 4, 4096
    T = 1048576 + 10000
    pos = R.expected_pos_after(T, n_sink, C)
    assert sorted(pos) == A.window_positions(T, n_sink, C - n_sink).tolist()
    assert pos[:4] == [0, 1, 2, 3]
    # position T-1 sits at n_sink + (T-1-n_sink) mod 4092
    assert pos[n_sink + (T - 1 - n_sink) % (C - n_sink)] == T - 1
