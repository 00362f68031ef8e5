"""Pins for the float64 attention oracle (CPU only).

Each test checks the oracle against something other than itself: brute force in
pure Python (math.fsum / math.exp), closed forms and special cases, invariants of
softmax attention, and the window statements of the pages.  A plausible slip in
the oracle (a dropped max subtraction, a missing normalisation, a wrong GQA index,
an off-by-one in the window or the causal limit, a transposed operand) fails at
least one of them.
"""

import math

import numpy as np
import pytest

from oracle import attention as A
from workloads import bf16_round, bf16_to_f32


def _bf16(rng, *shape, scale=1.0):
    return bf16_round((rng.standard_normal(shape) * scale).astype(np.float32))


def _brute(q, K, V, scale):
    """Pure-Python softmax attention of one query over all rows of K/V."""
    q = [float(x) for x in q]
    logits = [scale * math.fsum(qi * float(k) for qi, k in zip(q, row)) for row in K]
    m = max(logits)
    w = [math.exp(s - m) for s in logits]
    l = math.fsum(w)
    D = len(V[0])
    o = [math.fsum(w[j] * float(V[j][c]) for j in range(len(w))) / l for c in range(D)]
    return o, m + math.log(l)


def test_widen_bf16_known_values():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x3EAA, 0x7F80, 0x0001], dtype=np.uint16)
    v = A.widen_bf16(bits)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 0.0
    assert math.copysign(1.0, v[3]) == -1.0
    assert v[4] == float.fromhex("0x1.54p-2")            # 0x3EAA: exponent 0x7D, mantissa 0x2A
    assert v[5] == math.inf
    assert v[6] == 2.0 ** -133                            # smallest bf16 subnormal
    with pytest.raises(TypeError):
        A.widen_bf16(np.zeros(3, dtype=np.float32))


@pytest.mark.parametrize("N,D,R", [(1, 4, 1), (7, 16, 3), (33, 8, 2), (64, 16, 4)])
def test_attend_matches_pure_python_bruteforce(N, D, R):
    rng = np.random.default_rng(N * 100 + D)
    q, K, V = _bf16(rng, R, D), _bf16(rng, N, D), _bf16(rng, N, D)
    qf, Kf, Vf = A.widen_bf16(q), A.widen_bf16(K), A.widen_bf16(V)
    scale = 1.0 / math.sqrt(D)
    o, lse = A.attend(q, K, V, scale)
    for r in range(R):
        ob, lb = _brute(qf[r], Kf, Vf, scale)
        assert np.max(np.abs(o[r] - ob)) <= 1e-12
        assert abs(lse[r] - lb) <= 1e-12


def test_single_key_returns_its_value_and_logit():
    rng = np.random.default_rng(1)
    q, K, V = _bf16(rng, 3, 8), _bf16(rng, 1, 8), _bf16(rng, 1, 8)
    o, lse = A.attend(q, K, V, 0.7)
    assert np.array_equal(o, np.repeat(A.widen_bf16(V), 3, axis=0))
    s0 = 0.7 * (A.widen_bf16(q) @ A.widen_bf16(K)[0])
    assert np.allclose(lse, s0, rtol=0, atol=1e-15)


def test_zero_query_is_uniform_mean():
    rng = np.random.default_rng(2)
    N, D = 50, 16
    K, V = _bf16(rng, N, D), _bf16(rng, N, D)
    o, lse = A.attend(np.zeros((1, D)), K, V, 1.0)
    assert np.allclose(o[0], A.widen_bf16(V).mean(axis=0), rtol=0, atol=1e-14)
    assert abs(lse[0] - math.log(N)) <= 1e-14


def test_constant_logit_shift_leaves_output_moves_lse():
    # Append a constant feature: every logit grows by c * scale, so o is unchanged
    # and lse shifts by exactly that amount.
    rng = np.random.default_rng(3)
    N, D, c, scale = 40, 8, 3.0, 0.5
    q, K, V = A.widen_bf16(_bf16(rng, 2, D)), A.widen_bf16(_bf16(rng, N, D)), A.widen_bf16(_bf16(rng, N, D))
    o0, l0 = A.attend(q, K, V, scale)
    q1 = np.concatenate([q, np.full((2, 1), c)], axis=1)
    K1 = np.concatenate([K, np.ones((N, 1))], axis=1)
    o1, l1 = A.attend(q1, K1, V, scale)
    assert np.max(np.abs(o1 - o0)) <= 1e-13
    assert np.max(np.abs(l1 - (l0 + c * scale))) <= 1e-12


def test_large_logits_do_not_overflow():
    # Logits near 1000 overflow exp() unless the maximum is subtracted first.
    K = np.array([[1000.0], [999.0], [998.0]])
    V = np.array([[1.0], [2.0], [4.0]])
    o, lse = A.attend(np.array([[1.0]]), K, V, 1.0)
    w = np.exp([0.0, -1.0, -2.0])
    assert abs(o[0, 0] - (w @ V[:, 0]) / w.sum()) <= 1e-13
    assert abs(lse[0] - (1000.0 + math.log(w.sum()))) <= 1e-12


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(4)
    N, D = 30, 8
    K, V = A.widen_bf16(_bf16(rng, N, D)), A.widen_bf16(_bf16(rng, N, D))
    q = np.zeros((1, D))
    q[0, 0] = 1.0
    K[:, 0] = 0.0
    K[17, 0] = 50.0                                   # +50 logit on key 17
    o, _ = A.attend(q, K, V, 1.0)
    assert np.max(np.abs(o[0] - V[17])) <= N * math.exp(-50) * 10


def test_key_permutation_invariance():
    rng = np.random.default_rng(5)
    q, K, V = _bf16(rng, 4, 16), _bf16(rng, 100, 16), _bf16(rng, 100, 16)
    perm = rng.permutation(100)
    o0, l0 = A.attend(q, K, V, 0.25)
    o1, l1 = A.attend(q, K[perm], V[perm], 0.25)
    assert np.max(np.abs(o0 - o1)) <= 1e-14 and np.max(np.abs(l0 - l1)) <= 1e-13


def test_transposed_operand_would_differ():
    # Non-square shapes: a swapped K/V or q/K role cannot go unnoticed.
    rng = np.random.default_rng(6)
    q, K, V = _bf16(rng, 2, 8), _bf16(rng, 11, 8), _bf16(rng, 11, 8)
    o, _ = A.attend(q, K, V, 1.0)
    o_swapped, _ = A.attend(q, V, K, 1.0)
    assert np.max(np.abs(o - o_swapped)) > 1e-3


@pytest.mark.parametrize("L,ns,nr", [(0, 4, 8), (3, 4, 8), (10, 4, 8), (12, 4, 8), (13, 4, 8),
                                     (100, 4, 8), (100, 0, 8), (100, 4, 0), (100, 200, 5), (5000, 4, 1020)])
def test_window_positions_match_set_definition(L, ns, nr):
    got = A.window_positions(L, ns, nr)
    want = [p for p in range(L) if p < ns or p >= L - nr]
    assert got.tolist() == want
    assert len(set(got.tolist())) == len(got)
    assert len(got) == min(L, ns + nr)


def _kv(rng, L, Hkv, D):
    return _bf16(rng, L, Hkv, D), _bf16(rng, L, Hkv, D)


def test_gqa_head_mapping_bruteforce():
    rng = np.random.default_rng(7)
    Hq, Hkv, D, L = 6, 3, 8, 9
    q = _bf16(rng, Hq, D)
    K, V = _kv(rng, L, Hkv, D)
    o, lse = A.draft_full(q, K, V, L, 0.3)
    qf, Kf, Vf = A.widen_bf16(q), A.widen_bf16(K), A.widen_bf16(V)
    for h in range(Hq):
        g = h // (Hq // Hkv)                         # heads 0,1 -> kv 0; 2,3 -> kv 1; 4,5 -> kv 2
        ob, lb = _brute(qf[h], Kf[:, g, :], Vf[:, g, :], 0.3)
        assert np.max(np.abs(o[h] - ob)) <= 1e-12 and abs(lse[h] - lb) <= 1e-12


@pytest.mark.parametrize("L,ns,nr", [(50, 4, 46), (50, 4, 60), (50, 50, 0), (1, 4, 1), (8, 4, 4)])
def test_window_equals_full_when_window_covers_context(L, ns, nr):
    rng = np.random.default_rng(L + ns)
    q = _bf16(rng, 8, 16)
    K, V = _kv(rng, L, 2, 16)
    of, lf = A.draft_full(q, K, V, L, 0.25)
    ow, lw = A.draft_window(q, K, V, L, ns, nr, 0.25)
    assert np.array_equal(of, ow) and np.array_equal(lf, lw)


@pytest.mark.parametrize("L,ns,nr", [(200, 4, 20), (200, 0, 30), (200, 10, 1), (64, 4, 28)])
def test_window_equals_explicitly_masked_full(L, ns, nr):
    # A second route: full attention with the logits of every key outside the
    # sink/recent mask set to -inf (mask built with a Python loop).
    rng = np.random.default_rng(L * 7 + nr)
    Hq, Hkv, D = 4, 2, 8
    q = _bf16(rng, Hq, D)
    K, V = _kv(rng, L, Hkv, D)
    ow, lw = A.draft_window(q, K, V, L, ns, nr, 0.5)
    mask = np.array([(p < ns) or (p >= L - nr) for p in range(L)])
    qf, Kf, Vf = A.widen_bf16(q), A.widen_bf16(K), A.widen_bf16(V)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        s = 0.5 * (Kf[:, g, :] @ qf[h])
        s[~mask] = -np.inf
        w = np.exp(s - s.max())
        ref = (w @ Vf[:, g, :]) / w.sum()
        assert np.max(np.abs(ow[h] - ref)) <= 1e-13
        assert abs(lw[h] - (s.max() + math.log(w.sum()))) <= 1e-12


def test_needle_outside_window_moves_full_not_window():
    # A planted high-logit key just outside the recent window (and not a sink)
    # changes the native draft's output but not the windowed draft's.
    rng = np.random.default_rng(8)
    L, ns, nr, D = 300, 4, 64, 16
    q = _bf16(rng, 2, D)
    K, V = _kv(rng, L, 1, D)
    Kf = A.widen_bf16(K)
    o_full0, _ = A.draft_full(q, Kf, A.widen_bf16(V), L, 1.0)
    o_win0, _ = A.draft_window(q, Kf, A.widen_bf16(V), L, ns, nr, 1.0)
    needle = L - nr - 1
    K2 = Kf.copy()
    K2[needle, 0, :] = 20.0 * np.sign(A.widen_bf16(q)[0])
    o_full1, _ = A.draft_full(q, K2, A.widen_bf16(V), L, 1.0)
    o_win1, _ = A.draft_window(q, K2, A.widen_bf16(V), L, ns, nr, 1.0)
    assert np.max(np.abs(o_full1 - o_full0)) > 0.1
    assert np.array_equal(o_win1, o_win0)


def test_verify_single_query_is_full_draft():
    rng = np.random.default_rng(9)
    L, Hq, Hkv, D = 77, 8, 2, 16
    q = _bf16(rng, 1, Hq, D)
    K, V = _kv(rng, L, Hkv, D)
    ov, lv = A.verify(q, K, V, L, 0.25)
    of, lf = A.draft_full(q[0], K, V, L, 0.25)
    assert np.array_equal(ov[0], of) and np.array_equal(lv[0], lf)


def test_verify_query_i_sees_its_causal_prefix():
    rng = np.random.default_rng(10)
    S, n_q, Hq, Hkv, D = 40, 5, 4, 1, 8
    L = S + n_q
    q = _bf16(rng, n_q, Hq, D)
    K, V = _kv(rng, L + 3, Hkv, D)                   # extra trailing keys must be ignored
    ov, lv = A.verify(q, K, V, L, 0.5)
    for i in range(n_q):
        of, lf = A.draft_full(q[i], K, V, S + i + 1, 0.5)
        assert np.array_equal(ov[i], of) and np.array_equal(lv[i], lf)
    # the last query sees every key; the first does not see the other appended ones
    of_all, _ = A.draft_full(q[0], K, V, L, 0.5)
    assert np.max(np.abs(ov[0] - of_all)) > 1e-6


def test_tree_verify_with_chain_masks_is_the_causal_verify():
    rng = np.random.default_rng(14)
    S, n_q, Hq, Hkv, D = 33, 5, 4, 2, 8
    L = S + n_q
    q = _bf16(rng, n_q, Hq, D)
    K, V = _kv(rng, L, Hkv, D)
    ot, lt = A.verify_tree(q, K, V, L, [(1 << (i + 1)) - 1 for i in range(n_q)], 0.5)
    ov, lv = A.verify(q, K, V, L, 0.5)
    assert np.array_equal(ot, ov) and np.array_equal(lt, lv)


def test_tree_verify_bruteforce_on_a_small_tree():
    """Root 0 with children 1 and 2, node 3 under 1: each query against pure-Python
    attention over the prefix plus its ancestors."""
    rng = np.random.default_rng(15)
    S, Hq, Hkv, D = 9, 2, 1, 4
    masks = [0b0001, 0b0011, 0b0101, 0b1011]
    n_q = len(masks)
    L = S + n_q
    q = _bf16(rng, n_q, Hq, D)
    K, V = _kv(rng, L, Hkv, D)
    o, lse = A.verify_tree(q, K, V, L, masks, 0.7)
    Kf, Vf, qf = bf16_to_f32(K), bf16_to_f32(V), bf16_to_f32(q)
    for i, mk in enumerate(masks):
        rows = list(range(S)) + [S + a for a in range(n_q) if (mk >> a) & 1]
        for h in range(Hq):
            bo, bl = _brute(qf[i, h], [Kf[r, 0] for r in rows], [Vf[r, 0] for r in rows], 0.7)
            assert np.max(np.abs(o[i, h] - np.array(bo))) < 1e-12
            assert abs(lse[i, h] - bl) < 1e-12


def test_tree_verify_ignores_non_ancestors_and_empty_masks_read_the_prefix():
    rng = np.random.default_rng(16)
    S, Hq, Hkv, D = 20, 2, 1, 8
    masks = [0b001, 0b011, 0b101]
    n_q = 3
    L = S + n_q
    q = _bf16(rng, n_q, Hq, D)
    K, V = _kv(rng, L, Hkv, D)
    base, _ = A.verify_tree(q, K, V, L, masks, 1.0)
    V2 = A.widen_bf16(V).copy()
    V2[S + 1] += 50.0                           # appended position 1: not an ancestor of query 2
    moved, _ = A.verify_tree(q, K, V2, L, masks, 1.0)
    assert np.array_equal(moved[2], base[2]) and np.max(np.abs(moved[1] - base[1])) > 1e-3
    o0, l0 = A.verify_tree(q, K, V, L, [0, 0, 0], 1.0)
    of, lf = A.draft_full(q[1], K, V, S, 1.0)
    assert np.allclose(o0[1], of, rtol=0, atol=1e-14) and np.allclose(l0[1], lf, rtol=0, atol=1e-14)


def test_context_window_covering_everything_is_the_causal_verify():
    """A window that covers the whole context turns the windowed draft context
    pass into the native one, which is the causal verify over the draft KV."""
    rng = np.random.default_rng(11)
    S, n_q, Hq, Hkv, D = 50, 6, 4, 2, 8
    L = S + n_q
    q = _bf16(rng, n_q, Hq, D)
    K, V = _kv(rng, L, Hkv, D)
    oc, lc = A.draft_context_window(q, K, V, L, 4, L, 0.5)
    ov, lv = A.verify(q, K, V, L, 0.5)
    assert np.allclose(oc, ov, rtol=0, atol=1e-13) and np.allclose(lc, lv, rtol=0, atol=1e-13)


def test_context_window_of_one_recent_key_returns_that_key():
    """No sink and a one-key window: query i sees only its own position, so its
    output is that key's value and its lse that key's logit (a closed form)."""
    rng = np.random.default_rng(12)
    S, n_q, Hq, Hkv, D = 30, 4, 4, 2, 8
    L = S + n_q
    q = _bf16(rng, n_q, Hq, D)
    K, V = _kv(rng, L, Hkv, D)
    Kf, Vf, qf = A.widen_bf16(K), A.widen_bf16(V), A.widen_bf16(q)
    oc, lc = A.draft_context_window(q, K, V, L, 0, 1, 0.25)
    G = Hq // Hkv
    for i in range(n_q):
        p = S + i
        for h in range(Hq):
            assert np.array_equal(oc[i, h], Vf[p, h // G])
            assert abs(lc[i, h] - 0.25 * float(qf[i, h] @ Kf[p, h // G])) < 1e-12


def test_context_window_queries_have_different_windows():
    """With sink 2 and window 5, query 0 still sees position S - 4, which the last
    query's window has left; one dominant value there moves query 0 only."""
    rng = np.random.default_rng(13)
    S, n_q, Hq, Hkv, D = 40, 4, 2, 1, 8
    L = S + n_q
    q = _bf16(rng, n_q, Hq, D)
    K, V = _kv(rng, L, Hkv, D)
    base, _ = A.draft_context_window(q, K, V, L, 2, 5, 1.0)
    V2 = A.widen_bf16(V).copy()
    V2[S - 4] += 100.0
    moved, _ = A.draft_context_window(q, K, V2, L, 2, 5, 1.0)
    assert np.max(np.abs(moved[0] - base[0])) > 1e-3
    assert np.array_equal(moved[n_q - 1], base[n_q - 1])


@pytest.mark.parametrize("cuts", [[0, 100], [0, 1, 100], [0, 37, 38, 64, 100], [0, 50, 50, 100]])
def test_combine_reproduces_attention_over_union(cuts):
    rng = np.random.default_rng(len(cuts))
    q, K, V = _bf16(rng, 3, 16), _bf16(rng, 100, 16), _bf16(rng, 100, 16)
    o_ref, l_ref = A.attend(q, K, V, 0.25)
    parts = [A.attend(q, K[a:b], V[a:b], 0.25) for a, b in zip(cuts[:-1], cuts[1:])]
    po = np.stack([p[0] for p in parts])
    pl = np.stack([p[1] for p in parts])
    o, l = A.combine(po, pl)
    assert np.max(np.abs(o - o_ref)) <= 1e-13 and np.max(np.abs(l - l_ref)) <= 1e-12


def test_combine_all_empty():
    o, l = A.combine(np.zeros((3, 2, 4)), np.full((3, 2), -np.inf))
    assert np.all(o == 0) and np.all(np.isneginf(l))


def test_bf16_round_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -3.0, 1e-40], dtype=np.float32)
    r = bf16_to_f32(bf16_round(x))
    assert r[0] == 1.0
    assert r[1] == 1.0                     # tie -> even (mantissa 0)
    assert r[2] == np.float32(1.0 + 4 * 2 ** -8)  # tie -> even (rounds up)
    assert r[3] == 1.0
    assert r[4] == -3.0
    assert abs(r[5] - 1e-40) < 2 ** -133
