"""GPU parity of the fused windowed draft step (``wmtp_draft_step_window``) and of
the fused draft context pass (``wmtp_draft_context_step_window``).

One call (two launches) appends the step's new positions to the ring and attends
over the window that ends with them (the context pass: each of the last n_q
positions over its own window).  Each step is checked two ways: the output
against the float64 oracle's windowed attention over the positions appended so
far, and the ring afterwards (slot positions, count and every K/V byte) against a
second ring driven by ``wmtp_ring_append``, bit for bit.
"""

import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from oracle import ring as OR
from tests.gpu_common import compare, dev_bf16, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a GPU"
    import long_context_decode_attention_amd as lib
    lib.load()
    yield


def _lib():
    import long_context_decode_attention_amd as lib
    return lib


def _rings(B, C, Hkv, D, n_sink, n_recent, K, V, S):
    """Two identical rings (unwritten slots NaN) holding positions [0, S_b)."""
    lib = _lib()
    from long_context_decode_attention_amd import scenario as sc
    rings = []
    for _ in range(2):
        r = lib.new_ring(B, C, Hkv, D, n_sink, n_recent)
        sc.poison(r.k)
        sc.poison(r.v)
        for b in range(B):
            if S[b]:
                sc.fill_ring(r, b, K[b][:S[b]], V[b][:S[b]])
        rings.append(r)
    return rings


def _same_ring(a, b, what):
    t = torch()
    t.cuda.synchronize()
    assert t.equal(a.T, b.T), f"{what}: ring_T differs"
    assert t.equal(a.pos, b.pos), f"{what}: ring_pos differs"
    assert t.equal(a.k.view(t.int16), b.k.view(t.int16)), f"{what}: ring K bytes differ"
    assert t.equal(a.v.view(t.int16), b.v.view(t.int16)), f"{what}: ring V bytes differ"


def _run_chain(Hq, Hkv, D, C, n_sink, n_recent, S, steps, n_new=1, num_splits=0, seed=11,
               peak=1.0, n_q=0):
    """n_q = 0: the single-query step; n_q >= 1: the context pass with n_q queries."""
    lib = _lib()
    B = len(S)
    total = [s + steps * n_new for s in S]
    K = [W.kv_positions(seed, "draft_k", b, 0, total[b], Hkv, D) for b in range(B)]
    V = [W.kv_positions(seed, "draft_v", b, 0, total[b], Hkv, D) for b in range(B)]
    fused, ref = _rings(B, C, Hkv, D, n_sink, n_recent, K, V, S)
    ws = lib.new_workspace(lib.step_workspace_bytes(B, Hq, Hkv, D, C, num_splits, max(n_q, 1)))
    errs = []
    for j in range(1, steps + 1):
        lo = [s + (j - 1) * n_new for s in S]
        kn = np.stack([K[b][lo[b]:lo[b] + n_new] for b in range(B)])
        vn = np.stack([V[b][lo[b]:lo[b] + n_new] for b in range(B)])
        kt, vt = dev_bf16(kn), dev_bf16(vn)
        if n_q:
            q = W.queries(seed, "q_ctx", (B, n_q, Hq), D, step=j, peak=peak)
            o, lse = lib.draft_context_step_window(dev_bf16(q), fused, kt, vt, 1.0, workspace=ws,
                                                   num_splits=num_splits)
        else:
            q = W.queries(seed, "q_draft", (B, Hq), D, step=j, peak=peak)
            o, lse = lib.draft_step_window(dev_bf16(q), fused, kt, vt, 1.0, workspace=ws,
                                           num_splits=num_splits)
        lib.ring_append(ref, kt, vt)
        torch().cuda.synchronize()
        for b in range(B):
            L = lo[b] + n_new
            if n_q:
                ro, rl = OA.draft_context_window(q[b], K[b], V[b], L, n_sink, n_recent, 1.0)
            else:
                ro, rl = OA.draft_window(q[b], K[b], V[b], L, n_sink, n_recent, 1.0)
            errs.append(compare(o[b], lse[b], ro, rl, f"fused step b={b} step={j} L={L}"))
        _same_ring(fused, ref, f"step {j}")
        for b in range(B):
            assert fused.pos[b].cpu().tolist() == OR.expected_pos_after(lo[b] + n_new, n_sink, C)
    return errs


@pytest.mark.parametrize("Hq,Hkv,D,C,n_sink,n_recent,S,steps,num_splits", [
    (16, 2, 128, 1024, 4, 1020, [8192], 3, 0),       # the 8k workload's shapes, window 4 + 1020
    (32, 4, 128, 4096, 4, 4092, [9000], 3, 0),       # 32/4 heads, 4096-slot ring, wrapped
    (32, 2, 256, 4096, 4, 4092, [4500], 2, 0),       # 1M workload's heads and ring
    (32, 2, 256, 4096, 4, 4092, [4500], 2, 1),       # one ring split per group
    (32, 2, 256, 4096, 4, 4092, [4500], 2, 128),     # one tile per split
    (64, 2, 128, 4096, 4, 4092, [10300], 2, 0),      # 32 query rows per kv head
    (8, 1, 64, 128, 4, 100, [300], 3, 3),            # head_dim 64, slack 24
    (64, 1, 128, 4096, 4, 4092, [5000], 2, 0),       # 64 query rows per kv head: two row groups
])
def test_fused_step_chain(Hq, Hkv, D, C, n_sink, n_recent, S, steps, num_splits):
    _run_chain(Hq, Hkv, D, C, n_sink, n_recent, S, steps, num_splits=num_splits)


def test_fused_step_fresh_ring():
    """From an empty ring: the first steps fill the sink slots (their old slots are
    empty), later ones the recent slots."""
    _run_chain(16, 2, 128, 1024, 4, 1020, [0], 6)


def test_fused_step_ragged_batch():
    """Two requests at different lengths, one short of a full ring, one wrapped."""
    _run_chain(16, 2, 128, 1024, 4, 1020, [100, 5000], 3)


def test_fused_step_peaked_queries():
    """Queries x 8: O(1) outputs, far from the absolute tolerance's floor."""
    _run_chain(32, 2, 256, 4096, 4, 4092, [6000], 2, peak=8.0)


@pytest.mark.parametrize("n_new,S,C,n_sink,n_recent", [
    (3, 5000, 1024, 4, 1020),
    (32, 5000, 1024, 4, 1020),
    (32, 2, 1024, 4, 1020),        # fills the sinks and starts the recent slots in one call
    (32, 200, 64, 40, 24),         # more new positions than recent slots: some overwrite others
])
def test_fused_step_several_positions(n_new, S, C, n_sink, n_recent):
    _run_chain(16, 2, 128, C, n_sink, n_recent, [S], 2, n_new=n_new)


def test_fused_step_matches_unfused_window():
    """The fused step and append-then-window agree (different split grouping, so
    within rounding, not bitwise)."""
    lib = _lib()
    Hq, Hkv, D, C, n_sink, n_recent, S = 32, 2, 256, 4096, 4, 4092, 7000
    K = [W.kv_positions(3, "draft_k", 0, 0, S + 1, Hkv, D)]
    V = [W.kv_positions(3, "draft_v", 0, 0, S + 1, Hkv, D)]
    fused, ref = _rings(1, C, Hkv, D, n_sink, n_recent, K, V, [S])
    q = dev_bf16(W.queries(3, "q_draft", (1, Hq), D, step=1))
    kt, vt = dev_bf16(K[0][S:S + 1][None]), dev_bf16(V[0][S:S + 1][None])
    o1, l1 = lib.draft_step_window(q, fused, kt, vt, 1.0)
    lib.ring_append(ref, kt, vt)
    o2, l2 = lib.draft_attn_window(q, ref, 1.0)
    torch().cuda.synchronize()
    assert float((o1 - o2).abs().max()) <= 1e-5
    assert float((l1 - l2).abs().max()) <= 1e-5
    _same_ring(fused, ref, "single step")


def test_fused_step_errors():
    """Host checks: nothing is launched and the ring is untouched."""
    lib = _lib()
    t = torch()
    Hq, Hkv, D, C = 16, 2, 128, 1024
    ring = lib.new_ring(1, C, Hkv, D, 4, 1020)
    q = t.zeros(1, Hq, D, dtype=t.bfloat16, device="cuda")
    k33 = t.zeros(1, 33, Hkv, D, dtype=t.bfloat16, device="cuda")
    with pytest.raises(lib.WmtpError) as e:
        lib.draft_step_window(q, ring, k33, k33)
    assert e.value.status == 1                     # more than 32 new positions
    k1 = t.zeros(1, 1, Hkv, D, dtype=t.bfloat16, device="cuda")
    small = lib.new_workspace(64)
    with pytest.raises(lib.WmtpError) as e:
        lib.draft_step_window(q, ring, k1, k1, workspace=small)
    assert e.value.status == 3                     # workspace too small
    ring_wide = lib.new_ring(1, C, 1, D, 4, 1020)
    q512 = t.zeros(1, 512, D, dtype=t.bfloat16, device="cuda")
    k1w = t.zeros(1, 1, 1, D, dtype=t.bfloat16, device="cuda")
    with pytest.raises(lib.WmtpError) as e:
        lib.draft_step_window(q512, ring_wide, k1w, k1w, workspace=lib.new_workspace(1 << 20))
    assert e.value.status == 2                     # 512 query rows per kv head
    qc = t.zeros(1, 2, Hq, D, dtype=t.bfloat16, device="cuda")
    with pytest.raises(lib.WmtpError) as e:        # window 4 + 1020 fills the ring: no slack
        lib.draft_context_step_window(qc, ring, k1, k1, workspace=lib.new_workspace(1 << 24))
    assert e.value.status == 1
    with pytest.raises(lib.WmtpError) as e:
        lib.draft_step_window(q, ring, k1, k1, softmax_scale=-1.0)
    assert e.value.status == 1                     # the scale must be positive
    t.cuda.synchronize()
    assert int(ring.T[0]) == 0 and int((ring.pos >= 0).sum()) == 0


def _random_cases(n, seed=2027):
    """Seeded random shapes for the fused step: ring capacity, sink and window sizes
    (including windows smaller than the ring, slack, tiny rings), head dims, batch,
    context lengths around the wrap points, new positions per call and split counts."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        C = int(rng.choice([64, 128, 192, 1024]))
        n_sink = int(rng.integers(0, min(16, C - 1) + 1))
        n_recent = int(rng.integers(1, C - n_sink + 1))
        D = int(rng.choice([64, 128, 256]))
        Hkv = int(rng.choice([1, 2]))
        G = int(rng.choice([1, 4, 8, 16, 32]))
        B = int(rng.integers(1, 4))
        S = [int(rng.choice([0, 1, n_sink, C - 1, C, C + 1, 3 * C + 5, int(rng.integers(0, 4 * C))]))
             for _ in range(B)]
        n_new = int(rng.choice([1, 2, 7, 32]))
        num_splits = int(rng.choice([0, 1, 2, 5]))
        cases.append((Hkv * G, Hkv, D, C, n_sink, n_recent, S, n_new, num_splits))
    return cases


@pytest.mark.parametrize("case", _random_cases(24), ids=lambda c: "H{}x{}_D{}_C{}_s{}_r{}_B{}_n{}_p{}".format(
    c[0], c[1], c[2], c[3], c[4], c[5], len(c[6]), c[7], c[8]))
def test_fused_step_random_shapes(case):
    """Seeded random shapes, two steps each: oracle parity and ring state equal to
    append-then-window's, bit for bit."""
    Hq, Hkv, D, C, n_sink, n_recent, S, n_new, num_splits = case
    _run_chain(Hq, Hkv, D, C, n_sink, n_recent, S, 2, n_new=n_new, num_splits=num_splits,
               seed=31)


# The fused draft context pass: n_q queries (the accepted positions after a verify)
# over rings with slack >= n_q - 1.
@pytest.mark.parametrize("Hq,Hkv,D,C,n_sink,n_recent,S,n_new,n_q", [
    (32, 2, 256, 4160, 4, 4092, [9000], 8, 8),      # the 1M workload's heads, 8 queries, 128 rows
    (32, 2, 256, 4160, 4, 4092, [0], 8, 8),         # fresh ring
    (16, 2, 128, 1088, 4, 1020, [3000, 50], 4, 4),  # ragged batch, one request short of a ring
    (64, 2, 128, 4160, 4, 4092, [10300], 4, 4),     # 32 rows per kv head and query
    (8, 1, 64, 128, 4, 100, [300], 2, 5),           # more queries than new positions
    (8, 1, 64, 64, 40, 16, [200], 32, 9),           # new positions overwrite each other
    (4, 4, 128, 1024, 0, 1000, [2500], 1, 1),       # one query, no sink
])
def test_fused_context_step_chain(Hq, Hkv, D, C, n_sink, n_recent, S, n_new, n_q):
    _run_chain(Hq, Hkv, D, C, n_sink, n_recent, S, 3, n_new=n_new, n_q=n_q, seed=17)


def test_fused_context_step_matches_unfused():
    """Fused context pass against append then ``draft_context_window``: within
    rounding (different split grouping), ring state bit for bit."""
    lib = _lib()
    Hq, Hkv, D, C, n_sink, n_recent, S, n = 32, 2, 256, 4160, 4, 4092, 7000, 8
    K = [W.kv_positions(5, "draft_k", 0, 0, S + n, Hkv, D)]
    V = [W.kv_positions(5, "draft_v", 0, 0, S + n, Hkv, D)]
    fused, ref = _rings(1, C, Hkv, D, n_sink, n_recent, K, V, [S])
    q = dev_bf16(W.queries(5, "q_ctx", (1, n, Hq), D, step=1))
    kt, vt = dev_bf16(K[0][S:S + n][None]), dev_bf16(V[0][S:S + n][None])
    o1, l1 = lib.draft_context_step_window(q, fused, kt, vt, 1.0)
    lib.ring_append(ref, kt, vt)
    o2, l2 = lib.draft_context_window(q, ref, 1.0)
    torch().cuda.synchronize()
    assert float((o1 - o2).abs().max()) <= 1e-5
    assert float((l1 - l2).abs().max()) <= 1e-5
    _same_ring(fused, ref, "context pass")


def _random_context_cases(n, seed=2029):
    """Seeded random shapes for the fused context pass: slack drawn first so that
    n_q - 1 fits it, then the rest as for the single-query step."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        C = int(rng.choice([64, 128, 192, 1088]))
        n_sink = int(rng.integers(0, min(16, C - 2) + 1))
        slack = int(rng.integers(0, min(40, C - n_sink - 1) + 1))
        n_recent = C - n_sink - slack
        n_q = int(rng.integers(1, slack + 2))
        D = int(rng.choice([64, 128, 256]))
        Hkv = int(rng.choice([1, 2]))
        G = int(rng.choice([1, 4, 8, 16]))
        while n_q * G > 256:
            G //= 2
        B = int(rng.integers(1, 4))
        n_new = int(rng.choice([1, 2, 7, 32]))
        S = [max(int(rng.choice([0, 1, n_sink, C - 1, C, 3 * C + 5, int(rng.integers(0, 4 * C))])),
                 n_q) for _ in range(B)]
        num_splits = int(rng.choice([0, 1, 2, 5]))
        cases.append((Hkv * G, Hkv, D, C, n_sink, n_recent, S, n_new, n_q, num_splits))
    return cases


@pytest.mark.parametrize("case", _random_context_cases(16),
                         ids=lambda c: "H{}x{}_D{}_C{}_s{}_r{}_B{}_n{}_q{}_p{}".format(
                             c[0], c[1], c[2], c[3], c[4], c[5], len(c[6]), c[7], c[8], c[9]))
def test_fused_context_step_random_shapes(case):
    Hq, Hkv, D, C, n_sink, n_recent, S, n_new, n_q, num_splits = case
    _run_chain(Hq, Hkv, D, C, n_sink, n_recent, S, 2, n_new=n_new, num_splits=num_splits,
               seed=37, n_q=n_q)


@pytest.mark.parametrize("n_q,n_new,rolled", [
    (0, 1, 3),     # single-query step after rolling back 3 speculative positions
    (0, 2, 3),     # two new positions; one stale slot stays past the window's end
    (4, 3, 3),     # context pass over the re-appended positions
    (8, 8, 8),     # context pass re-appending every rolled-back position
])
def test_fused_steps_after_rollback(n_q, n_new, rolled):
    """A rollback (a smaller ring_T) leaves slots holding positions >= ring_T with
    the rejected drafts' K/V.  The fused step re-appends those positions with new
    values: its result must count each position once, with the new values (the
    oracle over the accepted prefix plus the new positions), and the ring afterwards
    must equal the one that append-then-window leaves."""
    lib = _lib()
    Hq, Hkv, D, C, n_sink, n_recent, T = 16, 2, 128, 1024, 4, 960, 5000
    K_old = W.kv_positions(60, "draft_k", 0, 0, T + rolled, Hkv, D)
    V_old = W.kv_positions(60, "draft_v", 0, 0, T + rolled, Hkv, D)
    K_new = W.kv_positions(61, "draft_k", 0, T, T + n_new, Hkv, D)
    V_new = W.kv_positions(61, "draft_v", 0, T, T + n_new, Hkv, D)
    fused, ref = _rings(1, C, Hkv, D, n_sink, n_recent, [K_old], [V_old], [T + rolled])
    fused.T.fill_(T)
    ref.T.fill_(T)
    K = np.concatenate([K_old[:T], K_new])
    V = np.concatenate([V_old[:T], V_new])
    kt, vt = dev_bf16(K_new[None]), dev_bf16(V_new[None])
    L = T + n_new
    if n_q:
        q = W.queries(62, "q_ctx", (1, n_q, Hq), D)
        ws = lib.new_workspace(lib.step_workspace_bytes(1, Hq, Hkv, D, C, 0, n_q))
        o, lse = lib.draft_context_step_window(dev_bf16(q), fused, kt, vt, 1.0, workspace=ws)
        ro, rl = OA.draft_context_window(q[0], K, V, L, n_sink, n_recent, 1.0)
    else:
        q = W.queries(62, "q_draft", (1, Hq), D)
        o, lse = lib.draft_step_window(dev_bf16(q), fused, kt, vt, 1.0)
        ro, rl = OA.draft_window(q[0], K, V, L, n_sink, n_recent, 1.0)
    lib.ring_append(ref, kt, vt)
    torch().cuda.synchronize()
    compare(o[0], lse[0], ro, rl, f"fused step after rollback of {rolled}")
    _same_ring(fused, ref, "after rollback")
