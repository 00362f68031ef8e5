"""GPU parity: every C-ABI call against the float64 oracle on the same seeded inputs.

Sizes are chosen so that the oracle finishes in seconds while the kernels still
run many tiles, several splits and a ragged tail; the full 1M-context sizes are
covered by sampled outputs in ``test_gpu_fullsize.py``.
"""

import math

import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from oracle import ring as OR
from tests.gpu_common import DraftScenario, VerifyScenario, compare, dev_bf16, dev_i32, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a GPU"
    import long_context_decode_attention_amd as lib
    lib.load()
    yield


CFG = W.CONFIGS


def _lib():
    import long_context_decode_attention_amd as lib
    return lib


def _draft_chain(sc: DraftScenario, num_splits=0, check_window=True):
    lib = _lib()
    cfg = sc.cfg
    res = []
    for j in range(1, sc.gamma + 1):
        sc.append(j)
        q = sc.q(j)
        qt = dev_bf16(q)
        lens = sc.lens(j)
        o_f, l_f = lib.draft_attn_full(qt, sc.kv.k, sc.kv.v, sc.kv.block_table, dev_i32(lens),
                                       max(lens), 1.0, num_splits=num_splits)
        o_w, l_w = lib.draft_attn_window(qt, sc.ring, 1.0, num_splits=num_splits)
        o_p, l_p = lib.draft_attn_window_paged(qt, sc.kv.k, sc.kv.v, sc.kv.block_table,
                                               dev_i32(lens), max(lens), cfg["n_sink"],
                                               cfg["n_recent"], 1.0, num_splits=num_splits)
        torch().cuda.synchronize()
        for b in range(sc.B):
            of, lf = OA.draft_full(q[b], sc.K[b], sc.V[b], lens[b], 1.0)
            compare(o_f[b], l_f[b], of, lf, f"full b={b} step={j} L={lens[b]}")
            ow, lw = OA.draft_window(q[b], sc.K[b], sc.V[b], lens[b], cfg["n_sink"],
                                     cfg["n_recent"], 1.0)
            # the truncated paged index reads the window's keys from the paged cache
            compare(o_p[b], l_p[b], ow, lw, f"paged window b={b} step={j} L={lens[b]}")
            if check_window:
                compare(o_w[b], l_w[b], ow, lw, f"window b={b} step={j} L={lens[b]}")
        res.append((o_f, l_f, o_w, l_w))
    return res


# ------------------------------------------------------------------ draft: full and windowed

def test_draft_ctx8k_full_size():
    """Single decode query, 16/2 heads, D 128, context 8192, window 4 + 1020, one step."""
    cfg = CFG["ctx8k_g16x2_d128"]
    _draft_chain(DraftScenario(cfg, 1, [cfg["S"]], cfg["gamma"]))


def test_draft_ctx128k_shape_three_steps():
    """32/4 heads, D 128, window 4 + 4092, 3 chained steps; context cut to a ragged 20011."""
    cfg = CFG["ctx128k_g32x4_d128"]
    _draft_chain(DraftScenario(cfg, 2, [20011], 3))


def test_draft_ctx1m_shape_permuted_pages():
    """32/2 heads, D 256, permuted 64-token pages, 2 steps; context cut to 40000."""
    cfg = CFG["ctx1m_g32x2_d256"]
    _draft_chain(DraftScenario(cfg, 3, [40000], 2))


def test_draft_ragged_batch():
    """Batch 8 with ragged contexts in a shared permuted pool, 32/4 heads, D 128."""
    cfg = CFG["ragged8_256k_1m_g32x4_d128"]
    S = [int(x) for x in W.ragged_lengths(4, 8, 3000, 9000)]
    _draft_chain(DraftScenario(cfg, 4, S, 2))


def test_draft_ragged_long_four_rounds():
    """Several sequences, the longest past 64K keys: the plan runs four workgroups
    per CU (lengths on the device), splits of short sequences end up empty."""
    lib = _lib()
    cfg = CFG["ragged8_256k_1m_g32x4_d128"]
    S = [66000, 140000, 9000]
    # more than two rounds of one workgroup per CU (256 CUs)
    assert lib.plan_splits(3, cfg["Hq"], cfg["Hkv"], cfg["D"], 1, max(S) + 1) * 3 * cfg["Hkv"] > 512
    _draft_chain(DraftScenario(cfg, 6, S, 1))


def test_draft_g64x2_wrapped_ring():
    """64/2 heads (G = 32, two row blocks), D 128; ring of 4096 wrapped (T > C)."""
    cfg = CFG["nope8l_1m_g64x2_d128"]
    _draft_chain(DraftScenario(cfg, 5, [11000], 2))


@pytest.mark.parametrize("S", [0, 1, 3, 63, 64, 65, 1023, 1024, 1025])
def test_draft_short_contexts(S):
    """Contexts shorter than, equal to and just past the window and the tile sizes."""
    cfg = dict(CFG["ctx8k_g16x2_d128"])
    _draft_chain(DraftScenario(cfg, 10 + S, [S], 2))


def test_draft_peaked_and_scaled():
    """Sharper attention (q x 8) and an explicit 1/sqrt(D) softmax scale."""
    cfg = CFG["ctx1m_g32x2_d256"]
    sc = DraftScenario(cfg, 6, [9000], 1, peak=8.0)
    lib = _lib()
    sc.append(1)
    q = sc.q(1)
    lens = sc.lens(1)
    s = 1.0 / math.sqrt(cfg["D"]) * 4.0
    o, l = lib.draft_attn_full(dev_bf16(q), sc.kv.k, sc.kv.v, sc.kv.block_table, dev_i32(lens),
                               lens[0], s)
    ow, lw = lib.draft_attn_window(dev_bf16(q), sc.ring, s)
    torch().cuda.synchronize()
    of, lf = OA.draft_full(q[0], sc.K[0], sc.V[0], lens[0], s)
    compare(o[0], l[0], of, lf, "peaked full")
    ow_ref, lw_ref = OA.draft_window(q[0], sc.K[0], sc.V[0], lens[0], 4, 4092, s)
    compare(ow[0], lw[0], ow_ref, lw_ref, "peaked window")


@pytest.mark.parametrize("num_splits", [1, 3, 64])
def test_paged_window_split_counts(num_splits):
    """Truncated paged index with the sink tile and the recent tiles in one split,
    in a few, and one tile per split; window 4 + 4092 over a 40000-key context."""
    lib = _lib()
    cfg = CFG["ctx1m_g32x2_d256"]
    sc = DraftScenario(cfg, 12, [40000], 1)
    sc.append(1)
    q = sc.q(1)
    lens = sc.lens(1)
    o, l = lib.draft_attn_window_paged(dev_bf16(q), sc.kv.k, sc.kv.v, sc.kv.block_table,
                                       dev_i32(lens), lens[0], cfg["n_sink"], cfg["n_recent"],
                                       1.0, num_splits=num_splits)
    torch().cuda.synchronize()
    ow, lw = OA.draft_window(q[0], sc.K[0], sc.V[0], lens[0], cfg["n_sink"], cfg["n_recent"], 1.0)
    compare(o[0], l[0], ow, lw, f"paged window num_splits={num_splits}")


@pytest.mark.parametrize("cfg_name,C,n_sink,n_recent,L,n_q", [
    ("ctx1m_g32x2_d256", 4160, 4, 4092, 6000, 8),      # 128 query rows, ring wrapped
    ("ctx128k_g32x4_d128", 4160, 4, 4092, 3000, 4),    # ring not yet full
    ("nope8l_1m_g64x2_d128", 128, 4, 60, 1000, 8),     # 256 rows; small window, many wraps
])
def test_draft_context_pass_over_the_ring(cfg_name, C, n_sink, n_recent, L, n_q):
    """Draft context pass: n_q causal queries, each over the window of its own
    position, read from a ring whose slack (C - n_sink - n_recent >= n_q - 1)
    still holds the earliest query's window."""
    lib = _lib()
    from long_context_decode_attention_amd import scenario as scn
    cfg = CFG[cfg_name]
    Hq, Hkv, D = cfg["Hq"], cfg["Hkv"], cfg["D"]
    seed = 70 + n_q
    K = W.kv_positions(seed, "draft_k", 0, 0, L, Hkv, D)
    V = W.kv_positions(seed, "draft_v", 0, 0, L, Hkv, D)
    ring = lib.new_ring(1, C, Hkv, D, n_sink, n_recent)
    scn.poison(ring.k)
    scn.poison(ring.v)
    scn.fill_ring(ring, 0, K, V)
    q = W.queries(seed, "q_ctx", (1, n_q, Hq), D)
    o, l = lib.draft_context_window(dev_bf16(q), ring, 1.0)
    torch().cuda.synchronize()
    ro, rl = OA.draft_context_window(q[0], K, V, L, n_sink, n_recent, 1.0)
    compare(o[0], l[0], ro, rl, f"context pass {cfg_name} n_q={n_q}")
    # one query is a draft step: the same as the windowed draft call
    o1, l1 = lib.draft_context_window(dev_bf16(q[:, -1:]), ring, 1.0)
    ow, lw = lib.draft_attn_window(dev_bf16(q[:, -1]), ring, 1.0)
    torch().cuda.synchronize()
    assert torch().equal(o1[:, 0], ow) and torch().equal(l1[:, 0], lw)


def test_draft_context_pass_needs_slack():
    """Without slack for the earlier queries' windows the call is refused."""
    lib = _lib()
    cfg = CFG["ctx1m_g32x2_d256"]
    ring = lib.new_ring(1, 4096, cfg["Hkv"], cfg["D"], 4, 4092)
    q = dev_bf16(W.queries(3, "q_ctx", (1, 2, cfg["Hq"]), cfg["D"]))
    with pytest.raises(lib.WmtpError):
        lib.draft_context_window(q, ring, 1.0)


def test_window_equals_full_when_window_covers_context():
    cfg = CFG["ctx128k_g32x4_d128"]
    sc = DraftScenario(cfg, 7, [3000], 1)
    lib = _lib()
    sc.append(1)
    q = dev_bf16(sc.q(1))
    lens = sc.lens(1)
    o_f, l_f = lib.draft_attn_full(q, sc.kv.k, sc.kv.v, sc.kv.block_table, dev_i32(lens), lens[0])
    o_w, l_w = lib.draft_attn_window(q, sc.ring)
    torch().cuda.synchronize()
    assert float((o_f - o_w).abs().max()) <= 1e-5
    assert float((l_f - l_w).abs().max()) <= 1e-5


def test_needle_outside_window_moves_full_only():
    """A planted high-logit key just outside the recent window changes the native
    draft's output but not the windowed one."""
    lib = _lib()
    cfg = dict(CFG["ctx8k_g16x2_d128"])
    S = 5000
    sc = DraftScenario(cfg, 8, [S], 1)
    q = sc.q(1)
    L = S + 1
    needle = L - cfg["n_recent"] - 1
    qf = W.bf16_to_f32(q[0])
    K2 = sc.K[0].copy()
    for g in range(cfg["Hkv"]):
        K2[needle, g] = W.bf16_round(4.0 * np.sign(qf[g * 8]) * np.ones(cfg["D"], np.float32))
    sc2 = DraftScenario(cfg, 8, [S], 1)
    sc2.K[0] = K2
    from long_context_decode_attention_amd import scenario as scn
    scn.fill_paged(sc2.kv, 0, needle, K2[needle:needle + 1], sc2.V[0][needle:needle + 1])
    sc.append(1)
    sc2.append(1)
    qt = dev_bf16(q)
    a = lib.draft_attn_full(qt, sc.kv.k, sc.kv.v, sc.kv.block_table, dev_i32([L]), L)
    b = lib.draft_attn_full(qt, sc2.kv.k, sc2.kv.v, sc2.kv.block_table, dev_i32([L]), L)
    wa = lib.draft_attn_window(qt, sc.ring)
    wb = lib.draft_attn_window(qt, sc2.ring)
    torch().cuda.synchronize()
    of, lf = OA.draft_full(q[0], K2, sc2.V[0], L, 1.0)
    compare(b[0][0], b[1][0], of, lf, "needle full")
    assert float((a[0] - b[0]).abs().max()) > 0.05
    assert torch().equal(wa[0], wb[0])


@pytest.mark.parametrize("call", ["full", "window", "verify"])
def test_logit_jump_takes_the_rescale_path(call):
    """Two keys whose logits sit about 1000 above every other key's, placed after
    many ordinary tiles: the running maximum must be raised far beyond the
    kernels' lazy margin, which sends the tile to the general (rescaling) loop;
    the second key, a few units below the first and later in the sequence, checks
    that tiles after the rescale are still accumulated with the right weight."""
    lib = _lib()
    cfg = CFG["ctx1m_g32x2_d256"]
    D, Hkv, Hq = cfg["D"], cfg["Hkv"], cfg["Hq"]
    G = Hq // Hkv
    rng = np.random.default_rng(1234)
    u = np.sign(rng.standard_normal((Hkv, D))).astype(np.float32)
    S = 3000
    # q.k about 4 D = 1024 and 4 below it; with one split both spikes fall in the
    # same wave's tiles (59 and 79), the second after the rescale
    spikes = ((1900, 4.0), (2540, 3.99))
    if call == "verify":
        n_q = 8
        sc = VerifyScenario(cfg, 41, [S], n_q)
        qf = 0.25 * W.bf16_to_f32(sc.q) + np.repeat(u, G, axis=0)[None, None]
        q = W.bf16_round(qf)
        from long_context_decode_attention_amd import scenario as scn
        for p_, c in spikes:
            sc.K[0][p_] = W.bf16_round(c * u)
            scn.fill_paged(sc.kv, 0, p_, sc.K[0][p_:p_ + 1], sc.V[0][p_:p_ + 1])
        sc.append_proposed()
        L = S + n_q
        o, l = lib.verify_attn(dev_bf16(q), sc.kv.k, sc.kv.v, sc.kv.block_table, dev_i32([L]), L,
                               num_splits=1)
        torch().cuda.synchronize()
        ro, rl = OA.verify(q[0], sc.K[0], sc.V[0], L, 1.0)
        compare(o[0], l[0], ro, rl, "verify logit jump")
        return
    sc = DraftScenario(cfg, 42, [S], 1)
    qf = 0.25 * W.bf16_to_f32(sc.q(1)) + np.repeat(u, G, axis=0)[None]
    q = W.bf16_round(qf)
    from long_context_decode_attention_amd import scenario as scn
    for p_, c in spikes:
        sc.K[0][p_] = W.bf16_round(c * u)
        scn.fill_paged(sc.kv, 0, p_, sc.K[0][p_:p_ + 1], sc.V[0][p_:p_ + 1])
    sc.ring = lib.new_ring(1, cfg["C"], Hkv, D, cfg["n_sink"], cfg["n_recent"])
    scn.fill_ring(sc.ring, 0, sc.K[0][:S], sc.V[0][:S])
    sc.append(1)
    L = S + 1
    if call == "full":
        o, l = lib.draft_attn_full(dev_bf16(q), sc.kv.k, sc.kv.v, sc.kv.block_table, dev_i32([L]), L,
                                   num_splits=1)
        ro, rl = OA.draft_full(q[0], sc.K[0], sc.V[0], L, 1.0)
    else:
        o, l = lib.draft_attn_window(dev_bf16(q), sc.ring, num_splits=1)
        ro, rl = OA.draft_window(q[0], sc.K[0], sc.V[0], L, cfg["n_sink"], cfg["n_recent"], 1.0)
    torch().cuda.synchronize()
    compare(o[0], l[0], ro, rl, f"{call} logit jump")


# ------------------------------------------------------------------ split structure

@pytest.mark.parametrize("num_splits", [1, 2, 7, 64])
def test_split_count_invariance(num_splits):
    lib = _lib()
    cfg = CFG["ctx1m_g32x2_d256"]
    sc = DraftScenario(cfg, 9, [30000], 1)
    sc.append(1)
    q = sc.q(1)
    lens = sc.lens(1)
    o, l = lib.draft_attn_full(dev_bf16(q), sc.kv.k, sc.kv.v, sc.kv.block_table, dev_i32(lens),
                               lens[0], num_splits=num_splits)
    torch().cuda.synchronize()
    of, lf = OA.draft_full(q[0], sc.K[0], sc.V[0], lens[0], 1.0)
    compare(o[0], l[0], of, lf, f"num_splits={num_splits}")


def test_deterministic_bitwise():
    lib = _lib()
    cfg = CFG["ctx1m_g32x2_d256"]
    sc = DraftScenario(cfg, 11, [25000], 1)
    sc.append(1)
    q = dev_bf16(sc.q(1))
    lens = dev_i32(sc.lens(1))
    r1 = lib.draft_attn_full(q, sc.kv.k, sc.kv.v, sc.kv.block_table, lens, 25001)
    r2 = lib.draft_attn_full(q, sc.kv.k, sc.kv.v, sc.kv.block_table, lens, 25001)
    w1 = lib.draft_attn_window(q, sc.ring)
    w2 = lib.draft_attn_window(q, sc.ring)
    torch().cuda.synchronize()
    assert torch().equal(r1[0], r2[0]) and torch().equal(r1[1], r2[1])
    assert torch().equal(w1[0], w2[0]) and torch().equal(w1[1], w2[1])


def test_partials_only_then_combine_equals_direct():
    lib = _lib()
    cfg = CFG["ctx128k_g32x4_d128"]
    sc = DraftScenario(cfg, 12, [20000], 1)
    sc.append(1)
    q = dev_bf16(sc.q(1))
    lens = dev_i32(sc.lens(1))
    B, Hq, Hkv, D = 1, cfg["Hq"], cfg["Hkv"], cfg["D"]
    o, l = lib.draft_attn_full(q, sc.kv.k, sc.kv.v, sc.kv.block_table, lens, 20001)
    ws = lib.draft_attn_full(q, sc.kv.k, sc.kv.v, sc.kv.block_table, lens, 20001,
                             partials_only=True)
    po, pl = lib.partials_view(ws, B, Hq, Hkv, D, 1, 20001)
    splits = lib.plan_splits(B, Hq, Hkv, D, 1, 20001)
    assert splits > 1
    o2, l2 = lib.split_combine(po, pl, B, Hkv, Hq // Hkv, 1, splits_per_group=splits)
    torch().cuda.synchronize()
    assert torch().equal(o.view(-1), o2.view(-1)) and torch().equal(l.view(-1), l2.view(-1))


@pytest.mark.parametrize("D,G,n_q,csr", [
    (128, 4, 2, True),      # 8 rows: the few-row merge
    (96, 4, 2, True),       # head dims that are not powers of two: every column written
    (192, 8, 1, True),
    (48, 2, 1, False),
    (80, 16, 1, False),
    (240, 4, 4, False),
    (16, 1, 1, True),
    (96, 16, 4, True),      # 64 rows: the many-row merge
    (192, 32, 4, False),
])
def test_split_combine_against_oracle_csr(D, G, n_q, csr):
    """Direct test of the combine with empty splits and an empty group, at head dims
    that are multiples of 16 up to 256, through a CSR split list or a fixed count."""
    lib = _lib()
    rng = np.random.default_rng(13)
    B, Hkv = 2, 3
    R = G * n_q
    counts = [3, 0, 5, 1, 7, 2] if csr else [4] * (B * Hkv)   # group 1 has no split (CSR)
    indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    P = int(indptr[-1])
    po = rng.standard_normal((P, R, D)).astype(np.float32)
    pl = (rng.standard_normal((P, R)) * 3).astype(np.float32)
    pl[1, :] = -np.inf                               # an empty split
    o = torch().full((B, n_q, Hkv * G, D), float("nan"), device="cuda")   # unwritten shows
    o, l = lib.split_combine(torch().tensor(po, device="cuda"), torch().tensor(pl, device="cuda"),
                             B, Hkv, G, n_q, split_indptr=dev_i32(indptr) if csr else None,
                             splits_per_group=0 if csr else 4, o=o)
    torch().cuda.synchronize()
    o = o.cpu().numpy()
    l = l.cpu().numpy()
    for grp in range(B * Hkv):
        b, g = divmod(grp, Hkv)
        a, e = indptr[grp], indptr[grp + 1]
        if a == e:
            ro, rl = np.zeros((R, D)), np.full(R, -np.inf)
        else:
            ro, rl = OA.combine(po[a:e], pl[a:e])
        for r in range(R):
            i, hl = divmod(r, G)
            h = g * G + hl
            got_o, got_l = o[b, i, h], l[b, i, h]
            if np.isneginf(rl[r]):
                assert np.isneginf(got_l) and np.all(got_o == 0)
            else:
                assert np.max(np.abs(got_o - ro[r])) <= 1e-5 * (1 + np.max(np.abs(ro[r])))
                assert abs(got_l - rl[r]) <= 1e-5


# ------------------------------------------------------------------ verify

def _verify_case(cfg, seed, S, n_q, num_splits=0):
    lib = _lib()
    vs = VerifyScenario(cfg, seed, S, n_q)
    vs.append_proposed()
    lens = vs.lens()
    o, l = lib.verify_attn(dev_bf16(vs.q), vs.kv.k, vs.kv.v, vs.kv.block_table, dev_i32(lens),
                           max(lens), 1.0, num_splits=num_splits)
    torch().cuda.synchronize()
    for b in range(vs.B):
        ro, rl = OA.verify(vs.q[b], vs.K[b], vs.V[b], lens[b], 1.0)
        compare(o[b], l[b], ro, rl, f"verify b={b} L={lens[b]}")
    return vs, o, l


def test_verify_ctx1m_shape():
    """8 causal queries, 32/2 heads, D 256 (128 query rows per kv head); context 20000."""
    _verify_case(CFG["ctx1m_g32x2_d256"], 21, [20000], 8)


def test_verify_ragged_batch():
    cfg = CFG["ragged8_256k_1m_g32x4_d128"]
    S = [int(x) for x in W.ragged_lengths(22, 8, 2000, 7000)]
    _verify_case(cfg, 22, S, 4)


@pytest.mark.parametrize("cfg_name,S,n_q", [
    ("ragged8_256k_1m_g32x4_d128", [70000, 30000], 4),    # 32 rows: split kernel
    ("ctx128k_g32x4_d128", [66000, 20000], 8),            # 64 rows: shared kernel, two row blocks
])
def test_verify_ragged_long_four_rounds(cfg_name, S, n_q):
    """Verify over several sequences, the longest past 64K keys (four workgroup rounds)."""
    _verify_case(CFG[cfg_name], 24, S, n_q)


def test_verify_g64x2_256_rows():
    """G = 32 and 8 queries: 256 query rows per kv head."""
    _verify_case(CFG["nope8l_1m_g64x2_d128"], 23, [6000], 8)


@pytest.mark.parametrize("S", [0, 1, 60, 64, 100])
def test_verify_short(S):
    _verify_case(CFG["ctx1m_g32x2_d256"], 30 + S, [S], 8)


G64D64 = dict(Hq=64, Hkv=2, D=64)   # head dim 64, 256 rows: two row blocks per wave


@pytest.mark.parametrize("cfg_name,S,n_q,num_splits,peak", [
    ("ctx1m_g32x2_d256", 20000, 8, 2, 1.0),
    ("ctx1m_g32x2_d256", 16000, 8, 1, 4.0),
    ("nope8l_1m_g64x2_d128", 12000, 8, 1, 1.0),
    ("ctx128k_g32x4_d128", 15000, 8, 2, 2.0),
    (G64D64, 12000, 8, 1, 1.0),
    (G64D64, 9000, 8, 2, 3.0),
])
def test_verify_long_splits(cfg_name, S, n_q, num_splits, peak):
    """Splits of hundreds of 32-key tiles, so that most tiles take the verify's
    fast path, whose PV sees the weights rounded to bf16 (the normaliser then
    uses the same rounded weights); plain and peaked queries (q x peak).  The
    shapes cover every way the fast tiles sum their hi weight parts: products
    with a V^T of ones (head dim 256; head dim 64 with two row blocks per wave)
    and bf16 dot products (head dim 128 with eight waves)."""
    lib = _lib()
    cfg = CFG[cfg_name] if isinstance(cfg_name, str) else cfg_name
    vs = VerifyScenario(cfg, 60 + S % 97, [S], n_q)
    vs.append_proposed()
    q = W.bf16_round(peak * W.bf16_to_f32(vs.q))
    L = S + n_q
    o, l = lib.verify_attn(dev_bf16(q), vs.kv.k, vs.kv.v, vs.kv.block_table, dev_i32([L]), L,
                           1.0, num_splits=num_splits)
    torch().cuda.synchronize()
    ro, rl = OA.verify(q[0], vs.K[0], vs.V[0], L, 1.0)
    err, lerr = compare(o[0], l[0], ro, rl, f"verify long splits {cfg_name} peak {peak}")
    print(f"verify long splits {cfg_name} S={S} splits={num_splits} peak={peak}: "
          f"max|o err| {err:.2e} (max|o| {float(np.max(np.abs(ro))):.2e}), max|lse err| {lerr:.2e}")


def _verify_custom(cfg_name, seed, S, n_q, K, V, q, num_splits):
    """Verify over caller-built K/V bits (positions 0 .. S + n_q - 1) against the oracle."""
    lib = _lib()
    from long_context_decode_attention_amd import scenario as scn
    cfg = CFG[cfg_name] if isinstance(cfg_name, str) else cfg_name
    L = S + n_q
    kv = scn.alloc_paged_kv([L], cfg["Hkv"], cfg["D"], W.page_permutation(seed, "target_k", (L + 63) // 64))
    scn.poison(kv.k)
    scn.poison(kv.v)
    scn.fill_paged(kv, 0, 0, K, V)
    o, l = lib.verify_attn(dev_bf16(q), kv.k, kv.v, kv.block_table, dev_i32([L]), L, 1.0,
                           num_splits=num_splits)
    torch().cuda.synchronize()
    ro, rl = OA.verify(q[0], K, V, L, 1.0)
    return o[0], l[0], ro, rl


@pytest.mark.parametrize("cfg_name,S,num_splits", [
    ("ctx1m_g32x2_d256", 24000, 1),          # 128 rows per kv head, one split of 750 tiles
    ("nope8l_1m_g64x2_d128", 16000, 1),      # 256 rows per kv head
])
def test_verify_long_split_wide_values(cfg_name, S, num_splits):
    """V x 16 (exact in bf16: an exponent shift): outputs ~16x larger, so the fast
    tiles' bf16-rounded weights are checked against the relative bound (error at
    most 1e-2 of the largest output), not only the absolute one."""
    cfg = CFG[cfg_name]
    n_q, Hkv, D = 8, cfg["Hkv"], cfg["D"]
    K = W.kv_positions(91, "target_k", 0, 0, S + n_q, Hkv, D)
    V = W.bf16_round(16.0 * W.bf16_to_f32(W.kv_positions(91, "target_v", 0, 0, S + n_q, Hkv, D)))
    q = W.queries(91, "q_verify", (1, n_q, cfg["Hq"]), D)
    o, l, ro, rl = _verify_custom(cfg_name, 91, S, n_q, K, V, q, num_splits)
    got = o.double().cpu().numpy().reshape(ro.shape)
    err = float(np.max(np.abs(got - ro)))
    scale = float(np.max(np.abs(ro)))
    lerr = float(np.max(np.abs(l.double().cpu().numpy().reshape(rl.shape) - rl)))
    print(f"verify wide values {cfg_name}: max|o err| {err:.2e}, max|o| {scale:.2e}, "
          f"relative {err / scale:.2e}, max|lse err| {lerr:.2e}")
    assert err <= 1e-2 * scale
    assert lerr <= 1e-3


@pytest.mark.parametrize("cfg_name,S,num_splits", [
    ("ctx1m_g32x2_d256", 24000, 1),          # four waves, hi parts summed by products
    ("nope8l_1m_g64x2_d128", 16000, 1),      # eight waves, hi parts summed by dot products
    (G64D64, 12000, 1),                      # two row blocks per wave
])
def test_verify_every_tile_heavy(cfg_name, S, num_splits):
    """Every 32-key tile holds one key whose weight is ~5 % of its row's running
    sum (its score grows by 0.05 per tile, staying inside the lazy margin of the
    split's first maximum), so every fast tile is heavy and keeps its weights' lo
    parts.  The result must then carry the hi + lo precision: well below the error
    that bf16-rounded weights alone give on the same input, computed here."""
    cfg = CFG[cfg_name] if isinstance(cfg_name, str) else cfg_name
    n_q, Hq, Hkv, D = 8, cfg["Hq"], cfg["Hkv"], cfg["D"]
    L = S + n_q
    rng = np.random.default_rng(93)
    # every query row ~ u = 1/16 per component (plus noise): a key c * 1 scores
    # ~ c * D / 16
    qf = 0.0625 + 0.01 * rng.standard_normal((1, n_q, Hq, D))
    q = W.bf16_round(qf.astype(np.float32))
    Kf = 0.25 * rng.standard_normal((L, Hkv, D))
    for n in range(S // 32):
        beta = 4.0 + 0.05 * n                 # the spike's score, in nats
        Kf[32 * n + (7 * n) % 32] = beta / (0.0625 * D)
    K = W.bf16_round(Kf.astype(np.float32))
    V = W.bf16_round(rng.standard_normal((L, Hkv, D)).astype(np.float32))
    o, l, ro, rl = _verify_custom(cfg_name, 93, S, n_q, K, V, q, num_splits)
    got = o.double().cpu().numpy().reshape(ro.shape)
    err = float(np.max(np.abs(got - ro)))
    lerr = float(np.max(np.abs(l.double().cpu().numpy().reshape(rl.shape) - rl)))
    # the same rows with every weight rounded to bf16 (what PV sees without the
    # lo parts), normalised by the rounded weights
    Qd = W.bf16_to_f32(q).astype(np.float64)[0]
    Kd = W.bf16_to_f32(K).astype(np.float64)
    Vd = W.bf16_to_f32(V).astype(np.float64)
    G = Hq // Hkv
    hi_err = 0.0
    for g in range(Hkv):
        for qi in (0, n_q - 1):
            lim = S + qi + 1                  # causal: keys up to the query's position
            s = Qd[qi, g * G] @ Kd[:lim, g].T
            w = np.exp(s - s.max())
            wh = W.bf16_to_f32(W.bf16_round(w.astype(np.float32))).astype(np.float64)
            ex = w @ Vd[:lim, g] / w.sum()
            hi = wh @ Vd[:lim, g] / wh.sum()
            hi_err = max(hi_err, float(np.max(np.abs(hi - ex))))
    print(f"verify every tile heavy {cfg_name}: max|o err| {err:.2e} (bf16 weights alone: "
          f"{hi_err:.2e}), max|lse err| {lerr:.2e}")
    assert err <= 0.1 * hi_err
    assert lerr <= 1e-4


@pytest.mark.parametrize("cfg_name,S,num_splits", [
    ("ctx1m_g32x2_d256", 20000, 1),
    ("nope8l_1m_g64x2_d128", 12000, 2),
])
def test_verify_needle_raises_the_maximum_mid_split(cfg_name, S, num_splits):
    """A key aligned with one query row's query, in the middle of a long split, lifts
    that row's score far above the running maximum (a raise beyond the lazy margin):
    the row owner rescales and the other waves' accumulators of that row block
    follow the published factors."""
    cfg = CFG[cfg_name]
    n_q, Hq, Hkv, D = 8, cfg["Hq"], cfg["Hkv"], cfg["D"]
    K = W.kv_positions(92, "target_k", 0, 0, S + n_q, Hkv, D)
    V = W.kv_positions(92, "target_v", 0, 0, S + n_q, Hkv, D)
    q = W.queries(92, "q_verify", (1, n_q, Hq), D)
    qf = W.bf16_to_f32(q)
    p = S // 2 + 7
    for g in range(Hkv):
        # query 3 of the first head of kv head g: score ~ 8 * sum |q| ~ 100+
        K[p, g] = W.bf16_round(8.0 * np.sign(qf[0, 3, g * (Hq // Hkv)]))
    o, l, ro, rl = _verify_custom(cfg_name, 92, S, n_q, K, V, q, num_splits)
    compare(o, l, ro, rl, f"verify needle {cfg_name}")


def _tree_masks(n_q, kind):
    if kind == "binary":      # node i's parent is (i - 1) // 2
        masks = []
        for i in range(n_q):
            mk, j = 0, i
            while True:
                mk |= 1 << j
                if j == 0:
                    break
                j = (j - 1) // 2
            masks.append(mk)
        return masks
    if kind == "star":        # every node a child of the root
        return [1] + [1 | (1 << i) for i in range(1, n_q)]
    return [(1 << (i + 1)) - 1 for i in range(n_q)]   # chain


@pytest.mark.parametrize("cfg_name,S,n_q,kind,num_splits", [
    ("ctx1m_g32x2_d256", 20000, 8, "binary", 2),       # shared kernel, 128 rows, long splits
    ("ctx1m_g32x2_d256", 3000, 8, "star", 0),
    ("ctx128k_g32x4_d128", 9000, 4, "binary", 0),      # split kernel, 32 rows
    ("nope8l_1m_g64x2_d128", 6000, 8, "star", 1),      # shared kernel, two row blocks
    ("ctx1m_g32x2_d256", 5000, 8, "chain", 3),
])
def test_verify_tree(cfg_name, S, n_q, kind, num_splits):
    """Verify of a tree of proposals: query i sees the prefix and its ancestors."""
    lib = _lib()
    cfg = CFG[cfg_name]
    vs = VerifyScenario(cfg, 80 + n_q, [S], n_q)
    vs.append_proposed()
    masks = _tree_masks(n_q, kind)
    tm = torch().tensor([masks], dtype=torch().int64, device="cuda")
    L = S + n_q
    o, l = lib.verify_attn_tree(dev_bf16(vs.q), vs.kv.k, vs.kv.v, vs.kv.block_table, dev_i32([L]),
                                tm, L, 1.0, num_splits=num_splits)
    torch().cuda.synchronize()
    ro, rl = OA.verify_tree(vs.q[0], vs.K[0], vs.V[0], L, masks, 1.0)
    compare(o[0], l[0], ro, rl, f"tree verify {cfg_name} {kind}")


def test_verify_same_in_both_arms():
    """The verify call reads only the target KV: repeated calls (one per arm) agree bitwise."""
    lib = _lib()
    vs, o1, l1 = _verify_case(CFG["ctx128k_g32x4_d128"], 24, [9000], 4)
    lens = vs.lens()
    o2, l2 = lib.verify_attn(dev_bf16(vs.q), vs.kv.k, vs.kv.v, vs.kv.block_table, dev_i32(lens),
                             max(lens))
    torch().cuda.synchronize()
    assert torch().equal(o1, o2) and torch().equal(l1, l2)


def test_verify_single_query_equals_draft_full():
    lib = _lib()
    cfg = CFG["ctx1m_g32x2_d256"]
    vs = VerifyScenario(cfg, 25, [7000], 1)
    vs.append_proposed()
    lens = vs.lens()
    o, l = lib.verify_attn(dev_bf16(vs.q), vs.kv.k, vs.kv.v, vs.kv.block_table, dev_i32(lens),
                           lens[0])
    od, ld = lib.draft_attn_full(dev_bf16(vs.q[:, 0]), vs.kv.k, vs.kv.v, vs.kv.block_table,
                                 dev_i32(lens), lens[0])
    torch().cuda.synchronize()
    assert torch().equal(o[:, 0], od) and torch().equal(l[:, 0], ld)


# ------------------------------------------------------------------ appends (bit-exact)

def _unpack_k(kc, D):
    """Tiled K cache -> [page, Hkv, 64, D] bit patterns (layout of include/wmtp.h)."""
    a = kc.view(torch().int16).cpu().numpy().view(np.uint16)
    P, Hkv = a.shape[:2]
    a = a.reshape(P, Hkv, 2, D // 16, 32, 16)                      # [P, Hkv, half, dblock, pos, 16]
    a = a.transpose(0, 1, 2, 4, 3, 5)                              # [P, Hkv, half, pos, dblock, 16]
    return a.reshape(P, Hkv, 64, D)


def _unpack_v(vc, D):
    a = vc.view(torch().int16).cpu().numpy().view(np.uint16)
    P, Hkv = a.shape[:2]
    a = a.reshape(P, Hkv, 2, 2, D, 16)                             # [P, Hkv, half, kstep, D, 16]
    a = a.transpose(0, 1, 2, 3, 5, 4)                              # [P, Hkv, half, kstep, 16, D]
    return a.reshape(P, Hkv, 64, D)


def test_paged_append_layout_bitexact():
    cfg = CFG["ctx1m_g32x2_d256"]
    sc = DraftScenario(cfg, 40, [1000, 77], 3, perm=True, poison=False)
    for j in range(1, 4):
        sc.append(j)
    torch().cuda.synchronize()
    Kp = _unpack_k(sc.kv.k, cfg["D"])
    Vp = _unpack_v(sc.kv.v, cfg["D"])
    bt = sc.kv.block_table.cpu().numpy()
    for b in range(sc.B):
        L = sc.S[b] + 3
        for p in range(L):
            page = bt[b, p // 64]
            assert np.array_equal(Kp[page, :, p % 64], sc.K[b][p]), (b, p)
            assert np.array_equal(Vp[page, :, p % 64], sc.V[b][p]), (b, p)


@pytest.mark.parametrize("n_sink,C,T0,n_new", [(4, 1024, 0, 5000), (4, 1024, 3000, 1),
                                               (4, 4096, 0, 10000), (0, 64, 10, 200),
                                               (63, 128, 50, 3), (4, 1024, 2, 1)])
def test_ring_append_bitexact(n_sink, C, T0, n_new):
    """ring_pos against the oracle ring model, and every filled slot's K/V against
    the logical K/V of the position it holds; bulk and single appends."""
    lib = _lib()
    from long_context_decode_attention_amd import scenario as scn
    B, Hkv, D = 2, 2, 128
    K = [W.kv_positions(50 + b, "draft_k", b, 0, T0 + n_new, Hkv, D) for b in range(B)]
    V = [W.kv_positions(50 + b, "draft_v", b, 0, T0 + n_new, Hkv, D) for b in range(B)]
    ring = lib.new_ring(B, C, Hkv, D, n_sink, C - n_sink)
    model = OR.RingModel(B, C, n_sink)
    for b in range(B):
        scn.fill_ring(ring, b, K[b][:T0], V[b][:T0])
        model.append(b, T0)
    # then the rest: one bulk call for the batch
    kn = np.stack([K[b][T0:] for b in range(B)])
    vn = np.stack([V[b][T0:] for b in range(B)])
    if n_new:
        lib.ring_append(ring, dev_bf16(kn), dev_bf16(vn))
    for b in range(B):
        model.append(b, n_new)
    torch().cuda.synchronize()
    pos = ring.pos.cpu().numpy()
    T = ring.T.cpu().numpy()
    # ring page i of request b is pool page b * C/64 + i: [B, C/64, Hkv, 64, D] -> [B, C, Hkv, D]
    Kp = _unpack_k(ring.k, D).reshape(B, C // 64, Hkv, 64, D).transpose(0, 1, 3, 2, 4)
    Kp = Kp.reshape(B, C, Hkv, D)
    Vp = _unpack_v(ring.v, D).reshape(B, C // 64, Hkv, 64, D).transpose(0, 1, 3, 2, 4)
    Vp = Vp.reshape(B, C, Hkv, D)
    for b in range(B):
        assert T[b] == T0 + n_new
        assert pos[b].tolist() == model.pos[b]
        assert pos[b].tolist() == OR.expected_pos_after(T0 + n_new, n_sink, C)
        for s in range(C):
            p = pos[b, s]
            if p >= 0:
                assert np.array_equal(Kp[b, s], K[b][p]) and np.array_equal(Vp[b, s], V[b][p])


def test_ring_rollback_with_slack():
    """Slack slots absorb a rollback: after appending 3 speculative positions and
    rolling T back by 3, the window read equals the oracle window."""
    lib = _lib()
    from long_context_decode_attention_amd import scenario as scn
    Hq, Hkv, D, n_sink, n_recent, C = 16, 2, 128, 4, 1020 - 60, 1024
    T = 5000
    K = W.kv_positions(60, "draft_k", 0, 0, T + 3, Hkv, D)
    V = W.kv_positions(60, "draft_v", 0, 0, T + 3, Hkv, D)
    ring = lib.new_ring(1, C, Hkv, D, n_sink, n_recent)
    scn.fill_ring(ring, 0, K[:T + 3], V[:T + 3])
    ring.T.fill_(T)
    q = W.queries(61, "q_draft", (1, Hq), D)
    o, l = lib.draft_attn_window(dev_bf16(q), ring)
    torch().cuda.synchronize()
    ro, rl = OA.draft_window(q[0], K, V, T, n_sink, n_recent, 1.0)
    compare(o[0], l[0], ro, rl, "window after rollback")


# ------------------------------------------------------------------ argument checks

def test_error_codes():
    lib = _lib()
    cfg = CFG["ctx8k_g16x2_d128"]
    sc = DraftScenario(cfg, 70, [100], 1, poison=False)
    q = dev_bf16(sc.q(1))
    lens = dev_i32([100])
    with pytest.raises(lib.WmtpError) as e:
        lib.draft_attn_full(q, sc.kv.k, sc.kv.v, sc.kv.block_table, lens, 100, float("nan"))
    assert e.value.status == 1
    small = torch().empty(16, dtype=torch().uint8, device="cuda")
    with pytest.raises(lib.WmtpError) as e:
        lib.draft_attn_full(q, sc.kv.k, sc.kv.v, sc.kv.block_table, lens, 1 << 20, workspace=small,
                            num_splits=4)
    assert e.value.status == 3


# ------------------------------------------------------------------ fp8 draft KV

def _fp8_case(cfg_name, seed, S, k_scale, v_scale, perm=True):
    """A paged fp8 draft cache holding positions 0 .. S-1 of the seeded draft K/V,
    written by the fp8 append in a few calls; returns what the tests need.
    cfg_name is a workload name or a dict with Hq, Hkv and D."""
    from oracle import fp8 as F
    from long_context_decode_attention_amd import scenario as scn
    lib = _lib()
    cfg = cfg_name if isinstance(cfg_name, dict) else CFG[cfg_name]
    Hkv, D = cfg["Hkv"], cfg["D"]
    K = W.kv_positions(seed, "draft_k", 0, 0, S, Hkv, D)
    V = W.kv_positions(seed, "draft_v", 0, 0, S, Hkv, D)
    n_pages = (S + 63) // 64 + 1
    table = W.page_permutation(seed, "draft_k", n_pages) if perm else np.arange(n_pages, dtype=np.int32)
    k8, v8 = lib.new_paged_cache_fp8(n_pages, Hkv, D)
    k8.fill_(0x7F)                  # NaN codes wherever nothing was written
    v8.fill_(0x7F)
    bt = torch().tensor(table.reshape(1, -1), dtype=torch().int32, device="cuda")
    cuts = [0, S // 3, S // 3 + 1, S]
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        if hi > lo:
            lib.paged_append_fp8(k8, v8, bt, dev_i32([lo]), dev_bf16(K[lo:hi][None]),
                                 dev_bf16(V[lo:hi][None]), k_scale, v_scale)
    torch().cuda.synchronize()
    inv_k = np.float32(1.0) / np.float32(k_scale)
    inv_v = np.float32(1.0) / np.float32(v_scale)
    Kc, Vc = F.bf16_to_e4m3(K, inv_k), F.bf16_to_e4m3(V, inv_v)
    Kq, Vq = F.dequantize_e4m3(Kc, k_scale), F.dequantize_e4m3(Vc, v_scale)
    return dict(cfg=cfg, k8=k8, v8=v8, bt=bt, table=table, Kc=Kc, Vc=Vc, Kq=Kq, Vq=Vq)


@pytest.mark.parametrize("k_scale,v_scale", [(1.0, 1.0), (0.5, 2.0), (0.01, 0.003)])
def test_fp8_append_codes_bitexact(k_scale, v_scale):
    """The fp8 append stores exactly the oracle quantizer's codes, in the tile layout."""
    c = _fp8_case("ctx1m_g32x2_d256", 90, 1000, k_scale, v_scale)
    D = c["cfg"]["D"]
    Kp = c["k8"].cpu().numpy().reshape(-1, c["cfg"]["Hkv"], 2, D // 16, 32, 16)
    Kp = Kp.transpose(0, 1, 2, 4, 3, 5).reshape(Kp.shape[0], c["cfg"]["Hkv"], 64, D)
    Vp = c["v8"].cpu().numpy().reshape(-1, c["cfg"]["Hkv"], 2, 2, D, 16)
    Vp = Vp.transpose(0, 1, 2, 3, 5, 4).reshape(Vp.shape[0], c["cfg"]["Hkv"], 64, D)
    for p in range(1000):
        page = c["table"][p // 64]
        assert np.array_equal(Kp[page, :, p % 64], c["Kc"][p]), p
        assert np.array_equal(Vp[page, :, p % 64], c["Vc"][p]), p


@pytest.mark.parametrize("cfg_name,S,k_scale,v_scale,num_splits", [
    ("ctx1m_g32x2_d256", 40000, 1.0, 1.0, 0),
    ("ctx1m_g32x2_d256", 9000, 0.5, 2.0, 1),
    ("ctx128k_g32x4_d128", 20011, 0.25, 0.5, 0),
    ("ctx128k_g32x4_d128", 70001, 1.0, 1.0, 0),     # >= 64K keys: twice the workgroups
    ("nope8l_1m_g64x2_d128", 3000, 1.0, 1.0, 3),     # 32 rows per kv head
    ("ctx8k_g16x2_d128", 65, 1.0, 1.0, 0),
])
def test_fp8_draft_full_and_window(cfg_name, S, k_scale, v_scale, num_splits):
    """Native draft and truncated-index window over fp8 caches against the oracle
    over the dequantized keys and values."""
    lib = _lib()
    c = _fp8_case(cfg_name, 91 + S % 7, S, k_scale, v_scale)
    cfg = c["cfg"]
    q = W.queries(92, "q_draft", (1, cfg["Hq"]), cfg["D"])
    o, l = lib.draft_attn_full_fp8(dev_bf16(q), c["k8"], c["v8"], c["bt"], dev_i32([S]), S,
                                   k_scale, v_scale, 1.0, num_splits=num_splits)
    ow, lw = lib.draft_attn_full_fp8(dev_bf16(q), c["k8"], c["v8"], c["bt"], dev_i32([S]), S,
                                     k_scale, v_scale, 1.0, num_splits=num_splits,
                                     window=(cfg["n_sink"], cfg["n_recent"]))
    torch().cuda.synchronize()
    ro, rl = OA.draft_full(q[0], c["Kq"], c["Vq"], S, 1.0)
    compare(o[0], l[0], ro, rl, f"fp8 full {cfg_name} S={S}")
    rwo, rwl = OA.draft_window(q[0], c["Kq"], c["Vq"], S, cfg["n_sink"], cfg["n_recent"], 1.0)
    compare(ow[0], lw[0], rwo, rwl, f"fp8 window {cfg_name} S={S}")
    if S >= 65536:
        # the partials of the fp8 plan (twice the workgroups at D = 128) merge to the same
        # result through the exported combine, in the layout partials_view(fp8=True) gives
        G = cfg["Hq"] // cfg["Hkv"]
        ws = lib.draft_attn_full_fp8(dev_bf16(q), c["k8"], c["v8"], c["bt"], dev_i32([S]), S,
                                     k_scale, v_scale, 1.0, partials_only=True)
        po, pl = lib.partials_view(ws, 1, cfg["Hq"], cfg["Hkv"], cfg["D"], 1, S, fp8=True)
        splits = lib.plan_splits(1, cfg["Hq"], cfg["Hkv"], cfg["D"], 1, S, fp8=True)
        bf16_splits = lib.plan_splits(1, cfg["Hq"], cfg["Hkv"], cfg["D"], 1, S)
        assert bf16_splits < splits <= 2 * bf16_splits     # about twice (whole tiles per split)
        oc, lc = lib.split_combine(po, pl, 1, cfg["Hkv"], G, 1, splits_per_group=splits)
        torch().cuda.synchronize()
        assert torch().equal(oc.view(o.shape), o) and torch().equal(lc.view(l.shape), l)


D64 = dict(Hq=16, Hkv=2, D=64)   # head dim 64: fewer 1 KB tile chunks than waves in the fp8 verify


@pytest.mark.parametrize("cfg_name,S,n_q,k_scale,v_scale,num_splits", [
    ("ctx1m_g32x2_d256", 20000, 8, 1.0, 1.0, 1),       # 128 rows, one split of 625 tiles
    ("ctx1m_g32x2_d256", 9000, 8, 0.5, 2.0, 0),
    ("nope8l_1m_g64x2_d128", 12000, 8, 1.0, 1.0, 2),   # 256 rows: eight waves
    ("ctx128k_g32x4_d128", 15000, 8, 0.25, 0.5, 2),    # 64 rows: two row blocks per wave
    ("ctx8k_g16x2_d128", 3000, 4, 1.0, 1.0, 0),        # 32 rows: the split kernel
    (D64, 7000, 8, 1.0, 1.0, 1),                       # 64 rows at D = 64
    ("ctx1m_g32x2_d256", 100, 8, 1.0, 1.0, 0),         # short: a masked tail over NaN codes
    ("ctx1m_g32x2_d256", 0, 8, 1.0, 1.0, 0),           # the proposed positions only
])
def test_fp8_verify(cfg_name, S, n_q, k_scale, v_scale, num_splits):
    """The causal verify over fp8 target caches against the oracle's verify over the
    dequantized keys and values (slots past the sequence hold NaN codes)."""
    lib = _lib()
    L = S + n_q
    c = _fp8_case(cfg_name, 93 + S % 11, L, k_scale, v_scale)
    cfg = c["cfg"]
    q = W.queries(94 + S % 5, "q_verify", (1, n_q, cfg["Hq"]), cfg["D"])
    o, l = lib.verify_attn_fp8(dev_bf16(q), c["k8"], c["v8"], c["bt"], dev_i32([L]), L, k_scale,
                               v_scale, 1.0, num_splits=num_splits)
    torch().cuda.synchronize()
    ro, rl = OA.verify(q[0], c["Kq"], c["Vq"], L, 1.0)
    err, lerr = compare(o[0], l[0], ro, rl, f"fp8 verify S={S} n_q={n_q}")
    print(f"fp8 verify D={cfg['D']} rows={n_q * cfg['Hq'] // cfg['Hkv']} S={S}: "
          f"max|o err| {err:.2e}, max|lse err| {lerr:.2e}")


def test_draft_context_pass_batch_of_two():
    """Two rings at different lengths (one not yet full): each request's queries
    sit at its own ring_T - n_q + i."""
    lib = _lib()
    from long_context_decode_attention_amd import scenario as scn
    cfg = CFG["ctx128k_g32x4_d128"]
    Hq, Hkv, D = cfg["Hq"], cfg["Hkv"], cfg["D"]
    C, ns, nr, n_q = 1088, 4, 1020, 8
    lens = [5000, 700]
    ring = lib.new_ring(2, C, Hkv, D, ns, nr)
    scn.poison(ring.k)
    scn.poison(ring.v)
    KV = []
    for b, L in enumerate(lens):
        K = W.kv_positions(140 + b, "draft_k", b, 0, L, Hkv, D)
        V = W.kv_positions(140 + b, "draft_v", b, 0, L, Hkv, D)
        scn.fill_ring(ring, b, K, V)
        KV.append((K, V))
    q = W.queries(141, "q_ctx", (2, n_q, Hq), D)
    o, l = lib.draft_context_window(dev_bf16(q), ring, 1.0)
    torch().cuda.synchronize()
    for b, L in enumerate(lens):
        ro, rl = OA.draft_context_window(q[b], KV[b][0], KV[b][1], L, ns, nr, 1.0)
        compare(o[b], l[b], ro, rl, f"context pass b={b} L={L}")


def test_verify_tree_ragged_batch():
    """Two sequences of different lengths, each with its own tree."""
    lib = _lib()
    cfg = CFG["ctx1m_g32x2_d256"]
    n_q = 8
    vs = VerifyScenario(cfg, 150, [3000, 7777], n_q)
    vs.append_proposed()
    masks = [_tree_masks(n_q, "binary"), _tree_masks(n_q, "star")]
    tm = torch().tensor(masks, dtype=torch().int64, device="cuda")
    lens = vs.lens()
    o, l = lib.verify_attn_tree(dev_bf16(vs.q), vs.kv.k, vs.kv.v, vs.kv.block_table, dev_i32(lens),
                                tm, max(lens), 1.0)
    torch().cuda.synchronize()
    for b in range(2):
        ro, rl = OA.verify_tree(vs.q[b], vs.K[b], vs.V[b], lens[b], masks[b], 1.0)
        compare(o[b], l[b], ro, rl, f"tree verify b={b}")
