"""GPU parity at the full 1M-context size, in the launch configuration the
benchmark times (automatic split plan): the oracle checks sampled outputs (one
kv head's query rows; two of the eight verify queries)."""

import sys
import time

import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from tests.gpu_common import DraftScenario, VerifyScenario, compare, dev_bf16, dev_i32, torch

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[fullsize {time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def _group(q, K, V, g, G):
    """The one-kv-head sub-problem of kv head g."""
    return q[..., g * G:(g + 1) * G, :], K[:, g:g + 1, :], V[:, g:g + 1, :]


def test_ctx1m_draft_chain_and_verify_full_size():
    import long_context_decode_attention_amd as lib
    cfg = W.CONFIGS["ctx1m_g32x2_d256"]
    S, gamma, n_q = cfg["S"], cfg["gamma"], cfg["n_q"]
    G = cfg["Hq"] // cfg["Hkv"]
    _say("building draft state (1M positions, permuted pages, ring)")
    sc = DraftScenario(cfg, 100, [S], gamma, poison=False)
    # the windowed arm as the benchmark runs it: the fused draft step on a second
    # ring holding the same 1M positions
    from long_context_decode_attention_amd import scenario as scn
    ring2 = lib.new_ring(1, cfg["C"], cfg["Hkv"], cfg["D"], cfg["n_sink"], cfg["n_recent"])
    scn.fill_ring(ring2, 0, sc.K[0][:S], sc.V[0][:S])
    outs = {}
    for j in range(1, gamma + 1):
        sc.append(j)
        q = sc.q(j)
        qt = dev_bf16(q)
        lens = sc.lens(j)
        of, lf = lib.draft_attn_full(qt, sc.kv.k, sc.kv.v, sc.kv.block_table, dev_i32(lens), lens[0])
        ow, lw = lib.draft_attn_window(qt, sc.ring)
        kn = dev_bf16(sc.K[0][S + j - 1][None, None])
        vn = dev_bf16(sc.V[0][S + j - 1][None, None])
        os_, ls_ = lib.draft_step_window(qt, ring2, kn, vn)
        outs[j] = (q, of, lf, ow, lw, os_, ls_)
    torch().cuda.synchronize()
    t = torch()
    assert t.equal(ring2.T, sc.ring.T) and t.equal(ring2.pos, sc.ring.pos)
    assert t.equal(ring2.k.view(t.int16), sc.ring.k.view(t.int16))
    assert t.equal(ring2.v.view(t.int16), sc.ring.v.view(t.int16))
    _say("draft chain done (fused-step ring equals the appended ring); oracle on kv head 1, steps 1 and 7")
    for j in (1, gamma):
        q, of, lf, ow, lw, os_, ls_ = outs[j]
        L = S + j
        qg, Kg, Vg = _group(q[0], sc.K[0], sc.V[0], 1, G)
        ro, rl = OA.draft_full(qg, Kg, Vg, L, 1.0)
        compare(of[0, G:2 * G], lf[0, G:2 * G], ro, rl, f"full 1M step {j}")
        ro, rl = OA.draft_window(qg, Kg, Vg, L, cfg["n_sink"], cfg["n_recent"], 1.0)
        compare(ow[0, G:2 * G], lw[0, G:2 * G], ro, rl, f"window 1M step {j}")
        compare(os_[0, G:2 * G], ls_[0, G:2 * G], ro, rl, f"fused window step 1M step {j}")
        _say(f"step {j} matches")
    del sc, outs
    _say("building target state (1M + 8 positions)")
    vs = VerifyScenario(cfg, 101, [S], n_q, poison=False)
    vs.append_proposed()
    lens = vs.lens()
    o, l = lib.verify_attn(dev_bf16(vs.q), vs.kv.k, vs.kv.v, vs.kv.block_table, dev_i32(lens), lens[0])
    torch().cuda.synchronize()
    for i in (0, n_q - 1):
        qg, Kg, Vg = _group(vs.q[0, i], vs.K[0], vs.V[0], 0, G)
        ro, rl = OA.draft_full(qg, Kg, Vg, S + i + 1, 1.0)
        compare(o[0, i, :G], l[0, i, :G], ro, rl, f"verify 1M query {i}")
        _say(f"verify query {i} matches")


def test_ctx1m_next_rows_full_size():
    """The widened rows at 1M: the truncated paged index, the fp8 draft KV, the
    draft context pass over a ring with slack (also fused with its append), the
    tree verify and the verify over fp8 target KV, each in its automatic split
    plan, checked on kv head 1's rows (the verifies on kv head 0's)."""
    import long_context_decode_attention_amd as lib
    from long_context_decode_attention_amd import scenario as scn
    from oracle import fp8 as F
    cfg = W.CONFIGS["ctx1m_g32x2_d256"]
    S, n_q, Hkv, D = cfg["S"], cfg["n_q"], cfg["Hkv"], cfg["D"]
    ns, nr = cfg["n_sink"], cfg["n_recent"]
    G = cfg["Hq"] // Hkv
    _say("building draft state (1M positions, permuted pages)")
    sc = DraftScenario(cfg, 102, [S], 1, poison=False)
    sc.append(1)
    q = sc.q(1)
    qt = dev_bf16(q)
    L = S + 1
    op, lp = lib.draft_attn_window_paged(qt, sc.kv.k, sc.kv.v, sc.kv.block_table, dev_i32([L]), L,
                                         ns, nr)
    # the same draft KV as fp8 codes, on the same pages
    k8, v8 = lib.new_paged_cache_fp8(sc.kv.k.shape[0], Hkv, D)
    for lo in range(0, L, 1 << 16):
        hi = min(L, lo + (1 << 16))
        lib.paged_append_fp8(k8, v8, sc.kv.block_table, dev_i32([lo]), dev_bf16(sc.K[0][lo:hi][None]),
                             dev_bf16(sc.V[0][lo:hi][None]))
    o8, l8 = lib.draft_attn_full_fp8(qt, k8, v8, sc.kv.block_table, dev_i32([L]), L)
    # the context pass: a ring with 64 slots of slack, the last 8 positions as queries
    ring = lib.new_ring(1, cfg["C"] + 64, Hkv, D, ns, nr)
    scn.fill_ring(ring, 0, sc.K[0][:L], sc.V[0][:L])
    qc = W.queries(103, "q_ctx", (1, n_q, cfg["Hq"]), D)
    oc, lc = lib.draft_context_window(dev_bf16(qc), ring)
    # the same pass fused with the append of its 8 positions, on a ring holding the rest
    ring_f = lib.new_ring(1, cfg["C"] + 64, Hkv, D, ns, nr)
    scn.fill_ring(ring_f, 0, sc.K[0][:L - n_q], sc.V[0][:L - n_q])
    kc, vc = dev_bf16(sc.K[0][L - n_q:L][None]), dev_bf16(sc.V[0][L - n_q:L][None])
    ocf, lcf = lib.draft_context_step_window(dev_bf16(qc), ring_f, kc, vc)
    torch().cuda.synchronize()
    t = torch()
    assert t.equal(ring_f.T, ring.T) and t.equal(ring_f.pos, ring.pos)
    assert t.equal(ring_f.k.view(t.int16), ring.k.view(t.int16))
    assert t.equal(ring_f.v.view(t.int16), ring.v.view(t.int16))
    _say("oracle on kv head 1")
    qg, Kg, Vg = _group(q[0], sc.K[0], sc.V[0], 1, G)
    ro, rl = OA.draft_window(qg, Kg, Vg, L, ns, nr, 1.0)
    compare(op[0, G:2 * G], lp[0, G:2 * G], ro, rl, "paged window 1M")
    _say("truncated paged index matches")
    Kq = F.dequantize_e4m3(F.bf16_to_e4m3(Kg[:L]))
    Vq = F.dequantize_e4m3(F.bf16_to_e4m3(Vg[:L]))
    ro, rl = OA.draft_full(qg, Kq, Vq, L, 1.0)
    compare(o8[0, G:2 * G], l8[0, G:2 * G], ro, rl, "fp8 full 1M")
    del Kq, Vq
    _say("fp8 native draft matches")
    qcg = qc[0][:, G:2 * G]
    ro, rl = OA.draft_context_window(qcg, Kg, Vg, L, ns, nr, 1.0)
    compare(oc[0, :, G:2 * G], lc[0, :, G:2 * G], ro, rl, "context pass 1M")
    compare(ocf[0, :, G:2 * G], lcf[0, :, G:2 * G], ro, rl, "fused context pass 1M")
    _say("context pass matches (and fused with its append; rings equal)")
    del sc, ring, ring_f, k8, v8
    _say("building target state (1M + 8 positions)")
    vs = VerifyScenario(cfg, 104, [S], n_q, poison=False)
    vs.append_proposed()
    Lt = S + n_q
    masks = []
    for i in range(n_q):          # binary tree: node i's parent (i - 1) // 2
        mk, j = 0, i
        while True:
            mk |= 1 << j
            if j == 0:
                break
            j = (j - 1) // 2
        masks.append(mk)
    tm = torch().tensor([masks], dtype=torch().int64, device="cuda")
    o, l = lib.verify_attn_tree(dev_bf16(vs.q), vs.kv.k, vs.kv.v, vs.kv.block_table, dev_i32([Lt]),
                                tm, Lt)
    torch().cuda.synchronize()
    # each sampled query over the prefix plus its ancestors
    for i in (0, n_q - 1):
        rows = np.concatenate([np.arange(S), [S + a for a in range(n_q) if (masks[i] >> a) & 1]])
        qg, Kg, Vg = _group(vs.q[0, i], vs.K[0], vs.V[0], 0, G)
        ro, rl = OA.draft_over(qg, Kg, Vg, rows.astype(np.int64), 1.0)
        compare(o[0, i, :G], l[0, i, :G], ro, rl, f"tree verify 1M query {i}")
        _say(f"tree verify query {i} matches")
    # the causal verify over the same target KV as fp8 codes, on the same pages
    k8, v8 = lib.new_paged_cache_fp8(vs.kv.k.shape[0], Hkv, D)
    for lo in range(0, Lt, 1 << 16):
        hi = min(Lt, lo + (1 << 16))
        lib.paged_append_fp8(k8, v8, vs.kv.block_table, dev_i32([lo]), dev_bf16(vs.K[0][lo:hi][None]),
                             dev_bf16(vs.V[0][lo:hi][None]))
    o8, l8 = lib.verify_attn_fp8(dev_bf16(vs.q), k8, v8, vs.kv.block_table, dev_i32([Lt]), Lt)
    torch().cuda.synchronize()
    _say("fp8 verify done; oracle on kv head 0 over the dequantized KV")
    qg, Kg, Vg = _group(vs.q[0], vs.K[0], vs.V[0], 0, G)
    Kq = F.dequantize_e4m3(F.bf16_to_e4m3(Kg[:Lt]))
    Vq = F.dequantize_e4m3(F.bf16_to_e4m3(Vg[:Lt]))
    for i in (0, n_q - 1):
        ro, rl = OA.draft_full(qg[i], Kq, Vq, S + i + 1, 1.0)
        compare(o8[0, i, :G], l8[0, i, :G], ro, rl, f"fp8 verify 1M query {i}")
        _say(f"fp8 verify query {i} matches")
