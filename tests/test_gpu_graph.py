"""The calls under HIP graph capture: a decode step's launches recorded once and
replayed, each replay checked against the same calls run eagerly.

Every call only launches kernels on the given stream (no allocation, no memset, no
synchronisation), so a graph holds the whole step.  Between replays the test
restores the ring and caches eagerly and synchronises, then compares every output
and the ring afterwards with the eager results, bit for bit (same kernels, same
split plan, same inputs).
"""

import numpy as np
import pytest

import workloads as W
from tests.gpu_common import dev_bf16, dev_i32, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a GPU"
    import long_context_decode_attention_amd as lib
    lib.load()
    yield


def test_decode_step_graph_replays_match_eager():
    import long_context_decode_attention_amd as lib
    from long_context_decode_attention_amd import scenario as sc
    t = torch()
    Hq, Hkv, D, C, n_sink, n_recent = 16, 2, 128, 1024, 4, 1020
    S, steps, n_q, seed = 3000, 3, 4, 21
    K = W.kv_positions(seed, "draft_k", 0, 0, S + steps + n_q, Hkv, D)
    V = W.kv_positions(seed, "draft_v", 0, 0, S + steps + n_q, Hkv, D)
    ring = lib.new_ring(1, C, Hkv, D, n_sink, n_recent)
    sc.fill_ring(ring, 0, K[:S], V[:S])
    ring_c = lib.new_ring(1, C + 64, Hkv, D, n_sink, n_recent)   # slack for the context pass
    sc.fill_ring(ring_c, 0, K[:S], V[:S])
    n_pages = (S + steps + n_q + 63) // 64
    kv = sc.alloc_paged_kv([S + steps + n_q], Hkv, D, W.page_permutation(seed, "draft_k", n_pages))
    sc.fill_paged(kv, 0, 0, K[:S], V[:S])
    state = [ring.k, ring.v, ring.pos, ring.T, kv.k, kv.v, ring_c.k, ring_c.v, ring_c.pos, ring_c.T]
    snap = [x.clone() for x in state]

    qd = [dev_bf16(W.queries(seed, "q_draft", (1, Hq), D, step=j)) for j in range(steps)]
    kn = [dev_bf16(K[S + j][None, None]) for j in range(steps)]
    vn = [dev_bf16(V[S + j][None, None]) for j in range(steps)]
    qv = dev_bf16(W.queries(seed, "q_verify", (1, n_q, Hq), D))
    kt = dev_bf16(K[S + steps:S + steps + n_q][None])
    vt = dev_bf16(V[S + steps:S + steps + n_q][None])
    pos = dev_i32([S])
    pos_t = dev_i32([S + steps])
    lens = dev_i32([S + 1])
    lens_t = dev_i32([S + steps + n_q])
    Lmax = S + steps + n_q
    ws = lib.new_workspace(lib.step_workspace_bytes(1, Hq, Hkv, D, C))
    ws_f = lib.new_workspace(lib.workspace_bytes(1, Hq, Hkv, D, 1, Lmax))
    ws_v = lib.new_workspace(lib.workspace_bytes(1, Hq, Hkv, D, n_q, Lmax))
    outs = [t.empty(1, Hq, D, device="cuda") for _ in range(steps)]
    lses = [t.empty(1, Hq, device="cuda") for _ in range(steps)]
    o_f, l_f = t.empty(1, Hq, D, device="cuda"), t.empty(1, Hq, device="cuda")
    o_v, l_v = t.empty(1, n_q, Hq, D, device="cuda"), t.empty(1, n_q, Hq, device="cuda")
    qc = dev_bf16(W.queries(seed, "q_ctx", (1, n_q, Hq), D))
    ws_c = lib.new_workspace(lib.step_workspace_bytes(1, Hq, Hkv, D, C + 64, 0, n_q))
    o_c, l_c = t.empty(1, n_q, Hq, D, device="cuda"), t.empty(1, n_q, Hq, device="cuda")

    def step():
        for j in range(steps):
            lib.draft_step_window(qd[j], ring, kn[j], vn[j], 1.0, outs[j], lses[j], ws)
        lib.paged_append(kv.k, kv.v, kv.block_table, pos, kn[0], vn[0])
        lib.draft_attn_full(qd[0], kv.k, kv.v, kv.block_table, lens, Lmax, 1.0, o_f, l_f, ws_f)
        lib.paged_append(kv.k, kv.v, kv.block_table, pos_t, kt, vt)
        lib.verify_attn(qv, kv.k, kv.v, kv.block_table, lens_t, Lmax, 1.0, o_v, l_v, ws_v)
        lib.draft_context_step_window(qc, ring_c, kt, vt, 1.0, o_c, l_c, ws_c)

    def restore():
        for x, y in zip(state, snap):
            x.copy_(y)
        t.cuda.synchronize()

    def results():
        return [x.clone() for x in outs + lses + [o_f, l_f, o_v, l_v, o_c, l_c] + state]

    restore()
    step()
    t.cuda.synchronize()
    eager = results()

    restore()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        step()
    t.cuda.synchronize()
    for r in range(4):
        restore()
        for x in outs + lses + [o_f, l_f, o_v, l_v, o_c, l_c]:
            x.fill_(float("nan"))   # stale results must not pass for replayed ones
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        got = results()
        for i, (a, b) in enumerate(zip(got, eager)):
            if a.dtype in (t.float32,):
                assert t.equal(a.view(t.int32), b.view(t.int32)), f"replay {r}: output {i} differs"
            elif a.dtype == t.bfloat16:
                assert t.equal(a.view(t.int16), b.view(t.int16)), f"replay {r}: cache {i} differs"
            else:
                assert t.equal(a, b), f"replay {r}: state {i} differs"
        assert int(ring.T[0]) == S + steps and int(ring_c.T[0]) == S + n_q
    assert np.isfinite(eager[0].cpu().numpy()).all()
