"""GPU test of ``wmtp_draft_step_window_static``: the fused windowed draft step
with its split partials in the library's static scratch instead of a caller's
workspace.  Two calls in a row, the second with a smaller input, each checked
against ``wmtp_draft_step_window`` on an identical ring (the same kernels and
plan, so bit for bit: output, lse and the ring afterwards) and against the
float64 oracle."""

import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from tests.gpu_common import compare, dev_bf16, torch

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, D, C, n_sink, n_recent, S, n_new, seed):
    import long_context_decode_attention_amd as lib
    from long_context_decode_attention_amd import scenario as sc
    t = torch()
    total = [s + n_new for s in S]
    K = [W.kv_positions(seed, "draft_k", b, 0, total[b], Hkv, D) for b in range(B)]
    V = [W.kv_positions(seed, "draft_v", b, 0, total[b], Hkv, D) for b in range(B)]
    rings = []
    for _ in range(2):
        r = lib.new_ring(B, C, Hkv, D, n_sink, n_recent)
        sc.poison(r.k)
        sc.poison(r.v)
        for b in range(B):
            sc.fill_ring(r, b, K[b][:S[b]], V[b][:S[b]])
        rings.append(r)
    ref, stat = rings
    q = W.queries(seed, "q_draft", (B, Hq), D, step=1)
    kn = dev_bf16(np.stack([K[b][S[b]:S[b] + n_new] for b in range(B)]))
    vn = dev_bf16(np.stack([V[b][S[b]:S[b] + n_new] for b in range(B)]))
    qt = dev_bf16(q)
    o1, l1 = lib.draft_step_window(qt, ref, kn, vn, 1.0)
    o2, l2 = lib.draft_step_window_static(qt, stat, kn, vn, 1.0)
    t.cuda.synchronize()
    assert t.equal(o1, o2) and t.equal(l1, l2), "static scratch result differs from the workspace call"
    assert t.equal(ref.T, stat.T) and t.equal(ref.pos, stat.pos)
    assert t.equal(ref.k.view(t.int16), stat.k.view(t.int16))
    assert t.equal(ref.v.view(t.int16), stat.v.view(t.int16))
    for b in range(B):
        ro, rl = OA.draft_window(q[b], K[b], V[b], total[b], n_sink, n_recent, 1.0)
        compare(o2[b], l2[b], ro, rl, f"static step b={b}")


def test_static_scratch_step_two_calls():
    t = torch()
    assert t.cuda.is_available(), "GPU tests need a GPU"
    import long_context_decode_attention_amd as lib
    lib.load()
    # the 1M workload's heads and ring, two requests
    _case(2, 32, 2, 256, 4096, 4, 4092, [9000, 5000], 1, seed=81)
    # then a smaller input on the same scratch: one request, 8k workload's shapes
    _case(1, 16, 2, 128, 1024, 4, 1020, [3000], 2, seed=82)


def test_static_scratch_rejects_oversized():
    """Partials beyond the scratch: WMTP_ERR_WORKSPACE, nothing launched."""
    t = torch()
    import long_context_decode_attention_amd as lib
    B, Hq, Hkv, D, C = 64, 256, 1, 256, 4096
    need = lib.step_workspace_bytes(B, Hq, Hkv, D, C)
    assert need > lib.STATIC_SCRATCH_BYTES
    ring = lib.new_ring(B, C, Hkv, D, 4, 4092)
    q = t.zeros(B, Hq, D, dtype=t.bfloat16, device="cuda")
    kn = t.zeros(B, 1, Hkv, D, dtype=t.bfloat16, device="cuda")
    with pytest.raises(lib.WmtpError) as e:
        lib.draft_step_window_static(q, ring, kn, kn)
    assert e.value.status == 3
    t.cuda.synchronize()
    assert int(ring.T.abs().sum()) == 0 and int((ring.pos >= 0).sum()) == 0
