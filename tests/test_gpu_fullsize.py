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
    outs = {}
    for j in range(1, gamma + 1):
        sc.append(j)
        q = sc.q(j)
        qt = dev_bf16(q)
        lens = sc.lens(j)
        of, lf = lib.draft_attn_full(qt, sc.kv.k, sc.kv.v, sc.kv.block_table, dev_i32(lens), lens[0])
        ow, lw = lib.draft_attn_window(qt, sc.ring)
        outs[j] = (q, of, lf, ow, lw)
    torch().cuda.synchronize()
    _say("draft chain done; oracle on kv head 1, steps 1 and 7")
    for j in (1, gamma):
        q, of, lf, ow, lw = outs[j]
        L = S + j
        qg, Kg, Vg = _group(q[0], sc.K[0], sc.V[0], 1, G)
        ro, rl = OA.draft_full(qg, Kg, Vg, L, 1.0)
        compare(of[0, G:2 * G], lf[0, G:2 * G], ro, rl, f"full 1M step {j}")
        ro, rl = OA.draft_window(qg, Kg, Vg, L, cfg["n_sink"], cfg["n_recent"], 1.0)
        compare(ow[0, G:2 * G], lw[0, G:2 * G], ro, rl, f"window 1M step {j}")
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
