"""Decode-step benchmark of Windowed-MTP draft/verify attention on one MI355X.

One benchmark step is one pass of the whole hot path over the 1M-context
workload (batch 1, 32 query / 2 kv heads, head_dim 256, 64-token pages in a
seeded permutation, draft depth 7, window 4 + 4092, verify of 8 causal queries):

  windowed arm   7 x (windowed draft step: the window over the ring plus the new
                 position in one launch, then the merge and the ring append in a second)
  native arm     7 x (paged append + full draft attention split pass + combine)
  verify         paged append of the 8 proposed positions + verify attention

Each step appends to both arms, so the context grows by 7 draft positions (and
the target by 8) per step, as in a decode loop that accepts every draft.  All
inputs are generated and uploaded before the timed region.  HIP events on the
launch stream time every phase; every figure is reported as the median with the
10th and 90th percentiles over the timed steps.  The per-step cost of each arm is
assembled two ways: ``decode_step_us`` = verify + the arm's draft steps (append +
attention), the step sum of the scope, and ``decode_step_eq1_us`` adds the draft
context pass (the accepted positions' pass through the draft head), the full
per-step cost identity.

Also timed beside them: the windowed arm as ring append + windowed attention
(three launches per draft step), the windowed draft step with L2/MALL flushed
before every step (cold) against back-to-back steps (warm), the windowed draft
through a truncated index of the paged draft KV, the draft context pass (fused
with its append, and as append then attention), the verify of a tree of
proposals, the native arm over fp8 draft KV and the verify over fp8 target KV.
Then the other workloads (8K,
128K, the ragged batch of 8 and the 8-layer stack) run the same arms at their own
shapes with K/V generated on the device, and the float64 oracle is timed on the
host for one native draft step, one windowed draft step and one verify of the 1M
workload.

Prints one JSON line.  ``value`` is the windowed arm's decode-step time (us).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "draft-attn µs/step + decode-step µs at 1M ctx (full vs window); HBM GB/s"
HBM_PEAK_GBS = 8000.0
WORKLOAD = "ctx1m_g32x2_d256"
W_CONFIG_NAMES = ("ctx8k_g16x2_d128", "ctx128k_g32x4_d128", "ctx1m_g32x2_d256",
                  "ragged8_256k_1m_g32x4_d128", "nope8l_1m_g64x2_d128")

# HBM bytes per launch of the native draft split pass measured with rocprofv3
# (FETCH_SIZE and WRITE_SIZE passes, each scaled by the same counter's reading of a
# plain 1 GiB device copy; summary in profiles/decode_step_ctx1m_g32x2_d256.md),
# keyed by a hash of the sources that kernel is built from: a changed kernel
# reports null until it is measured again.
MEASURED_TRAFFIC = {
    "0721af1bb0ea6695": {"read": 2.148e+09, "write": 4.211e+06, "keys": 1048587},
}
KERNEL_SOURCES = ("csrc/attn.hip", "csrc/attn_device.h", "csrc/common.h")


def log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def stats(xs) -> dict:
    """Median and the 10th / 90th percentiles (us) of a list of timings."""
    a = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(a)), 2), "p10": round(float(np.percentile(a, 10)), 2),
            "p90": round(float(np.percentile(a, 90)), 2)}


def oracle_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        return len(os.sched_getaffinity(0))


def cpu_baseline(Kd, Vd, Kt, Vt, q_draft, q_verify, S, n_q, n_sink, n_recent, gamma):
    """The float64 oracle, as it is, on one unit of each kind of the 1M workload:
    the native draft attention of the first draft step (S + 1 keys, every kv head),
    the windowed draft attention of the same step, and the verify of the first
    decode step (n_q causal queries over S + n_q target keys).  Returns seconds per
    unit and the threads the oracle's BLAS used."""
    from oracle import attention as OA
    t0 = time.perf_counter()
    OA.draft_full(q_draft, Kd, Vd, S + 1, 1.0)
    t1 = time.perf_counter()
    OA.draft_window(q_draft, Kd, Vd, S + 1, n_sink, n_recent, 1.0)
    t2 = time.perf_counter()
    OA.verify(q_verify, Kt, Vt, S + n_q, 1.0)
    t3 = time.perf_counter()
    return {"native_draft_step": t1 - t0, "window_draft_step": t2 - t1, "verify": t3 - t2}, \
        oracle_threads()


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    base = os.path.join(ROOT, "long_context_decode_attention_amd")
    for f in KERNEL_SOURCES:
        with open(os.path.join(base, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


SWEEP_CONTEXTS = (8192, 32768, 131072, 524288, 1048576)


def _fit(xs, ys):
    """Least-squares line y = a + b x: (a, b, R^2)."""
    x = np.asarray(xs, dtype=np.float64)
    y = np.asarray(ys, dtype=np.float64)
    b, a = np.polyfit(x, y, 1)
    r = y - (a + b * x)
    tot = float(np.sum((y - y.mean()) ** 2))
    r2 = 1.0 - float(np.sum(r * r)) / tot if tot > 0 else 1.0
    return float(a), float(b), r2


def run_sweep(args) -> int:
    """Decode-step time against context on the 1M workload's heads (32/2, head_dim 256,
    draft depth 7, window 4 + 4092, verify of 8 queries): at each context the native
    draft step (paged append + split pass + combine), the fused windowed draft step and
    the verify (target append + verify), then a straight-line fit of each against the
    context: the analogue of the pages' time-against-context fit.  K/V are random bf16
    generated on the device; one cache of the largest context serves every point (each
    point reads only its first L positions).  Prints one JSON line."""
    import torch

    import long_context_decode_attention_amd as lib
    import workloads as W
    from long_context_decode_attention_amd import scenario as sc

    dev = "cuda"
    cfg = W.CONFIGS[WORKLOAD]
    Hq, Hkv, D, gamma, n_q = cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["gamma"], cfg["n_q"]
    C, n_sink, n_recent = cfg["C"], cfg["n_sink"], cfg["n_recent"]
    G = Hq // Hkv
    B = 1
    nsteps = args.warmup + args.steps
    Lmax = max(SWEEP_CONTEXTS)
    extra = max(gamma, n_q) * nsteps
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)

    def randn(*shape, scale=1.0):
        x = torch.randn(*shape, device=dev, generator=gen)
        return (x * scale).to(torch.bfloat16)

    npg = (Lmax + extra + 63) // 64
    log("context sweep: filling draft and target KV (1M positions) and the ring")
    dkv = sc.alloc_paged_kv([Lmax + extra], Hkv, D, W.page_permutation(args.seed, "perm", npg), dev)
    tkv = sc.alloc_paged_kv([Lmax + extra], Hkv, D, W.page_permutation(args.seed + 1, "perm", npg),
                            dev)
    ring = lib.new_ring(B, C, Hkv, D, n_sink, n_recent, dev)
    chunk = 1 << 16
    for lo in range(0, Lmax, chunk):
        sp = torch.tensor([lo], dtype=torch.int32, device=dev)
        kn, vn = randn(1, chunk, Hkv, D), randn(1, chunk, Hkv, D)
        lib.paged_append(dkv.k, dkv.v, dkv.block_table, sp, kn, vn)
        lib.ring_append(ring, kn, vn)
        lib.paged_append(tkv.k, tkv.v, tkv.block_table, sp, randn(1, chunk, Hkv, D),
                         randn(1, chunk, Hkv, D))
    torch.cuda.synchronize()
    qs = 1.0 / math.sqrt(D)
    qd = randn(nsteps, gamma, B, Hq, D, scale=qs)
    kd = randn(nsteps, gamma, B, 1, Hkv, D)
    vd = randn(nsteps, gamma, B, 1, Hkv, D)
    qv = randn(nsteps, B, n_q, Hq, D, scale=qs)
    kt = randn(nsteps, B, n_q, Hkv, D)
    vt = randn(nsteps, B, n_q, Hkv, D)
    o_w, l_w = torch.empty(B, Hq, D, device=dev), torch.empty(B, Hq, device=dev)
    o_f, l_f = torch.empty(B, Hq, D, device=dev), torch.empty(B, Hq, device=dev)
    o_v, l_v = torch.empty(B, n_q, Hq, D, device=dev), torch.empty(B, n_q, Hq, device=dev)
    ws_s = lib.new_workspace(lib.step_workspace_bytes(B, Hq, Hkv, D, C), dev)
    ws_f = lib.new_workspace(max(lib.workspace_bytes(B, Hq, Hkv, D, 1, L + extra, partials_only=True)
                                 for L in SWEEP_CONTEXTS), dev)
    ws_v = lib.new_workspace(max(lib.workspace_bytes(B, Hq, Hkv, D, n_q, L + extra)
                                 for L in SWEEP_CONTEXTS), dev)
    stream = torch.cuda.current_stream()
    points = []
    for L in SWEEP_CONTEXTS:
        max_d = L + extra
        po, pl = lib.partials_view(ws_f, B, Hq, Hkv, D, 1, max_d)
        splits = lib.plan_splits(B, Hq, Hkv, D, 1, max_d)
        # positions and lengths live as long as the prepared calls that point at them
        d_pos = torch.tensor([[[L + k * gamma + j] for j in range(gamma)] for k in range(nsteps)],
                             dtype=torch.int32, device=dev)
        d_len = d_pos + 1
        t_pos = torch.tensor([[L + k * n_q] for k in range(nsteps)], dtype=torch.int32, device=dev)
        t_len = t_pos + n_q
        plan = []
        for k in range(nsteps):
            win = [lib.draft_step_window(qd[k, j], ring, kd[k, j], vd[k, j], 1.0, o_w, l_w, ws_s,
                                         prepare=True) for j in range(gamma)]
            full = []
            for j in range(gamma):
                full += [lib.paged_append(dkv.k, dkv.v, dkv.block_table, d_pos[k, j], kd[k, j],
                                          vd[k, j], prepare=True),
                         lib.draft_attn_full(qd[k, j], dkv.k, dkv.v, dkv.block_table, d_len[k, j],
                                             max_d, 1.0, workspace=ws_f, partials_only=True,
                                             prepare=True),
                         lib.split_combine(po, pl, B, Hkv, G, 1, splits_per_group=splits,
                                           o=o_f.view(B, 1, Hq, D), lse=l_f.view(B, 1, Hq),
                                           prepare=True)]
            ver = [lib.paged_append(tkv.k, tkv.v, tkv.block_table, t_pos[k], kt[k], vt[k],
                                    prepare=True),
                   lib.verify_attn(qv[k], tkv.k, tkv.v, tkv.block_table, t_len[k], max_d, 1.0,
                                   o_v, l_v, ws_v, prepare=True)]
            plan.append((win, full, ver))
        times = []
        for k in range(nsteps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            win, full, ver = plan[k]
            e[0].record(stream)
            for c in win:
                c()
            e[1].record(stream)
            for c in full:
                c()
            e[2].record(stream)
            for c in ver:
                c()
            e[3].record(stream)
            times.append(e)
        torch.cuda.synchronize()
        tw = float(np.median([a[0].elapsed_time(a[1]) * 1000.0 / gamma for a in times[args.warmup:]]))
        tf = float(np.median([a[1].elapsed_time(a[2]) * 1000.0 / gamma for a in times[args.warmup:]]))
        tv = float(np.median([a[2].elapsed_time(a[3]) * 1000.0 for a in times[args.warmup:]]))
        points.append({"context": L, "draft_full_us": round(tf, 2), "draft_window_us": round(tw, 2),
                       "verify_us": round(tv, 2), "step_full_us": round(tv + gamma * tf, 2),
                       "step_window_us": round(tv + gamma * tw, 2),
                       "full_over_window": round((tv + gamma * tf) / (tv + gamma * tw), 4)})
        log(f"context {L}: draft full {tf:.1f} us, window {tw:.1f} us, verify {tv:.1f} us")
    xs = [p["context"] / 1e6 for p in points]
    fits = {}
    for key in ("draft_full_us", "draft_window_us", "verify_us", "step_full_us", "step_window_us"):
        a, b, r2 = _fit(xs, [p[key] for p in points])
        fits[key.replace("_us", "")] = {"intercept_us": round(a, 2),
                                        "slope_us_per_million_keys": round(b, 2), "r2": round(r2, 5)}
    ratios = [p["full_over_window"] for p in points]
    out = {
        "metric": "decode-step us against context (1M workload's heads), straight-line fits",
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "data": "synthetic (random N(0,1) bf16 K/V generated on the device, q ~ N(0,1)/sqrt(D))",
        "config": {"workload": f"{WORKLOAD} heads, contexts {list(SWEEP_CONTEXTS)}", "batch": B,
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "draft_depth": gamma,
                   "window": f"{n_sink}+{n_recent}", "verify_queries": n_q},
        "points": points,
        "fits": fits,
        "step_slope_reduction": round(1.0 - fits["step_window"]["slope_us_per_million_keys"] /
                                      fits["step_full"]["slope_us_per_million_keys"], 4),
        "full_over_window_monotone_in_context": all(b >= a for a, b in zip(ratios, ratios[1:])),
    }
    print(json.dumps(out), flush=True)
    return 0


def measure_workload(name: str, steps: int, warmup: int, seed: int, num_splits: int = 0) -> dict:
    """The decode step of one workload: the windowed arm (fused draft steps), the
    native arm (paged append + split pass + combine per draft step) and the verify
    of every attention layer, each sequence at its own length.  K/V and queries are
    random bf16 (N(0, 1), q / sqrt(D)) generated on the device: only the timing is
    taken here, parity at these shapes is the tests' business.  Returns the
    figures as a dict; every device buffer is released on return."""
    import torch

    import long_context_decode_attention_amd as lib
    import workloads as W
    from long_context_decode_attention_amd import scenario as sc

    dev = "cuda"
    cfg = W.CONFIGS[name]
    B, Hq, Hkv, D = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["D"]
    gamma, n_q, layers = cfg["gamma"], cfg["n_q"], cfg["layers"]
    C, n_sink, n_recent = cfg["C"], cfg["n_sink"], cfg["n_recent"]
    G = Hq // Hkv
    S = [int(x) for x in W.context_lengths(cfg, seed)]
    nsteps = warmup + steps
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)

    def randn(*shape, scale=1.0):
        x = torch.randn(*shape, device=dev, generator=gen)
        return (x * scale).to(torch.bfloat16) if scale != 1.0 else x.to(torch.bfloat16)

    def paged_pool(extra):
        cap = [s + extra for s in S]
        n_pages = sum((c + 63) // 64 for c in cap)
        return sc.alloc_paged_kv(cap, Hkv, D, W.page_permutation(seed, "perm", n_pages), dev)

    chunk = 1 << 16
    log(f"{name}: filling draft KV, rings and {layers} target layer(s) (lengths {S})")
    dkv = paged_pool(gamma * nsteps)
    ring_s = lib.new_ring(B, C, Hkv, D, n_sink, n_recent, dev)
    for b in range(B):
        per = C // 64
        sub = lib.Ring(ring_s.k[b * per:(b + 1) * per], ring_s.v[b * per:(b + 1) * per],
                       ring_s.pos[b:b + 1], ring_s.T[b:b + 1], C, n_sink, n_recent)
        for lo in range(0, S[b], chunk):
            n = min(chunk, S[b] - lo)
            kn, vn = randn(1, n, Hkv, D), randn(1, n, Hkv, D)
            sp = torch.tensor([lo], dtype=torch.int32, device=dev)
            lib.paged_append(dkv.k, dkv.v, dkv.block_table[b:b + 1], sp, kn, vn)
            lib.ring_append(sub, kn, vn)
    tkvs = []
    if n_q:
        for _ in range(layers):
            tkv = paged_pool(n_q * nsteps)
            for b in range(B):
                for lo in range(0, S[b], chunk):
                    n = min(chunk, S[b] - lo)
                    sp = torch.tensor([lo], dtype=torch.int32, device=dev)
                    lib.paged_append(tkv.k, tkv.v, tkv.block_table[b:b + 1], sp,
                                     randn(1, n, Hkv, D), randn(1, n, Hkv, D))
            tkvs.append(tkv)
    torch.cuda.synchronize()

    qs = 1.0 / math.sqrt(D)
    qd = randn(nsteps, gamma, B, Hq, D, scale=qs)
    kd = randn(nsteps, gamma, B, 1, Hkv, D)
    vd = randn(nsteps, gamma, B, 1, Hkv, D)
    d_pos = torch.tensor([[[s + k * gamma + j for s in S] for j in range(gamma)]
                          for k in range(nsteps)], dtype=torch.int32, device=dev)
    d_len = d_pos + 1
    max_d = max(S) + gamma * nsteps
    o_w, l_w = torch.empty(B, Hq, D, device=dev), torch.empty(B, Hq, device=dev)
    o_f, l_f = torch.empty(B, Hq, D, device=dev), torch.empty(B, Hq, device=dev)
    ws_s = lib.new_workspace(lib.step_workspace_bytes(B, Hq, Hkv, D, C), dev)
    ns = num_splits
    ws_f = lib.new_workspace(lib.workspace_bytes(B, Hq, Hkv, D, 1, max_d, ns, partials_only=True),
                             dev)
    po, pl = lib.partials_view(ws_f, B, Hq, Hkv, D, 1, max_d, ns)
    splits_f = lib.plan_splits(B, Hq, Hkv, D, 1, max_d, ns)
    if n_q:
        qv = randn(nsteps, layers, B, n_q, Hq, D, scale=qs)
        kt = randn(nsteps, layers, B, n_q, Hkv, D)
        vt = randn(nsteps, layers, B, n_q, Hkv, D)
        t_pos = torch.tensor([[s + k * n_q for s in S] for k in range(nsteps)], dtype=torch.int32,
                             device=dev)
        t_len = t_pos + n_q
        max_t = max(S) + n_q * nsteps
        o_v = torch.empty(B, n_q, Hq, D, device=dev)
        l_v = torch.empty(B, n_q, Hq, device=dev)
        ws_v = lib.new_workspace(lib.workspace_bytes(B, Hq, Hkv, D, n_q, max_t, ns), dev)
    stream = torch.cuda.current_stream()
    plan = []
    for k in range(nsteps):
        win = [lib.draft_step_window(qd[k, j], ring_s, kd[k, j], vd[k, j], 1.0, o_w, l_w, ws_s,
                                     prepare=True) for j in range(gamma)]
        full = [(lib.paged_append(dkv.k, dkv.v, dkv.block_table, d_pos[k, j], kd[k, j], vd[k, j],
                                  prepare=True),
                 lib.draft_attn_full(qd[k, j], dkv.k, dkv.v, dkv.block_table, d_len[k, j], max_d,
                                     1.0, workspace=ws_f, num_splits=ns, partials_only=True,
                                     prepare=True),
                 lib.split_combine(po, pl, B, Hkv, G, 1, splits_per_group=splits_f,
                                   o=o_f.view(B, 1, Hq, D), lse=l_f.view(B, 1, Hq), prepare=True))
                for j in range(gamma)]
        ver = []
        if n_q:
            for li, tkv in enumerate(tkvs):
                ver.append(lib.paged_append(tkv.k, tkv.v, tkv.block_table, t_pos[k], kt[k, li],
                                            vt[k, li], prepare=True))
                ver.append(lib.verify_attn(qv[k, li], tkv.k, tkv.v, tkv.block_table, t_len[k],
                                           max_t, 1.0, o_v, l_v, ws_v, num_splits=ns,
                                           prepare=True))
        plan.append((win, full, ver))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4 + 2 * gamma)]
           for _ in range(nsteps)]

    def step(k):
        win, full, ver = plan[k]
        e = evs[k]
        e[0].record(stream)
        for c in win:
            c()
        e[1].record(stream)
        for j, (app, attn, comb) in enumerate(full):
            app()
            e[4 + 2 * j].record(stream)
            attn()
            e[5 + 2 * j].record(stream)
            comb()
        e[2].record(stream)
        for c in ver:
            c()
        e[3].record(stream)
        return e

    for k in range(warmup):
        step(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks = [step(k) for k in range(warmup, nsteps)]
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    def us(a, b):
        return a.elapsed_time(b) * 1000.0

    win_chain = [us(e[0], e[1]) for e in marks]
    full_chain = [us(e[1], e[2]) for e in marks]
    verify_all = [us(e[2], e[3]) if n_q else 0.0 for e in marks]
    attn = [us(e[4 + 2 * j], e[5 + 2 * j]) for e in marks for j in range(gamma)]
    attn_us = float(np.mean(attn))
    kv_bytes = 2 * Hkv * D * 2
    # mean keys read by a timed draft step, summed over the batch
    keys = sum(S) + B * (gamma * (warmup + nsteps - 1) / 2.0 + (gamma + 1) / 2.0)
    attn_bytes = kv_bytes * keys + B * Hq * D * 2
    achieved = attn_bytes / (attn_us * 1e-6) / 1e9
    step_window = [v + w for v, w in zip(verify_all, win_chain)]
    step_full = [v + f for v, f in zip(verify_all, full_chain)]
    sw, sf = float(np.median(step_window)), float(np.median(step_full))
    res = {
        "config": {"workload": name, "batch": B, "context": S, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": D, "page_tokens": 64, "pages": "seeded permutation",
                   "draft_depth": gamma, "window": f"{n_sink}+{n_recent}", "ring_slots": C,
                   "verify_queries": n_q, "attention_layers": layers,
                   "splits_per_kv_head": {"draft": splits_f}},
        "steps": steps, "warmup": warmup, "ms_per_step": round(wall / steps * 1000.0, 4),
        "draft_attn_us_per_step": {"full": stats([x / gamma for x in full_chain]),
                                   "window": stats([x / gamma for x in win_chain]),
                                   "full_attention_kernel": stats(attn)},
        "decode_step_us": {"full": stats(step_full), "window": stats(step_window),
                           "verify_all_layers": stats(verify_all)},
        "cost_reduction": {"native_over_window_minus_1": round(sf / sw - 1.0, 4),
                           "one_minus_window_over_native": round(1.0 - sw / sf, 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "kernel": "attn_split_kernel (native draft, split pass)",
                     "bytes_per_launch": int(attn_bytes)},
    }
    if n_q:
        v_keys = sum(S) + B * n_q * (warmup + nsteps) / 2.0
        v_bytes = layers * (kv_bytes * v_keys + B * n_q * Hq * (D * 2 + D * 4 + 4))
        vg = v_bytes / (float(np.median(verify_all)) * 1e-6) / 1e9
        res["roofline_verify"] = {"bound": "hbm", "achieved": round(vg, 1), "peak": HBM_PEAK_GBS,
                                  "unit": "GB/s", "frac": round(vg / HBM_PEAK_GBS, 4),
                                  "note": "verify of every layer with its target append"}
    if layers > 1:
        # draft KV a native draft keeps (every position) against what the ring keeps,
        # over all the KV of the stack: the share the ring gives back
        t_d = sum(S)
        draft_bytes = kv_bytes * t_d
        ring_bytes = kv_bytes * B * C
        target_bytes = layers * kv_bytes * sum(S)
        res["draft_kv_reclaimed_fraction"] = round((draft_bytes - ring_bytes) /
                                                   (target_bytes + draft_bytes), 5)
    return res


def run_workload(args) -> int:
    """One other workload on its own: prints its JSON line (no CPU baseline)."""
    import torch  # noqa: F401  (initialises the device before the library is used)

    import long_context_decode_attention_amd as lib
    lib.load()
    res = measure_workload(args.workload, args.steps, args.warmup, args.seed, args.num_splits)
    sw = res["decode_step_us"]["window"]["median"]
    out = {
        "metric": METRIC, "value": sw, "unit": "us/step", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": res.pop("ms_per_step"), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (random N(0,1) bf16 K/V generated on the device, q ~ N(0,1)/sqrt(D))",
    }
    res.pop("steps"), res.pop("warmup")
    out.update(res)
    print(json.dumps(out), flush=True)
    return 0


def measure_main(args):
    """The 1M workload: every phase of the decode step; returns the JSON fields and
    the host arrays the CPU baseline needs (device buffers are released on return)."""
    import torch

    import long_context_decode_attention_amd as lib
    import workloads as W
    from long_context_decode_attention_amd import scenario as sc

    lib.load()
    dev = "cuda"
    cfg = W.CONFIGS[WORKLOAD]
    B, Hq, Hkv, D = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["D"]
    S, gamma, n_q = cfg["S"], cfg["gamma"], cfg["n_q"]
    C, n_sink, n_recent = cfg["C"], cfg["n_sink"], cfg["n_recent"]
    G = Hq // Hkv
    nsteps = args.warmup + args.steps
    seed = args.seed

    # ---------------------------------------------------------------- setup (untimed)
    log("generating inputs")
    d_extra = gamma * nsteps
    t_extra = n_q * nsteps
    Kd = W.kv_positions(seed, "draft_k", 0, 0, S + d_extra, Hkv, D)
    Vd = W.kv_positions(seed, "draft_v", 0, 0, S + d_extra, Hkv, D)
    Kt = W.kv_positions(seed, "target_k", 0, 0, S + t_extra, Hkv, D)
    Vt = W.kv_positions(seed, "target_v", 0, 0, S + t_extra, Hkv, D)
    log("filling caches and ring")
    npd = (S + d_extra + 63) // 64
    npt = (S + t_extra + 63) // 64
    dkv = sc.alloc_paged_kv([S + d_extra], Hkv, D, W.page_permutation(seed, "draft_k", npd), dev)
    tkv = sc.alloc_paged_kv([S + t_extra], Hkv, D, W.page_permutation(seed, "target_k", npt), dev)
    ring = lib.new_ring(B, C, Hkv, D, n_sink, n_recent, dev)
    ring_s = lib.new_ring(B, C, Hkv, D, n_sink, n_recent, dev)   # the windowed arm's ring
    ring_g = lib.new_ring(B, C, Hkv, D, n_sink, n_recent, dev)   # the same, replayed from graphs
    ring_k = lib.new_ring(B, C, Hkv, D, n_sink, n_recent, dev)   # the same, timed cold
    # the draft context pass over a ring needs slack for its earlier queries'
    # windows (n_q - 1 positions): a second ring with 64 more slots
    n_ctx = gamma + 1
    ring_c = lib.new_ring(B, C + 64, Hkv, D, n_sink, n_recent, dev)
    ring_cf = lib.new_ring(B, C + 64, Hkv, D, n_sink, n_recent, dev)   # the same, fused pass
    sc.fill_paged(dkv, 0, 0, Kd[:S], Vd[:S])
    sc.fill_paged(tkv, 0, 0, Kt[:S], Vt[:S])
    sc.fill_ring(ring, 0, Kd[:S], Vd[:S])
    sc.fill_ring(ring_s, 0, Kd[:S], Vd[:S])
    sc.fill_ring(ring_g, 0, Kd[:S], Vd[:S])
    sc.fill_ring(ring_k, 0, Kd[:S], Vd[:S])
    sc.fill_ring(ring_c, 0, Kd[:S], Vd[:S])
    sc.fill_ring(ring_cf, 0, Kd[:S], Vd[:S])
    # the same draft KV as fp8 e4m3 codes (scales 1: N(0, 1) values fit), same pages
    k8, v8 = lib.new_paged_cache_fp8(dkv.num_pages, Hkv, D, dev)
    for lo in range(0, S, 1 << 16):
        hi = min(S, lo + (1 << 16))
        lib.paged_append_fp8(k8, v8, dkv.block_table, torch.tensor([lo], dtype=torch.int32, device=dev),
                             sc.to_device_bf16(Kd[lo:hi]).unsqueeze(0),
                             sc.to_device_bf16(Vd[lo:hi]).unsqueeze(0))
    # the target KV as fp8 codes too, on the target's pages: the verify over fp8 KV
    kt8, vt8 = lib.new_paged_cache_fp8(tkv.num_pages, Hkv, D, dev)
    for lo in range(0, S, 1 << 16):
        hi = min(S, lo + (1 << 16))
        lib.paged_append_fp8(kt8, vt8, tkv.block_table, torch.tensor([lo], dtype=torch.int32, device=dev),
                             sc.to_device_bf16(Kt[lo:hi]).unsqueeze(0),
                             sc.to_device_bf16(Vt[lo:hi]).unsqueeze(0))
    # per-step inputs, resident on the device
    kd_new = sc.to_device_bf16(Kd[S:S + d_extra]).view(nsteps, gamma, 1, 1, Hkv, D)
    vd_new = sc.to_device_bf16(Vd[S:S + d_extra]).view(nsteps, gamma, 1, 1, Hkv, D)
    kt_new = sc.to_device_bf16(Kt[S:S + t_extra]).view(nsteps, 1, n_q, Hkv, D)
    vt_new = sc.to_device_bf16(Vt[S:S + t_extra]).view(nsteps, 1, n_q, Hkv, D)
    qd_host = np.stack([W.queries(seed, "q_draft", (B, Hq), D, step=k * gamma + j)
                        for k in range(nsteps) for j in range(gamma)])
    qd = sc.to_device_bf16(qd_host).view(nsteps, gamma, B, Hq, D)
    qv = sc.to_device_bf16(np.stack([W.queries(seed, "q_verify", (B, n_q, Hq), D, step=k)
                                     for k in range(nsteps)])).view(nsteps, B, n_q, Hq, D)
    qc = sc.to_device_bf16(np.stack([W.queries(seed, "q_ctx", (B, n_ctx, Hq), D, step=k)
                                     for k in range(nsteps)])).view(nsteps, B, n_ctx, Hq, D)
    # K/V the context pass appends to its ring: the step's drafts and one more
    # position (the bonus one; its values repeat the last draft's)
    kc_new = torch.cat([kd_new.view(nsteps, gamma, Hkv, D), kd_new.view(nsteps, gamma, Hkv, D)[:, -1:]],
                       1).view(nsteps, 1, n_ctx, Hkv, D).contiguous()
    vc_new = torch.cat([vd_new.view(nsteps, gamma, Hkv, D), vd_new.view(nsteps, gamma, Hkv, D)[:, -1:]],
                       1).view(nsteps, 1, n_ctx, Hkv, D).contiguous()
    # draft step j of bench step k appends position S + k*gamma + j - 1 and reads S + k*gamma + j keys
    d_pos = torch.tensor([[S + k * gamma + j for j in range(gamma)] for k in range(nsteps)],
                         dtype=torch.int32, device=dev).view(nsteps, gamma, 1)
    d_len = d_pos + 1
    t_pos = torch.tensor([S + k * n_q for k in range(nsteps)], dtype=torch.int32,
                         device=dev).view(nsteps, 1)
    t_len = t_pos + n_q
    max_d = S + d_extra
    max_t = S + t_extra
    # outputs and workspaces
    o_w = torch.empty(B, Hq, D, device=dev)
    l_w = torch.empty(B, Hq, device=dev)
    o_f = torch.empty(B, Hq, D, device=dev)
    l_f = torch.empty(B, Hq, device=dev)
    o_v = torch.empty(B, n_q, Hq, D, device=dev)
    l_v = torch.empty(B, n_q, Hq, device=dev)
    o_p = torch.empty(B, Hq, D, device=dev)
    l_p = torch.empty(B, Hq, device=dev)
    ws_w = lib.new_workspace(lib.workspace_bytes(B, Hq, Hkv, D, 1, C, ring=True), dev)
    ws_s = lib.new_workspace(lib.step_workspace_bytes(B, Hq, Hkv, D, C), dev)
    o_s = torch.empty(B, Hq, D, device=dev)
    l_s = torch.empty(B, Hq, device=dev)
    ws_p = lib.new_workspace(lib.workspace_bytes(B, Hq, Hkv, D, 1, n_sink + n_recent,
                                                 paged_window=True), dev)
    ws_f = lib.new_workspace(lib.workspace_bytes(B, Hq, Hkv, D, 1, max_d, args.num_splits,
                                                 partials_only=True), dev)
    ws_8 = lib.new_workspace(lib.workspace_bytes(B, Hq, Hkv, D, 1, max_d, args.num_splits,
                                                 partials_only=True, fp8=True), dev)
    splits_8 = lib.plan_splits(B, Hq, Hkv, D, 1, max_d, args.num_splits, fp8=True)
    o_8 = torch.empty(B, Hq, D, device=dev)
    l_8 = torch.empty(B, Hq, device=dev)
    ws_v = lib.new_workspace(lib.workspace_bytes(B, Hq, Hkv, D, n_q, max_t), dev)
    ws_v8 = lib.new_workspace(lib.workspace_bytes(B, Hq, Hkv, D, n_q, max_t, fp8=True), dev)
    o_v8 = torch.empty(B, n_q, Hq, D, device=dev)
    l_v8 = torch.empty(B, n_q, Hq, device=dev)
    o_c = torch.empty(B, n_ctx, Hq, D, device=dev)
    l_c = torch.empty(B, n_ctx, Hq, device=dev)
    ws_cw = lib.new_workspace(lib.workspace_bytes(B, Hq, Hkv, D, n_ctx, C + 64, ring=True), dev)
    ws_cf = lib.new_workspace(lib.step_workspace_bytes(B, Hq, Hkv, D, C + 64, 0, n_ctx), dev)
    ws_cn = lib.new_workspace(lib.workspace_bytes(B, Hq, Hkv, D, n_ctx, max_d), dev)
    # tree-shaped proposals of the same size for the tree verify: a binary tree
    # (node i's parent (i - 1) // 2), mask bit a = node a is an ancestor or itself
    tree = []
    for i in range(n_q):
        mk, j = 0, i
        while True:
            mk |= 1 << j
            if j == 0:
                break
            j = (j - 1) // 2
        tree.append(mk)
    tree_mask = torch.tensor([tree] * B, dtype=torch.int64, device=dev)
    po, pl = lib.partials_view(ws_f, B, Hq, Hkv, D, 1, max_d, args.num_splits)
    splits_f = lib.plan_splits(B, Hq, Hkv, D, 1, max_d, args.num_splits)
    stream = torch.cuda.current_stream()

    marks = []   # per step: dict of events

    # Marshal every launch of every step before the timed region.
    plan = []
    for k in range(nsteps):
        win = []
        for j in range(gamma):
            win.append(lib.ring_append(ring, kd_new[k, j], vd_new[k, j], prepare=True))
            win.append(lib.draft_attn_window(qd[k, j], ring, 1.0, o_w, l_w, ws_w, prepare=True))
        # the windowed arm's draft steps: window attention over the ring plus the
        # new position in one launch, the merge and the ring append in a second
        fused = [lib.draft_step_window(qd[k, j], ring_s, kd_new[k, j], vd_new[k, j], 1.0, o_s, l_s,
                                       ws_s, prepare=True) for j in range(gamma)]
        full = []
        for j in range(gamma):
            full.append((
                lib.paged_append(dkv.k, dkv.v, dkv.block_table, d_pos[k, j], kd_new[k, j],
                                 vd_new[k, j], prepare=True),
                lib.draft_attn_full(qd[k, j], dkv.k, dkv.v, dkv.block_table, d_len[k, j], max_d,
                                    1.0, workspace=ws_f, num_splits=args.num_splits,
                                    partials_only=True, prepare=True),
                lib.split_combine(po, pl, B, Hkv, G, 1, splits_per_group=splits_f,
                                  o=o_f.view(B, 1, Hq, D), lse=l_f.view(B, 1, Hq), prepare=True)))
        # the pages' own windowed draft: the draft KV stays in the paged cache and the
        # attention reads a truncated index (the appends rewrite the positions the
        # native arm has just written, with the same values)
        wpg = []
        for j in range(gamma):
            wpg.append(lib.paged_append(dkv.k, dkv.v, dkv.block_table, d_pos[k, j], kd_new[k, j],
                                        vd_new[k, j], prepare=True))
            wpg.append(lib.draft_attn_window_paged(qd[k, j], dkv.k, dkv.v, dkv.block_table,
                                                   d_len[k, j], max_d, n_sink, n_recent, 1.0,
                                                   o_p, l_p, ws_p, prepare=True))
        ver = (lib.paged_append(tkv.k, tkv.v, tkv.block_table, t_pos[k], kt_new[k], vt_new[k],
                                prepare=True),
               lib.verify_attn(qv[k], tkv.k, tkv.v, tkv.block_table, t_len[k], max_t, 1.0, o_v,
                               l_v, ws_v, prepare=True))
        # draft context pass over the n_ctx accepted positions (here: every draft
        # plus the bonus position): windowed over the slack ring (append, then
        # attention; and the two fused in ctx[4]), natively the causal verify
        # kernel over the whole paged draft KV
        ctx = (lib.ring_append(ring_c, kc_new[k], vc_new[k], prepare=True),
               lib.draft_context_window(qc[k], ring_c, 1.0, o_c, l_c, ws_cw, prepare=True),
               lib.verify_attn(qc[k], dkv.k, dkv.v, dkv.block_table, d_len[k, gamma - 1], max_d,
                               1.0, o_c, l_c, ws_cn, prepare=True),
               lib.verify_attn_tree(qv[k], tkv.k, tkv.v, tkv.block_table, t_len[k], tree_mask,
                                    max_t, 1.0, o_v, l_v, ws_v, prepare=True),
               lib.draft_context_step_window(qc[k], ring_cf, kc_new[k], vc_new[k], 1.0, o_c, l_c,
                                             ws_cf, prepare=True))
        # native arm over the fp8 draft KV: quantizing append, split pass, combine
        full8 = []
        for j in range(gamma):
            full8.append((
                lib.paged_append_fp8(k8, v8, dkv.block_table, d_pos[k, j], kd_new[k, j],
                                     vd_new[k, j], prepare=True),
                lib.draft_attn_full_fp8(qd[k, j], k8, v8, dkv.block_table, d_len[k, j], max_d,
                                        workspace=ws_8, num_splits=args.num_splits,
                                        partials_only=True, prepare=True),
                lib.split_combine(*lib.partials_view(ws_8, B, Hq, Hkv, D, 1, max_d, args.num_splits,
                                                     fp8=True),
                                  B, Hkv, G, 1, splits_per_group=splits_8,
                                  o=o_8.view(B, 1, Hq, D), lse=l_8.view(B, 1, Hq), prepare=True)))
        # the verify over the fp8 target KV: quantizing append of the proposed
        # positions, then the verify (same queries, same outputs' shapes)
        ver8 = (lib.paged_append_fp8(kt8, vt8, tkv.block_table, t_pos[k], kt_new[k], vt_new[k],
                                     prepare=True),
                lib.verify_attn_fp8(qv[k], kt8, vt8, tkv.block_table, t_len[k], max_t, 1.0, 1.0,
                                    1.0, o_v8, l_v8, ws_v8, prepare=True))
        plan.append((win, full, wpg, ver, ctx, full8, fused, ver8))
    # The windowed arm's draft steps once more, each bench step's seven recorded in a
    # HIP graph (14 launches) and replayed: the launches without per-call host work.
    ws_g = lib.new_workspace(lib.step_workspace_bytes(B, Hq, Hkv, D, C), dev)
    o_g = torch.empty(B, Hq, D, device=dev)
    l_g = torch.empty(B, Hq, device=dev)
    graphs = []
    torch.cuda.synchronize()
    for k in range(nsteps):
        gk = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gk):
            for j in range(gamma):
                lib.draft_step_window(qd[k, j], ring_g, kd_new[k, j], vd_new[k, j], 1.0, o_g, l_g,
                                      ws_g)
        graphs.append(gk)
    torch.cuda.synchronize()
    # The windowed draft steps once more on their own ring, each timed alone after a
    # 1 GiB write that flushes the caches (L2 and MALL: the 8 MiB window would
    # otherwise stay cached between back-to-back steps); the flush is outside the
    # timed region.
    ws_k = lib.new_workspace(lib.step_workspace_bytes(B, Hq, Hkv, D, C), dev)
    o_k = torch.empty(B, Hq, D, device=dev)
    l_k = torch.empty(B, Hq, device=dev)
    cold = [[lib.draft_step_window(qd[k, j], ring_k, kd_new[k, j], vd_new[k, j], 1.0, o_k, l_k,
                                   ws_k, prepare=True) for j in range(gamma)] for k in range(nsteps)]
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(17 + 4 * gamma)]
           for _ in range(nsteps)]
    evc = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(gamma)] for _ in range(nsteps)]

    def cold_steps(k):
        for j in range(gamma):
            flush.fill_(k & 0xFF)
            evc[k][j][0].record(stream)
            cold[k][j]()
            evc[k][j][1].record(stream)

    def step(k):
        win, full, wpg, ver, ctx, full8, fused, ver8 = plan[k]
        e = evs[k]
        e[11 + 4 * gamma].record(stream)
        for c in fused:                     # windowed arm: gamma x fused draft step
            c()
        e[12 + 4 * gamma].record(stream)
        graphs[k].replay()                  # the same steps replayed from a graph
        e[14 + 4 * gamma].record(stream)
        e[0].record(stream)
        for c in win:                       # the same as ring append + window attention
            c()
        e[1].record(stream)
        for j, (app, attn, comb) in enumerate(full):   # native arm
            app()
            e[5 + 2 * j].record(stream)
            attn()
            e[6 + 2 * j].record(stream)
            comb()
        e[2].record(stream)
        for c in wpg:                       # windowed arm by index truncation (no ring)
            c()
        e[5 + 2 * gamma].record(stream)
        ver[0]()                            # target append of the proposed positions
        e[3].record(stream)
        ver[1]()                            # verify attention
        e[4].record(stream)
        ctx[4]()                            # context pass, windowed: fused append + attention
        e[13 + 4 * gamma].record(stream)
        ctx[0]()                            # the same as ring append + ring attention
        ctx[1]()
        e[6 + 2 * gamma].record(stream)
        ctx[2]()                            # context pass, native: over all the draft KV
        e[7 + 2 * gamma].record(stream)
        ctx[3]()                            # the verify for a tree of proposals
        e[8 + 2 * gamma].record(stream)
        for j, (app, attn, comb) in enumerate(full8):  # native arm, fp8 draft KV
            app()
            e[10 + 2 * gamma + 2 * j].record(stream)
            attn()
            e[11 + 2 * gamma + 2 * j].record(stream)
            comb()
        e[9 + 2 * gamma].record(stream)
        ver8[0]()                           # fp8 target append of the proposed positions
        e[15 + 4 * gamma].record(stream)
        ver8[1]()                           # verify over the fp8 target KV
        e[16 + 4 * gamma].record(stream)
        return {"s0": e[11 + 4 * gamma], "s1": e[12 + 4 * gamma], "g1": e[14 + 4 * gamma],
                "t0": e[0], "t1": e[1], "t2": e[2], "p1": e[5 + 2 * gamma], "v0": e[3],
                "t3": e[4], "cf": e[13 + 4 * gamma], "c1": e[6 + 2 * gamma],
                "c2": e[7 + 2 * gamma], "c3": e[8 + 2 * gamma], "f8": e[9 + 2 * gamma],
                "v8a": e[15 + 4 * gamma], "v8": e[16 + 4 * gamma],
                "attn8": [(e[10 + 2 * gamma + 2 * j], e[11 + 2 * gamma + 2 * j]) for j in range(gamma)],
                "attn": [(e[5 + 2 * j], e[6 + 2 * j]) for j in range(gamma)]}

    if args.copy_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log("warmup")
    for k in range(args.warmup):
        step(k)
        cold_steps(k)
    torch.cuda.synchronize()
    log("timed steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.warmup, nsteps):
        marks.append(step(k))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log("cold windowed draft steps")
    for k in range(args.warmup, nsteps):
        cold_steps(k)
    torch.cuda.synchronize()

    def us(a, b):
        return a.elapsed_time(b) * 1000.0

    def per(key0, key1, div=1.0):
        return [us(m[key0], m[key1]) / div for m in marks]

    win3 = per("t0", "t1")                       # append, then window
    win = per("s0", "s1")                        # the fused step
    graph = per("s1", "g1")                      # the same, from graphs
    full = per("t1", "t2")
    wpg = per("t2", "p1")
    ctx_w = per("t3", "cf")                      # draft context pass, fused
    ctx_w3 = per("cf", "c1")                     # append, then window
    ctx_f = per("c1", "c2")
    tree = per("c2", "c3")
    full8 = per("c3", "f8")
    verify = per("p1", "t3")
    verify_k = per("v0", "t3")
    verify8 = per("f8", "v8")                    # fp8 append + verify over fp8 target KV
    verify8_k = per("v8a", "v8")
    attn8 = [us(a, b) for m in marks for (a, b) in m["attn8"]]
    attn = [us(a, b) for m in marks for (a, b) in m["attn"]]
    cold_step = [us(a, b) for k in range(args.warmup, nsteps) for (a, b) in evc[k]]
    attn_mean = float(np.mean(attn))
    attn8_mean = float(np.mean(attn8))
    step_window = [v + w for v, w in zip(verify, win)]
    step_full = [v + f for v, f in zip(verify, full)]
    step_window_eq1 = [s_ + c for s_, c in zip(step_window, ctx_w)]
    step_full_eq1 = [s_ + c for s_, c in zip(step_full, ctx_f)]
    md = lambda xs: float(np.median(xs))  # noqa: E731
    sw, sf = md(step_window), md(step_full)
    sw1, sf1 = md(step_window_eq1), md(step_full_eq1)
    # mean keys read by the timed draft steps (step k, draft j reads S + k*gamma + j keys)
    L_avg = S + gamma * (args.warmup + nsteps - 1) / 2.0 + (gamma + 1) / 2.0
    kv_bytes = 2 * Hkv * D * 2                             # K + V bytes per position
    attn8_bytes = kv_bytes / 2 * L_avg + B * Hq * D * 2    # fp8 K + V of the keys + q
    attn_bytes = kv_bytes * L_avg + B * Hq * D * 2         # keys' K/V + q (algorithmic)
    verify_bytes = kv_bytes * (S + n_q * (args.warmup + nsteps) / 2.0) + B * n_q * Hq * (D * 2 + D * 4 + 4)
    verify8_bytes = kv_bytes / 2 * (S + n_q * (args.warmup + nsteps) / 2.0) + B * n_q * Hq * (D * 2 + D * 4 + 4)
    win_bytes = kv_bytes * (n_sink + n_recent) + B * Hq * D * 2
    achieved = attn_bytes / (attn_mean * 1e-6) / 1e9
    verify_gbs = verify_bytes / (md(verify_k) * 1e-6) / 1e9
    rec = MEASURED_TRAFFIC.get(kernel_source_hash())
    traffic = None
    if rec is not None:
        # bytes per launch at the measured key count, rescaled to this run's mean keys
        scale = L_avg / rec["keys"]
        traffic = int(rec["read"] * scale + rec["write"])

    def per_step(xs):
        return stats([x / gamma for x in xs])

    out = {
        "metric": METRIC,
        "value": round(sw, 2),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1000.0, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 K/V, q ~ N(0,1)/sqrt(D))",
        "config": {"workload": WORKLOAD, "batch": B, "context": S, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": D, "page_tokens": 64, "pages": "seeded permutation",
                   "draft_depth": gamma, "window": f"{n_sink}+{n_recent}", "ring_slots": C,
                   "verify_queries": n_q},
        "value_definition": "windowed decode step = verify (target append + verify attention) + "
                            "the 7 fused windowed draft steps; median over the timed steps",
        "draft_attn_us_per_step": {"full": per_step(full),
                                   "full_fp8_kv": per_step(full8),
                                   "full_fp8_kv_attention_kernel": stats(attn8),
                                   "window": per_step(win),
                                   "window_cold": stats(cold_step),
                                   "window_append_then_attend": per_step(win3),
                                   "window_graph_replay": per_step(graph),
                                   "window_paged_index": per_step(wpg),
                                   "full_attention_kernel": stats(attn)},
        "decode_step_us": {"full": stats(step_full), "window": stats(step_window),
                           "full_fp8_kv": stats([v + f for v, f in zip(verify, full8)]),
                           "window_paged_index": stats([v + w for v, w in zip(verify, wpg)]),
                           "window_append_then_attend": stats([v + w for v, w in zip(verify, win3)]),
                           "verify": stats(verify),
                           "verify_kernel": stats(verify_k),
                           "verify_tree_kernel": stats(tree),
                           "verify_fp8_kv": stats(verify8),
                           "verify_fp8_kv_kernel": stats(verify8_k)},
        "cost_reduction": {"native_over_window_minus_1": round(sf / sw - 1.0, 4),
                           "one_minus_window_over_native": round(1.0 - sw / sf, 4)},
        "draft_context_pass_us": {"queries": n_ctx, "window": stats(ctx_w),
                                  "window_append_then_attend": stats(ctx_w3),
                                  "full": stats(ctx_f)},
        "decode_step_eq1_us": {"window": stats(step_window_eq1), "full": stats(step_full_eq1),
                               "definition": "verify + draft context pass (8 accepted positions) "
                                             "+ the 7 draft steps"},
        "cost_reduction_eq1": {"native_over_window_minus_1": round(sf1 / sw1 - 1.0, 4),
                               "one_minus_window_over_native": round(1.0 - sw1 / sf1, 4)},
        "hbm_gbs": {"full_draft_attention": round(achieved, 1), "verify": round(verify_gbs, 1)},
        "effective_gbs": {
            "window_draft_step_warm": round(win_bytes / (md(win) / gamma * 1e-6) / 1e9, 1),
            "window_draft_step_cold": round(win_bytes / (md(cold_step) * 1e-6) / 1e9, 1),
            "note": "window bytes over the whole fused step (two launches); warm steps run "
                    "back to back, so the 8 MiB window may be served from L2/MALL; cold steps "
                    "follow a 1 GiB cache flush"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "attn_split_kernel<256,1,false> (native draft, split pass)",
                     "bytes_per_launch": int(attn_bytes)},
        "roofline_verify": {"bound": "hbm", "achieved": round(verify_gbs, 1), "peak": HBM_PEAK_GBS,
                            "unit": "GB/s", "frac": round(verify_gbs / HBM_PEAK_GBS, 4),
                            "bytes_per_launch": int(verify_bytes)},
        "roofline_verify_fp8_kv": {
            "bound": "hbm", "achieved": round(verify8_bytes / (md(verify8_k) * 1e-6) / 1e9, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(verify8_bytes / (md(verify8_k) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes_per_launch": int(verify8_bytes)},
        "roofline_full_fp8_kv": {
            "bound": "hbm", "achieved": round(attn8_bytes / (attn8_mean * 1e-6) / 1e9, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(attn8_bytes / (attn8_mean * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes_per_launch": int(attn8_bytes)},
    }
    host = {"Kd": Kd, "Vd": Vd, "Kt": Kt, "Vt": Vt, "q_draft": qd_host[0][0],
            "q_verify": W.queries(seed, "q_verify", (B, n_q, Hq), D, step=0)[0],
            "S": S, "n_q": n_q, "n_sink": n_sink, "n_recent": n_recent, "gamma": gamma}
    return out, host


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=2026)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--main-only", action="store_true",
                    help="time the 1M workload only (skip the other workloads)")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--workload", default=WORKLOAD, choices=sorted(W_CONFIG_NAMES),
                    help="the workload to time; the default is the 1M-context single "
                         "sequence, the others time the same arms at their own shapes "
                         "with random bf16 inputs generated on the device")
    ap.add_argument("--context-sweep", action="store_true",
                    help="time the native and windowed draft steps and the verify at "
                         "contexts 8K..1M (the 1M workload's heads) and fit time against "
                         "context; prints its own JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one plain 1 GiB device copy before the steps, so that a profiler "
                         "pass sees a kernel of known traffic to scale its byte counters by")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this path is built and measured for a single "
              "MI355X (multi-GPU sharding is designed, not built); run with --gpus 1",
              file=sys.stderr)
        return 2

    import torch

    import long_context_decode_attention_amd as lib

    if args.context_sweep:
        return run_sweep(args)
    if args.workload != WORKLOAD:
        return run_workload(args)

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    lib.load()
    out, host = measure_main(args)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.main_only:
        # the other workloads, each with K/V generated on the device
        out["workloads"] = {}
        w_steps, w_warm = min(args.steps, 5), min(args.warmup, 2)
        for name in W_CONFIG_NAMES:
            if name == WORKLOAD:
                continue
            res = measure_workload(name, w_steps, w_warm, args.seed, args.num_splits)
            out["workloads"][name] = res
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            log(f"{name}: decode step window {res['decode_step_us']['window']['median']} us, "
                f"native {res['decode_step_us']['full']['median']} us")
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle: one native draft step, one windowed draft step, one verify)")
        h = host
        units, threads = cpu_baseline(h["Kd"], h["Vd"], h["Kt"], h["Vt"], h["q_draft"],
                                      h["q_verify"], h["S"], h["n_q"], h["n_sink"], h["n_recent"],
                                      h["gamma"])
        gamma = h["gamma"]
        window_step = units["verify"] + gamma * units["window_draft_step"]
        native_step = units["verify"] + gamma * units["native_draft_step"]
        out["cpu_baseline"] = {
            "value": round(window_step * 1e6, 1), "unit": "us/step", "cores": threads,
            "kind": "oracle",
            "sample": f"float64 oracle on the host, one unit of each kind of the 1M workload: "
                      f"native draft attention of the first draft step ({h['S'] + 1} keys, every kv "
                      f"head), windowed draft attention of the same step, and the verify of "
                      f"{h['n_q']} causal queries over {h['S'] + h['n_q']} target keys; value = "
                      f"verify + {gamma} windowed draft steps (the windowed decode step's attention)",
            "units_us": {k: round(v * 1e6, 1) for k, v in units.items()},
            "native_decode_step_us": round(native_step * 1e6, 1),
        }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
