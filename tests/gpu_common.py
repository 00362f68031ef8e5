"""Helpers shared by the GPU parity tests: building a decode step's device state
from the seeded workloads, running the library, and comparing with the oracle."""

from __future__ import annotations

import numpy as np

import workloads as W

TOL_ABS = 2e-3        # max |o_gpu - o_ref|, fp32 accumulate from bf16 inputs
TOL_REL = 1e-2        # max |o_gpu - o_ref| / max |o_ref|
TOL_LSE = 1e-3        # max |lse_gpu - lse_ref|


def torch():
    import torch as _t
    return _t


def dev_i32(a):
    return torch().tensor(np.asarray(a, dtype=np.int32), device="cuda")


def dev_bf16(bits):
    from long_context_decode_attention_amd.scenario import to_device_bf16
    return to_device_bf16(bits)


def compare(o_gpu, lse_gpu, o_ref, lse_ref, what=""):
    """Assert the GPU result matches the oracle within the stated tolerances;
    returns (max abs error of o, max abs error of lse)."""
    o = o_gpu.detach().double().cpu().numpy().reshape(np.shape(o_ref))
    lse = lse_gpu.detach().double().cpu().numpy().reshape(np.shape(lse_ref))
    o_ref = np.asarray(o_ref)
    lse_ref = np.asarray(lse_ref)
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: -inf lse pattern differs"
    err = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    scale = float(np.max(np.abs(o_ref))) if o.size else 0.0
    assert err <= TOL_ABS, f"{what}: max abs error {err:.3e} > {TOL_ABS}"
    assert err <= TOL_REL * scale + 1e-7, f"{what}: error {err:.3e} vs output scale {scale:.3e}"
    lerr = float(np.max(np.abs(lse[~empty] - lse_ref[~empty]))) if np.any(~empty) else 0.0
    assert lerr <= TOL_LSE, f"{what}: lse error {lerr:.3e} > {TOL_LSE}"
    return err, lerr


class DraftScenario:
    """One sequence batch of a draft chain: logical draft K/V, a paged cache holding
    the first S_b positions, a ring holding the same (sink + recent), and the
    queries of each draft step."""

    def __init__(self, cfg: dict, seed: int, S: list, gamma: int, perm: bool = None,
                 poison: bool = True, peak: float = 1.0):
        import long_context_decode_attention_amd as lib
        from long_context_decode_attention_amd import scenario as sc

        self.cfg, self.seed, self.S, self.gamma = cfg, seed, list(S), gamma
        B, Hkv, D = len(S), cfg["Hkv"], cfg["D"]
        self.B, self.Hq, self.Hkv, self.D = B, cfg["Hq"], Hkv, D
        self.K = [W.kv_positions(seed, "draft_k", b, 0, S[b] + gamma, Hkv, D) for b in range(B)]
        self.V = [W.kv_positions(seed, "draft_v", b, 0, S[b] + gamma, Hkv, D) for b in range(B)]
        cap = [s + gamma for s in S]
        permute = cfg.get("permute", False) if perm is None else perm
        n_pages = sum((c + 63) // 64 for c in cap)
        p = W.page_permutation(seed, "draft_k", n_pages) if permute else None
        self.kv = sc.alloc_paged_kv(cap, Hkv, D, p)
        self.ring = lib.new_ring(B, cfg["C"], Hkv, D, cfg["n_sink"], cfg["n_recent"])
        if poison:
            sc.poison(self.kv.k)
            sc.poison(self.kv.v)
            sc.poison(self.ring.k)
            sc.poison(self.ring.v)
        for b in range(B):
            sc.fill_paged(self.kv, b, 0, self.K[b][:S[b]], self.V[b][:S[b]])
            sc.fill_ring(self.ring, b, self.K[b][:S[b]], self.V[b][:S[b]])
        self.peak = peak
        self.step_done = 0

    def q(self, j):
        return W.queries(self.seed, "q_draft", (self.B, self.Hq), self.D, step=j, peak=self.peak)

    def append(self, j):
        """Draft step j (1-based) appends position S_b + j - 1 to both arms."""
        import long_context_decode_attention_amd as lib
        kn = np.stack([self.K[b][self.S[b] + j - 1][None] for b in range(self.B)])
        vn = np.stack([self.V[b][self.S[b] + j - 1][None] for b in range(self.B)])
        kt, vt = dev_bf16(kn), dev_bf16(vn)
        lib.paged_append(self.kv.k, self.kv.v, self.kv.block_table,
                         dev_i32([s + j - 1 for s in self.S]), kt, vt)
        lib.ring_append(self.ring, kt, vt)

    def lens(self, j):
        return [s + j for s in self.S]


class VerifyScenario:
    """Target K/V of a batch: S_b positions plus the n_q proposed ones appended."""

    def __init__(self, cfg: dict, seed: int, S: list, n_q: int, perm: bool = None,
                 poison: bool = True, layer: int = 0):
        from long_context_decode_attention_amd import scenario as sc
        B, Hkv, D = len(S), cfg["Hkv"], cfg["D"]
        self.B, self.Hq, self.Hkv, self.D, self.S, self.n_q = B, cfg["Hq"], Hkv, D, list(S), n_q
        self.seed = seed
        tk, tv = ("target_k", "target_v")
        self.K = [W.kv_positions(seed + 1000 * layer, tk, b, 0, S[b] + n_q, Hkv, D) for b in range(B)]
        self.V = [W.kv_positions(seed + 1000 * layer, tv, b, 0, S[b] + n_q, Hkv, D) for b in range(B)]
        cap = [s + n_q for s in S]
        permute = cfg.get("permute", False) if perm is None else perm
        n_pages = sum((c + 63) // 64 for c in cap)
        p = W.page_permutation(seed, "target_k", n_pages) if permute else None
        self.kv = sc.alloc_paged_kv(cap, Hkv, D, p)
        if poison:
            sc.poison(self.kv.k)
            sc.poison(self.kv.v)
        for b in range(B):
            sc.fill_paged(self.kv, b, 0, self.K[b][:S[b]], self.V[b][:S[b]])
        self.q = W.queries(seed + 1000 * layer, "q_verify", (B, n_q, self.Hq), D)

    def append_proposed(self):
        import long_context_decode_attention_amd as lib
        kn = np.stack([self.K[b][self.S[b]:self.S[b] + self.n_q] for b in range(self.B)])
        vn = np.stack([self.V[b][self.S[b]:self.S[b] + self.n_q] for b in range(self.B)])
        lib.paged_append(self.kv.k, self.kv.v, self.kv.block_table, dev_i32(self.S),
                         dev_bf16(kn), dev_bf16(vn))

    def lens(self):
        return [s + self.n_q for s in self.S]
