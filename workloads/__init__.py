"""Seeded synthetic inputs shared by the oracle-side tests and the GPU path.

This module holds the workload shapes and the random-number recipe and nothing
of the method's arithmetic: no attention, no softmax, no ring mapping, no split
bookkeeping.  Both sides receive the same arrays from here; neither side's code
lives here.

Recipe (the pages measure on real models and long-context task suites that are
not available here; these synthetic inputs stand in for them with the pages'
shapes: 1M-token context, one GPU, a 4K sink-plus-recent draft window, draft depth
up to 7):

* K, V: float32 draws of N(0, 1) rounded to bf16 (round to nearest even);
* q: N(0, 1) / sqrt(D) in float32, rounded to bf16; the softmax scale is then 1.0;
* every KV page of 64 positions gets its own PCG64 stream keyed by
  ``(seed, tensor, sequence, page)``, so any page can be regenerated alone and
  pages are generated in parallel threads;
* physical page order is a seeded permutation of the logical pages;
* ragged batch lengths are integers uniform on ``[lo, hi]`` inclusive.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

PAGE = 64

TENSORS = {
    "draft_k": 11, "draft_v": 12,        # the draft head's own KV (native arm reads all of it)
    "target_k": 21, "target_v": 22,      # the target's KV (verify reads all of it)
    "q_draft": 31, "q_verify": 32, "q_ctx": 33,   # q_ctx: the draft context pass
    "perm": 41, "lens": 42, "misc": 51,
}

# Workloads, named by what they are.  Sizes follow the five benchmark configurations.
CONFIGS = {
    # single decode query, batch 1, GQA 16/2, head_dim 128, context 8192, window 4 + 1020
    "ctx8k_g16x2_d128": dict(B=1, Hq=16, Hkv=2, D=128, S=8192, gamma=1,
                             n_sink=4, n_recent=1020, C=1024, n_q=0, permute=False, layers=1),
    # batch 1, GQA 32/4, head_dim 128, context 128K, 3 chained draft steps, window 4 + 4092
    "ctx128k_g32x4_d128": dict(B=1, Hq=32, Hkv=4, D=128, S=131072, gamma=3,
                               n_sink=4, n_recent=4092, C=4096, n_q=0, permute=False, layers=1),
    # batch 1, GQA 32/2, head_dim 256, context 1M in permuted 64-token pages, 7 draft
    # steps, window 4 + 4092, verify of 8 causal queries over the full 1M context
    "ctx1m_g32x2_d256": dict(B=1, Hq=32, Hkv=2, D=256, S=1048576, gamma=7,
                             n_sink=4, n_recent=4092, C=4096, n_q=8, permute=True, layers=1),
    # batch 8, ragged contexts uniform in [256K, 1M], GQA 32/4, head_dim 128, shared
    # permuted page pool, 3 draft steps, window 4096, verify of 4 causal queries
    "ragged8_256k_1m_g32x4_d128": dict(B=8, Hq=32, Hkv=4, D=128, S=None, len_lo=262144,
                                       len_hi=1048576, gamma=3, n_sink=4, n_recent=4092,
                                       C=4096, n_q=4, permute=True, layers=1),
    # hybrid-style stack: 8 attention layers (identity blocks between), batch 1, GQA
    # 64/2, head_dim 128, 1M context plus 10,000 decode appends (the draft ring wraps),
    # 7 draft steps, verify of 8 causal queries per layer
    "nope8l_1m_g64x2_d128": dict(B=1, Hq=64, Hkv=2, D=128, S=1048576 + 10000, gamma=7,
                                 n_sink=4, n_recent=4092, C=4096, n_q=8, permute=True, layers=8),
}


def _threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed)] + [int(k) for k in key])))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even.  Finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact).  For building inputs and plotting only."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _page(seed: int, tensor: int, b: int, page: int, Hkv: int, D: int) -> np.ndarray:
    g = _rng(seed, tensor, b, page)
    return bf16_round(g.standard_normal((PAGE, Hkv, D), dtype=np.float32))


def kv_positions(seed: int, name: str, b: int, lo: int, hi: int, Hkv: int, D: int,
                 out: np.ndarray | None = None) -> np.ndarray:
    """bf16 bits [hi - lo, Hkv, D] for positions ``lo .. hi-1`` of sequence ``b`` of KV tensor ``name``.

    Position ``p`` lives on logical page ``p // 64``; every page has its own stream,
    so the values of a position do not depend on ``lo``/``hi``.
    """
    tensor = TENSORS[name]
    n = hi - lo
    if out is None:
        out = np.empty((n, Hkv, D), dtype=np.uint16)
    if n <= 0:
        return out
    p0, p1 = lo // PAGE, (hi - 1) // PAGE + 1

    def fill(page: int):
        blk = _page(seed, tensor, b, page, Hkv, D)
        a = max(lo, page * PAGE)
        e = min(hi, (page + 1) * PAGE)
        out[a - lo:e - lo] = blk[a - page * PAGE:e - page * PAGE]

    pages = range(p0, p1)
    if len(pages) < 8:
        for p in pages:
            fill(p)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, pages))
    return out


def queries(seed: int, name: str, shape: tuple, D: int, step: int = 0, peak: float = 1.0) -> np.ndarray:
    """bf16 bits of shape ``shape + (D,)``: N(0, 1) / sqrt(D) * ``peak`` (``peak`` > 1 gives
    sharper attention).  ``step`` keys the draft step."""
    g = _rng(seed, TENSORS[name], step)
    x = g.standard_normal(tuple(shape) + (D,), dtype=np.float32)
    x = x * np.float32(peak / np.sqrt(D))
    return bf16_round(x)


def page_permutation(seed: int, name: str, n_pages: int) -> np.ndarray:
    """Seeded permutation of ``n_pages`` physical page ids (int32)."""
    if n_pages == 0:
        return np.zeros(0, dtype=np.int32)
    return _rng(seed, TENSORS["perm"], TENSORS[name]).permutation(n_pages).astype(np.int32)


def ragged_lengths(seed: int, B: int, lo: int, hi: int) -> np.ndarray:
    """``B`` context lengths uniform on ``[lo, hi]`` inclusive (int64)."""
    return _rng(seed, TENSORS["lens"]).integers(lo, hi + 1, size=B).astype(np.int64)


def context_lengths(cfg: dict, seed: int) -> np.ndarray:
    """Context ``S_b`` held before the decode step, per sequence."""
    if cfg.get("S") is not None:
        return np.full(cfg["B"], cfg["S"], dtype=np.int64)
    return ragged_lengths(seed, cfg["B"], cfg["len_lo"], cfg["len_hi"])


def shrink(cfg: dict, S: int | None = None, **over) -> dict:
    """A copy of ``cfg`` with a smaller context (and any other overrides), for
    oracle-sized parity cases of the same shape."""
    c = dict(cfg)
    if S is not None:
        c["S"] = S
        c.pop("len_lo", None)
        c.pop("len_hi", None)
    c.update(over)
    return c
