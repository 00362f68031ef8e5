"""Device state for a decode step: paged KV caches and draft rings, filled through
the library's own append kernels from host arrays of logical K/V.

Host arrays are bf16 bit patterns (numpy uint16) shaped [positions, Hkv, D];
where they come from is the caller's business.  Nothing here computes attention.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import PAGE, Ring, new_paged_cache, new_ring, paged_append, ring_append


def _torch():
    import torch
    return torch


def to_device_bf16(bits: np.ndarray, device="cuda"):
    """uint16 bf16 bit patterns -> a bf16 device tensor of the same shape (bit-exact)."""
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


@dataclass
class PagedKV:
    k: object                 # bf16 tiled pages
    v: object
    block_table: object       # int32 [B, max_pages]; -1 = no page
    num_pages: int
    max_pages: int
    capacity: list            # positions each sequence can hold


def alloc_paged_kv(capacity: list, Hkv: int, D: int, perm: np.ndarray | None = None,
                   device="cuda") -> PagedKV:
    """A shared pool with room for ``capacity[b]`` positions of each sequence.
    Logical pages are dealt out in order; ``perm`` (a permutation of the pool)
    scatters them over physical pages."""
    torch = _torch()
    pages = [(c + PAGE - 1) // PAGE for c in capacity]
    num_pages = max(1, sum(pages))
    max_pages = max(1, max(pages))
    if perm is None:
        perm = np.arange(num_pages, dtype=np.int32)
    if len(perm) != num_pages:
        raise ValueError("perm must have one entry per pool page")
    bt = np.full((len(capacity), max_pages), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[off:off + n]
        off += n
    k, v = new_paged_cache(num_pages, Hkv, D, device)
    return PagedKV(k, v, torch.from_numpy(bt).to(device), num_pages, max_pages, list(capacity))


def fill_paged(kv: PagedKV, b: int, start: int, k_bits: np.ndarray, v_bits: np.ndarray,
               chunk: int = 1 << 16, device="cuda") -> None:
    """Write logical positions ``start .. start + len - 1`` of sequence ``b``."""
    torch = _torch()
    n = k_bits.shape[0]
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        kn = to_device_bf16(k_bits[lo:hi], device).unsqueeze(0)
        vn = to_device_bf16(v_bits[lo:hi], device).unsqueeze(0)
        sp = torch.tensor([start + lo], dtype=torch.int32, device=device)
        paged_append(kv.k, kv.v, kv.block_table[b:b + 1], sp, kn, vn)


def fill_ring(ring: Ring, b: int, k_bits: np.ndarray, v_bits: np.ndarray,
              chunk: int = 1 << 16, device="cuda") -> None:
    """Append positions ``T .. T + len - 1`` to ring ``b`` (bulk appends)."""
    n = k_bits.shape[0]
    per = ring.C // PAGE
    sub = Ring(ring.k[b * per:(b + 1) * per], ring.v[b * per:(b + 1) * per],
               ring.pos[b:b + 1], ring.T[b:b + 1], ring.C, ring.n_sink, ring.n_recent)
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        kn = to_device_bf16(k_bits[lo:hi], device).unsqueeze(0)
        vn = to_device_bf16(v_bits[lo:hi], device).unsqueeze(0)
        ring_append(sub, kn, vn)


def poison(t, value=float("nan")) -> None:
    """Fill a tensor with NaN (or another value): slots no position was written to
    must then never reach a result."""
    t.view(_torch().bfloat16).fill_(value) if t.dtype == _torch().bfloat16 else t.fill_(value)


__all__ = ["PagedKV", "alloc_paged_kv", "fill_paged", "fill_ring", "to_device_bf16", "poison",
           "new_ring"]
