"""Windowed-MTP draft/verify attention for MI355X: Python binding of libwmtp.so.

Argument marshalling only: every step of the path runs in the HIP kernels of
``libwmtp.so`` (sources in ``csrc/``, C ABI in ``include/wmtp.h``).  PyTorch is
used for device memory and streams.  If the library is not built this module
still imports, but every call raises: there is no fallback path.

KV caches use the tiled page layout of the C ABI: a page of 64 positions and one
kv head is two tiles of 32 positions; K tiles are ``[D/16][32 pos][16 dims]``,
V tiles ``[2][D][16 pos]``.  :func:`new_paged_cache` and :func:`new_ring` allocate
tensors with those shapes; the append calls write them.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
# WMTP_LIBRARY names another build of the same library (e.g. the host-sanitized
# one the CPU tests load); there is no fallback when the file is missing.
LIB_PATH = os.environ.get("WMTP_LIBRARY") or os.path.join(HERE, "libwmtp.so")
PAGE = 64
FLAG_PARTIALS_ONLY = 1

# Every symbol include/wmtp.h declares.
EXPORTS = (
    "wmtp_status_string", "wmtp_plan_splits", "wmtp_workspace_bytes",
    "wmtp_draft_attn_full", "wmtp_draft_attn_window", "wmtp_draft_attn_window_paged",
    "wmtp_draft_context_window", "wmtp_verify_attn_tree", "wmtp_paged_append_fp8",
    "wmtp_draft_attn_full_fp8", "wmtp_draft_attn_window_paged_fp8", "wmtp_ring_append",
    "wmtp_paged_append", "wmtp_verify_attn", "wmtp_verify_attn_fp8", "wmtp_split_combine",
    "wmtp_draft_step_window",
    "wmtp_draft_context_step_window", "wmtp_draft_step_window_static",
)

STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported configuration",
          3: "workspace missing or too small", 4: "HIP launch error"}


class WmtpError(RuntimeError):
    """A libwmtp call returned a non-zero status."""

    def __init__(self, call: str, status: int):
        super().__init__(f"{call}: {STATUS.get(status, 'unknown status')} (status {status})")
        self.status = status


_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t
_U = ctypes.c_uint

_SIGS = {
    "wmtp_status_string": ([_I], ctypes.c_char_p),
    "wmtp_plan_splits": ([_I] * 8, _I),
    "wmtp_workspace_bytes": ([_I] * 9, _SZ),
    "wmtp_draft_attn_full": ([_P] * 5 + [_I] * 7 + [_F, _P, _P, _P, _SZ, _I, _U, _P], _I),
    "wmtp_draft_attn_window": ([_P] * 5 + [_I] * 7 + [_F, _P, _P, _P, _SZ, _I, _U, _P], _I),
    "wmtp_draft_attn_window_paged": ([_P] * 5 + [_I] * 9 + [_F, _P, _P, _P, _SZ, _I, _U, _P], _I),
    "wmtp_draft_context_window": ([_P] * 5 + [_I] * 8 + [_F, _P, _P, _P, _SZ, _I, _U, _P], _I),
    "wmtp_verify_attn_tree": ([_P] * 6 + [_I] * 8 + [_F, _P, _P, _P, _SZ, _I, _U, _P], _I),
    "wmtp_paged_append_fp8": ([_P] * 6 + [_I] * 6 + [_F, _F, _P], _I),
    "wmtp_draft_attn_full_fp8": ([_P] * 5 + [_I] * 7 + [_F, _F, _F, _P, _P, _P, _SZ, _I, _U, _P], _I),
    "wmtp_draft_attn_window_paged_fp8": ([_P] * 5 + [_I] * 9 + [_F, _F, _F, _P, _P, _P, _SZ, _I, _U, _P],
                                         _I),
    "wmtp_ring_append": ([_P] * 6 + [_I] * 6 + [_P], _I),
    "wmtp_draft_step_window": ([_P] * 7 + [_I] * 8 + [_F, _P, _P, _P, _SZ, _I, _P], _I),
    "wmtp_draft_context_step_window": ([_P] * 7 + [_I] * 9 + [_F, _P, _P, _P, _SZ, _I, _P], _I),
    "wmtp_draft_step_window_static": ([_P] * 7 + [_I] * 8 + [_F, _P, _P, _I, _P], _I),
    "wmtp_paged_append": ([_P] * 6 + [_I] * 6 + [_P], _I),
    "wmtp_verify_attn": ([_P] * 5 + [_I] * 8 + [_F, _P, _P, _P, _SZ, _I, _U, _P], _I),
    "wmtp_verify_attn_fp8": ([_P] * 5 + [_I] * 8 + [_F, _F, _F, _P, _P, _P, _SZ, _I, _U, _P], _I),
    "wmtp_split_combine": ([_P, _P, _I, _P] + [_I] * 6 + [_P, _P, _P], _I),
}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libwmtp.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m long_context_decode_attention_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (args, res) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().wmtp_status_string(int(status)).decode()


def _check(call: str, status: int) -> None:
    if status != 0:
        raise WmtpError(call, status)


class Call:
    """A library call with its arguments already marshalled: calling it launches
    the kernels again with the same buffers (no per-call Python checks)."""

    __slots__ = ("name", "fn", "args")

    def __init__(self, name: str, args: tuple):
        self.name = name
        self.fn = getattr(load(), name)
        self.args = args

    def __call__(self) -> None:
        st = self.fn(*self.args)
        if st != 0:
            raise WmtpError(self.name, st)


def _invoke(name: str, args: tuple, prepare: bool):
    c = Call(name, args)
    if prepare:
        return c
    c()
    return None


# ----------------------------------------------------------------------------- torch plumbing

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, shape, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def k_cache_shape(num_pages: int, Hkv: int, D: int) -> tuple:
    return (num_pages, Hkv, 2, D // 16, 32, 16)


def v_cache_shape(num_pages: int, Hkv: int, D: int) -> tuple:
    return (num_pages, Hkv, 2, 2, D, 16)


def new_paged_cache(num_pages: int, Hkv: int, D: int, device="cuda"):
    """Uninitialised K and V caches of ``num_pages`` tiled pages (bf16)."""
    torch = _torch()
    k = torch.empty(k_cache_shape(num_pages, Hkv, D), dtype=torch.bfloat16, device=device)
    v = torch.empty(v_cache_shape(num_pages, Hkv, D), dtype=torch.bfloat16, device=device)
    return k, v


def new_paged_cache_fp8(num_pages: int, Hkv: int, D: int, device="cuda"):
    """Uninitialised fp8 (e4m3 codes, uint8) K and V caches: the bf16 tile layout,
    one byte per element."""
    torch = _torch()
    k = torch.empty(k_cache_shape(num_pages, Hkv, D), dtype=torch.uint8, device=device)
    v = torch.empty(v_cache_shape(num_pages, Hkv, D), dtype=torch.uint8, device=device)
    return k, v


@dataclass
class Ring:
    """Draft-KV rings of a batch: ``C`` slots each, ``n_sink`` kept for good, the
    window reading the last ``n_recent`` positions (capacity beyond
    ``n_sink + n_recent`` is slack)."""
    k: object
    v: object
    pos: object          # int32 [B, C], -1 = empty
    T: object            # int64 [B]
    C: int
    n_sink: int
    n_recent: int

    @property
    def B(self) -> int:
        return self.pos.shape[0]

    @property
    def Hkv(self) -> int:
        return self.k.shape[1]

    @property
    def D(self) -> int:
        return self.v.shape[4]


def new_ring(B: int, C: int, Hkv: int, D: int, n_sink: int, n_recent: int, device="cuda") -> Ring:
    """Empty rings (positions -1, counts 0); K/V slots uninitialised."""
    torch = _torch()
    if C % PAGE:
        raise ValueError("ring capacity must be a multiple of 64")
    k, v = new_paged_cache(B * (C // PAGE), Hkv, D, device)
    pos = torch.full((B, C), -1, dtype=torch.int32, device=device)
    T = torch.zeros(B, dtype=torch.int64, device=device)
    return Ring(k, v, pos, T, C, n_sink, n_recent)


# ----------------------------------------------------------------------------- planning

CALL_PAGED = 0
CALL_RING = 1
CALL_PAGED_WINDOW = 2
CALL_RING_STEP = 3
CALL_PAGED_FP8 = 4


def _call_kind(ring, paged_window, fp8=False):
    if ring:
        return CALL_RING
    if paged_window:
        return CALL_PAGED_WINDOW
    return CALL_PAGED_FP8 if fp8 else CALL_PAGED


def plan_splits(B, Hq, Hkv, D, n_q, max_keys, num_splits=0, ring=False,
                paged_window=False, fp8=False) -> int:
    """Splits per (sequence, kv head); with ``paged_window`` max_keys is the window
    n_sink + n_recent of ``draft_attn_window_paged``; ``fp8`` for
    ``draft_attn_full_fp8``."""
    n = load().wmtp_plan_splits(_call_kind(ring, paged_window, fp8), B, Hq, Hkv, D, n_q, max_keys,
                                num_splits)
    if n < 0:
        raise WmtpError("wmtp_plan_splits", 1)
    return n


def workspace_bytes(B, Hq, Hkv, D, n_q, max_keys, num_splits=0, partials_only=False,
                    ring=False, paged_window=False, fp8=False) -> int:
    return int(load().wmtp_workspace_bytes(_call_kind(ring, paged_window, fp8), B, Hq, Hkv, D,
                                           n_q, max_keys, num_splits, 1 if partials_only else 0))


def step_splits(B, Hq, Hkv, D, C, num_splits=0, n_q=1) -> int:
    """Ring splits per (request, kv head) of ``draft_step_window`` and, with n_q
    queries, ``draft_context_step_window`` (each group then has that many plus one
    partials)."""
    n = load().wmtp_plan_splits(CALL_RING_STEP, B, Hq, Hkv, D, n_q, C, num_splits)
    if n < 0:
        raise WmtpError("wmtp_plan_splits", 1)
    return n


def step_workspace_bytes(B, Hq, Hkv, D, C, num_splits=0, n_q=1) -> int:
    return int(load().wmtp_workspace_bytes(CALL_RING_STEP, B, Hq, Hkv, D, n_q, C, num_splits, 0))


def new_workspace(nbytes: int, device="cuda"):
    torch = _torch()
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def partials_view(workspace, B, Hq, Hkv, D, n_q, max_keys, num_splits=0, ring=False,
                  paged_window=False, fp8=False):
    """(part_o [P, R, D], part_lse [P, R]) views of a workspace left by a
    partials-only call with the same arguments."""
    torch = _torch()
    splits = plan_splits(B, Hq, Hkv, D, n_q, max_keys, num_splits, ring, paged_window, fp8)
    P = B * Hkv * splits
    R = n_q * (Hq // Hkv)
    ob = P * R * D * 4
    off = (ob + 255) // 256 * 256
    po = workspace[:ob].view(torch.float32).view(P, R, D)
    pl = workspace[off:off + P * R * 4].view(torch.float32).view(P, R)
    return po, pl


# ----------------------------------------------------------------------------- calls

def _outputs(o, lse, shape, lse_shape, device):
    torch = _torch()
    if o is None:
        o = torch.empty(shape, dtype=torch.float32, device=device)
    if lse is None:
        lse = torch.empty(lse_shape, dtype=torch.float32, device=device)
    _need(o, torch.float32, shape, "o")
    _need(lse, torch.float32, lse_shape, "lse")
    return o, lse


def draft_attn_full(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, softmax_scale=1.0,
                    o=None, lse=None, workspace=None, num_splits=0, partials_only=False,
                    stream=None, prepare=False):
    """Native draft attention (``wmtp_draft_attn_full``).  Returns (o, lse), or the
    workspace holding the partials when ``partials_only``; with ``prepare`` a
    :class:`Call` that repeats the launch."""
    torch = _torch()
    B, Hq, D = q.shape
    num_pages, Hkv = k_cache.shape[0], k_cache.shape[1]
    max_pages = block_table.shape[1]
    _need(q, torch.bfloat16, None, "q")
    _need(k_cache, torch.bfloat16, k_cache_shape(num_pages, Hkv, D), "k_cache")
    _need(v_cache, torch.bfloat16, v_cache_shape(num_pages, Hkv, D), "v_cache")
    _need(block_table, torch.int32, (B, max_pages), "block_table")
    _need(seq_lens, torch.int32, (B,), "seq_lens")
    max_keys = min(int(max_seq_len), max_pages * PAGE)
    need = workspace_bytes(B, Hq, Hkv, D, 1, max_keys, num_splits, partials_only)
    if workspace is None:
        workspace = new_workspace(need, q.device)
    _need(workspace, torch.uint8, None, "workspace")
    if not partials_only:
        o, lse = _outputs(o, lse, (B, Hq, D), (B, Hq), q.device)
    c = _invoke("wmtp_draft_attn_full", (
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
        B, Hq, Hkv, D, num_pages, max_pages, int(max_seq_len), float(softmax_scale),
        _ptr(o), _ptr(lse), _ptr(workspace), workspace.numel(), int(num_splits),
        FLAG_PARTIALS_ONLY if partials_only else 0, _stream(stream)), prepare)
    if prepare:
        return c
    return workspace if partials_only else (o, lse)


def verify_attn_tree(q, k_cache, v_cache, block_table, seq_lens, tree_mask, max_seq_len,
                     softmax_scale=1.0, o=None, lse=None, workspace=None, num_splits=0,
                     partials_only=False, stream=None, prepare=False):
    """Verify of a tree of proposals (``wmtp_verify_attn_tree``): q is [B, n_q, Hq, D];
    tree_mask int64 [B, n_q], bit a of row i set when query i sees appended position a."""
    torch = _torch()
    B, n_q, Hq, D = q.shape
    num_pages, Hkv = k_cache.shape[0], k_cache.shape[1]
    max_pages = block_table.shape[1]
    _need(q, torch.bfloat16, None, "q")
    _need(k_cache, torch.bfloat16, k_cache_shape(num_pages, Hkv, D), "k_cache")
    _need(v_cache, torch.bfloat16, v_cache_shape(num_pages, Hkv, D), "v_cache")
    _need(block_table, torch.int32, (B, max_pages), "block_table")
    _need(seq_lens, torch.int32, (B,), "seq_lens")
    _need(tree_mask, torch.int64, (B, n_q), "tree_mask")
    max_keys = min(int(max_seq_len), max_pages * PAGE)
    need = workspace_bytes(B, Hq, Hkv, D, n_q, max_keys, num_splits, partials_only)
    if workspace is None:
        workspace = new_workspace(need, q.device)
    _need(workspace, torch.uint8, None, "workspace")
    if not partials_only:
        o, lse = _outputs(o, lse, (B, n_q, Hq, D), (B, n_q, Hq), q.device)
    c = _invoke("wmtp_verify_attn_tree", (
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens), _ptr(tree_mask),
        B, n_q, Hq, Hkv, D, num_pages, max_pages, int(max_seq_len), float(softmax_scale),
        _ptr(o), _ptr(lse), _ptr(workspace), workspace.numel(), int(num_splits),
        FLAG_PARTIALS_ONLY if partials_only else 0, _stream(stream)), prepare)
    if prepare:
        return c
    return workspace if partials_only else (o, lse)


def draft_attn_window_paged(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, n_sink,
                            n_recent, softmax_scale=1.0, o=None, lse=None, workspace=None,
                            num_splits=0, partials_only=False, stream=None, prepare=False):
    """Windowed draft attention by index truncation over the paged draft KV
    (``wmtp_draft_attn_window_paged``): keys [0, n_sink) and the last n_recent."""
    torch = _torch()
    B, Hq, D = q.shape
    num_pages, Hkv = k_cache.shape[0], k_cache.shape[1]
    max_pages = block_table.shape[1]
    _need(q, torch.bfloat16, None, "q")
    _need(k_cache, torch.bfloat16, k_cache_shape(num_pages, Hkv, D), "k_cache")
    _need(v_cache, torch.bfloat16, v_cache_shape(num_pages, Hkv, D), "v_cache")
    _need(block_table, torch.int32, (B, max_pages), "block_table")
    _need(seq_lens, torch.int32, (B,), "seq_lens")
    need = workspace_bytes(B, Hq, Hkv, D, 1, int(n_sink) + int(n_recent), num_splits,
                           partials_only, paged_window=True)
    if workspace is None:
        workspace = new_workspace(need, q.device)
    _need(workspace, torch.uint8, None, "workspace")
    if not partials_only:
        o, lse = _outputs(o, lse, (B, Hq, D), (B, Hq), q.device)
    c = _invoke("wmtp_draft_attn_window_paged", (
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
        B, Hq, Hkv, D, num_pages, max_pages, int(max_seq_len), int(n_sink), int(n_recent),
        float(softmax_scale), _ptr(o), _ptr(lse), _ptr(workspace), workspace.numel(),
        int(num_splits), FLAG_PARTIALS_ONLY if partials_only else 0, _stream(stream)), prepare)
    if prepare:
        return c
    return workspace if partials_only else (o, lse)


def verify_attn(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, softmax_scale=1.0,
                o=None, lse=None, workspace=None, num_splits=0, partials_only=False, stream=None,
                prepare=False):
    """Causal full-context verify (``wmtp_verify_attn``); q is [B, n_q, Hq, D]."""
    torch = _torch()
    B, n_q, Hq, D = q.shape
    num_pages, Hkv = k_cache.shape[0], k_cache.shape[1]
    max_pages = block_table.shape[1]
    _need(q, torch.bfloat16, None, "q")
    _need(k_cache, torch.bfloat16, k_cache_shape(num_pages, Hkv, D), "k_cache")
    _need(v_cache, torch.bfloat16, v_cache_shape(num_pages, Hkv, D), "v_cache")
    _need(block_table, torch.int32, (B, max_pages), "block_table")
    _need(seq_lens, torch.int32, (B,), "seq_lens")
    max_keys = min(int(max_seq_len), max_pages * PAGE)
    need = workspace_bytes(B, Hq, Hkv, D, n_q, max_keys, num_splits, partials_only)
    if workspace is None:
        workspace = new_workspace(need, q.device)
    _need(workspace, torch.uint8, None, "workspace")
    if not partials_only:
        o, lse = _outputs(o, lse, (B, n_q, Hq, D), (B, n_q, Hq), q.device)
    c = _invoke("wmtp_verify_attn", (
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
        B, n_q, Hq, Hkv, D, num_pages, max_pages, int(max_seq_len), float(softmax_scale),
        _ptr(o), _ptr(lse), _ptr(workspace), workspace.numel(), int(num_splits),
        FLAG_PARTIALS_ONLY if partials_only else 0, _stream(stream)), prepare)
    if prepare:
        return c
    return workspace if partials_only else (o, lse)


def verify_attn_fp8(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, k_scale=1.0,
                    v_scale=1.0, softmax_scale=1.0, o=None, lse=None, workspace=None,
                    num_splits=0, partials_only=False, stream=None, prepare=False):
    """Causal full-context verify over fp8 caches (``wmtp_verify_attn_fp8``); q is
    [B, n_q, Hq, D], the caches uint8 (e4m3 codes) in the tiled page layout."""
    torch = _torch()
    B, n_q, Hq, D = q.shape
    num_pages, Hkv = k_cache.shape[0], k_cache.shape[1]
    max_pages = block_table.shape[1]
    _need(q, torch.bfloat16, None, "q")
    _need(k_cache, torch.uint8, k_cache_shape(num_pages, Hkv, D), "k_cache")
    _need(v_cache, torch.uint8, v_cache_shape(num_pages, Hkv, D), "v_cache")
    _need(block_table, torch.int32, (B, max_pages), "block_table")
    _need(seq_lens, torch.int32, (B,), "seq_lens")
    max_keys = min(int(max_seq_len), max_pages * PAGE)
    need = workspace_bytes(B, Hq, Hkv, D, n_q, max_keys, num_splits, partials_only, fp8=True)
    if workspace is None:
        workspace = new_workspace(need, q.device)
    _need(workspace, torch.uint8, None, "workspace")
    if not partials_only:
        o, lse = _outputs(o, lse, (B, n_q, Hq, D), (B, n_q, Hq), q.device)
    c = _invoke("wmtp_verify_attn_fp8", (
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
        B, n_q, Hq, Hkv, D, num_pages, max_pages, int(max_seq_len), float(k_scale),
        float(v_scale), float(softmax_scale), _ptr(o), _ptr(lse), _ptr(workspace),
        workspace.numel(), int(num_splits), FLAG_PARTIALS_ONLY if partials_only else 0,
        _stream(stream)), prepare)
    if prepare:
        return c
    return workspace if partials_only else (o, lse)


def draft_attn_window(q, ring: Ring, softmax_scale=1.0, o=None, lse=None, workspace=None,
                      num_splits=0, partials_only=False, stream=None, prepare=False):
    """Windowed draft attention over the rings (``wmtp_draft_attn_window``)."""
    torch = _torch()
    B, Hq, D = q.shape
    Hkv, C = ring.Hkv, ring.C
    _need(q, torch.bfloat16, None, "q")
    _need(ring.k, torch.bfloat16, k_cache_shape(B * C // PAGE, Hkv, D), "ring.k")
    _need(ring.v, torch.bfloat16, v_cache_shape(B * C // PAGE, Hkv, D), "ring.v")
    _need(ring.pos, torch.int32, (B, C), "ring.pos")
    _need(ring.T, torch.int64, (B,), "ring.T")
    need = workspace_bytes(B, Hq, Hkv, D, 1, C, num_splits, partials_only, ring=True)
    if workspace is None:
        workspace = new_workspace(need, q.device)
    _need(workspace, torch.uint8, None, "workspace")
    if not partials_only:
        o, lse = _outputs(o, lse, (B, Hq, D), (B, Hq), q.device)
    c = _invoke("wmtp_draft_attn_window", (
        _ptr(q), _ptr(ring.k), _ptr(ring.v), _ptr(ring.pos), _ptr(ring.T),
        B, Hq, Hkv, D, C, ring.n_sink, ring.n_recent, float(softmax_scale),
        _ptr(o), _ptr(lse), _ptr(workspace), workspace.numel(), int(num_splits),
        FLAG_PARTIALS_ONLY if partials_only else 0, _stream(stream)), prepare)
    if prepare:
        return c
    return workspace if partials_only else (o, lse)


def draft_context_window(q, ring: Ring, softmax_scale=1.0, o=None, lse=None, workspace=None,
                         num_splits=0, partials_only=False, stream=None, prepare=False):
    """Draft context pass over the rings (``wmtp_draft_context_window``): q is
    [B, n_q, Hq, D], query i at position ring.T - n_q + i, each over its own window."""
    torch = _torch()
    B, n_q, Hq, D = q.shape
    Hkv, C = ring.Hkv, ring.C
    _need(q, torch.bfloat16, None, "q")
    _need(ring.k, torch.bfloat16, k_cache_shape(B * C // PAGE, Hkv, D), "ring.k")
    _need(ring.v, torch.bfloat16, v_cache_shape(B * C // PAGE, Hkv, D), "ring.v")
    _need(ring.pos, torch.int32, (B, C), "ring.pos")
    _need(ring.T, torch.int64, (B,), "ring.T")
    need = workspace_bytes(B, Hq, Hkv, D, n_q, C, num_splits, partials_only, ring=True)
    if workspace is None:
        workspace = new_workspace(need, q.device)
    _need(workspace, torch.uint8, None, "workspace")
    if not partials_only:
        o, lse = _outputs(o, lse, (B, n_q, Hq, D), (B, n_q, Hq), q.device)
    c = _invoke("wmtp_draft_context_window", (
        _ptr(q), _ptr(ring.k), _ptr(ring.v), _ptr(ring.pos), _ptr(ring.T),
        B, n_q, Hq, Hkv, D, C, ring.n_sink, ring.n_recent, float(softmax_scale),
        _ptr(o), _ptr(lse), _ptr(workspace), workspace.numel(), int(num_splits),
        FLAG_PARTIALS_ONLY if partials_only else 0, _stream(stream)), prepare)
    if prepare:
        return c
    return workspace if partials_only else (o, lse)


def draft_step_window(q, ring: Ring, k_new, v_new, softmax_scale=1.0, o=None, lse=None,
                      workspace=None, num_splits=0, stream=None, prepare=False):
    """One windowed draft step in two launches (``wmtp_draft_step_window``): append
    k_new, v_new (bf16 [B, n_new, Hkv, D]) to the rings and attend over the
    window ending with them; q is [B, Hq, D]."""
    torch = _torch()
    B, Hq, D = q.shape
    n_new = k_new.shape[1]
    Hkv, C = ring.Hkv, ring.C
    _need(q, torch.bfloat16, None, "q")
    _need(ring.k, torch.bfloat16, k_cache_shape(B * C // PAGE, Hkv, D), "ring.k")
    _need(ring.v, torch.bfloat16, v_cache_shape(B * C // PAGE, Hkv, D), "ring.v")
    _need(ring.pos, torch.int32, (B, C), "ring.pos")
    _need(ring.T, torch.int64, (B,), "ring.T")
    _need(k_new, torch.bfloat16, (B, n_new, Hkv, D), "k_new")
    _need(v_new, torch.bfloat16, (B, n_new, Hkv, D), "v_new")
    if workspace is None:
        workspace = new_workspace(step_workspace_bytes(B, Hq, Hkv, D, C, num_splits), q.device)
    _need(workspace, torch.uint8, None, "workspace")
    o, lse = _outputs(o, lse, (B, Hq, D), (B, Hq), q.device)
    c = _invoke("wmtp_draft_step_window", (
        _ptr(q), _ptr(ring.k), _ptr(ring.v), _ptr(ring.pos), _ptr(ring.T), _ptr(k_new), _ptr(v_new), B, n_new, Hq, Hkv, D, C, ring.n_sink, ring.n_recent,
        float(softmax_scale), _ptr(o), _ptr(lse), _ptr(workspace), workspace.numel(),
        int(num_splits), _stream(stream)), prepare)
    if prepare:
        return c
    return o, lse


STATIC_SCRATCH_BYTES = 16 << 20


def draft_step_window_static(q, ring: Ring, k_new, v_new, softmax_scale=1.0, o=None, lse=None,
                             num_splits=0, stream=None, prepare=False):
    """``draft_step_window`` without a workspace (``wmtp_draft_step_window_static``):
    the partials go to the library's static scratch on this GPU (at most
    ``STATIC_SCRATCH_BYTES``); calls overlapping in time on one GPU race."""
    torch = _torch()
    B, Hq, D = q.shape
    n_new = k_new.shape[1]
    Hkv, C = ring.Hkv, ring.C
    _need(q, torch.bfloat16, None, "q")
    _need(ring.k, torch.bfloat16, k_cache_shape(B * C // PAGE, Hkv, D), "ring.k")
    _need(ring.v, torch.bfloat16, v_cache_shape(B * C // PAGE, Hkv, D), "ring.v")
    _need(ring.pos, torch.int32, (B, C), "ring.pos")
    _need(ring.T, torch.int64, (B,), "ring.T")
    _need(k_new, torch.bfloat16, (B, n_new, Hkv, D), "k_new")
    _need(v_new, torch.bfloat16, (B, n_new, Hkv, D), "v_new")
    o, lse = _outputs(o, lse, (B, Hq, D), (B, Hq), q.device)
    c = _invoke("wmtp_draft_step_window_static", (
        _ptr(q), _ptr(ring.k), _ptr(ring.v), _ptr(ring.pos), _ptr(ring.T), _ptr(k_new),
        _ptr(v_new), B, n_new, Hq, Hkv, D, C, ring.n_sink, ring.n_recent, float(softmax_scale),
        _ptr(o), _ptr(lse), int(num_splits), _stream(stream)), prepare)
    if prepare:
        return c
    return o, lse


def draft_context_step_window(q, ring: Ring, k_new, v_new, softmax_scale=1.0, o=None, lse=None,
                              workspace=None, num_splits=0, stream=None, prepare=False):
    """The draft context pass fused with its append in two launches
    (``wmtp_draft_context_step_window``): append k_new, v_new (bf16 [B, n_new, Hkv,
    D]) to the rings, then query i of q ([B, n_q, Hq, D]) at position
    ring.T + n_new - n_q + i attends over its own window."""
    torch = _torch()
    B, n_q, Hq, D = q.shape
    n_new = k_new.shape[1]
    Hkv, C = ring.Hkv, ring.C
    _need(q, torch.bfloat16, None, "q")
    _need(ring.k, torch.bfloat16, k_cache_shape(B * C // PAGE, Hkv, D), "ring.k")
    _need(ring.v, torch.bfloat16, v_cache_shape(B * C // PAGE, Hkv, D), "ring.v")
    _need(ring.pos, torch.int32, (B, C), "ring.pos")
    _need(ring.T, torch.int64, (B,), "ring.T")
    _need(k_new, torch.bfloat16, (B, n_new, Hkv, D), "k_new")
    _need(v_new, torch.bfloat16, (B, n_new, Hkv, D), "v_new")
    if workspace is None:
        workspace = new_workspace(step_workspace_bytes(B, Hq, Hkv, D, C, num_splits, n_q),
                                  q.device)
    _need(workspace, torch.uint8, None, "workspace")
    o, lse = _outputs(o, lse, (B, n_q, Hq, D), (B, n_q, Hq), q.device)
    c = _invoke("wmtp_draft_context_step_window", (
        _ptr(q), _ptr(ring.k), _ptr(ring.v), _ptr(ring.pos), _ptr(ring.T), _ptr(k_new),
        _ptr(v_new), B, n_new, n_q, Hq, Hkv, D, C, ring.n_sink, ring.n_recent,
        float(softmax_scale), _ptr(o), _ptr(lse), _ptr(workspace), workspace.numel(),
        int(num_splits), _stream(stream)), prepare)
    if prepare:
        return c
    return o, lse


def ring_append(ring: Ring, k_new, v_new, stream=None, prepare=False):
    """Append ``n_new`` positions per request (``wmtp_ring_append``); k_new, v_new are
    bf16 [B, n_new, Hkv, D]."""
    torch = _torch()
    B, n_new, Hkv, D = k_new.shape
    _need(k_new, torch.bfloat16, (ring.B, n_new, ring.Hkv, ring.D), "k_new")
    _need(v_new, torch.bfloat16, (ring.B, n_new, ring.Hkv, ring.D), "v_new")
    _need(ring.k, torch.bfloat16, k_cache_shape(B * ring.C // PAGE, Hkv, D), "ring.k")
    _need(ring.v, torch.bfloat16, v_cache_shape(B * ring.C // PAGE, Hkv, D), "ring.v")
    _need(ring.pos, torch.int32, (B, ring.C), "ring.pos")
    _need(ring.T, torch.int64, (B,), "ring.T")
    return _invoke("wmtp_ring_append", (_ptr(ring.k), _ptr(ring.v), _ptr(ring.pos), _ptr(ring.T),
                                        _ptr(k_new), _ptr(v_new), B, n_new, Hkv, D, ring.C,
                                        ring.n_sink, _stream(stream)), prepare)


def paged_append_fp8(k_cache, v_cache, block_table, start_pos, k_new, v_new, k_scale=1.0,
                     v_scale=1.0, stream=None, prepare=False):
    """Quantize ``n_new`` bf16 positions per sequence into fp8 caches
    (``wmtp_paged_append_fp8``)."""
    torch = _torch()
    B, n_new, Hkv, D = k_new.shape
    num_pages = k_cache.shape[0]
    max_pages = block_table.shape[1]
    _need(k_cache, torch.uint8, k_cache_shape(num_pages, Hkv, D), "k_cache")
    _need(v_cache, torch.uint8, v_cache_shape(num_pages, Hkv, D), "v_cache")
    _need(block_table, torch.int32, (B, max_pages), "block_table")
    _need(start_pos, torch.int32, (B,), "start_pos")
    _need(k_new, torch.bfloat16, (B, n_new, Hkv, D), "k_new")
    _need(v_new, torch.bfloat16, (B, n_new, Hkv, D), "v_new")
    return _invoke("wmtp_paged_append_fp8", (
        _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(start_pos), _ptr(k_new),
        _ptr(v_new), B, n_new, Hkv, D, num_pages, max_pages, float(k_scale), float(v_scale),
        _stream(stream)), prepare)


def draft_attn_full_fp8(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, k_scale=1.0,
                        v_scale=1.0, softmax_scale=1.0, o=None, lse=None, workspace=None,
                        num_splits=0, partials_only=False, stream=None, prepare=False,
                        window=None):
    """Native draft attention over fp8 caches (``wmtp_draft_attn_full_fp8``); with
    ``window=(n_sink, n_recent)`` the truncated paged index
    (``wmtp_draft_attn_window_paged_fp8``)."""
    torch = _torch()
    B, Hq, D = q.shape
    num_pages, Hkv = k_cache.shape[0], k_cache.shape[1]
    max_pages = block_table.shape[1]
    _need(q, torch.bfloat16, None, "q")
    _need(k_cache, torch.uint8, k_cache_shape(num_pages, Hkv, D), "k_cache")
    _need(v_cache, torch.uint8, v_cache_shape(num_pages, Hkv, D), "v_cache")
    _need(block_table, torch.int32, (B, max_pages), "block_table")
    _need(seq_lens, torch.int32, (B,), "seq_lens")
    if window is None:
        need = workspace_bytes(B, Hq, Hkv, D, 1, min(int(max_seq_len), max_pages * PAGE),
                               num_splits, partials_only, fp8=True)
    else:
        need = workspace_bytes(B, Hq, Hkv, D, 1, int(window[0]) + int(window[1]), num_splits,
                               partials_only, paged_window=True)
    if workspace is None:
        workspace = new_workspace(need, q.device)
    _need(workspace, torch.uint8, None, "workspace")
    if not partials_only:
        o, lse = _outputs(o, lse, (B, Hq, D), (B, Hq), q.device)
    head = (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(seq_lens),
            B, Hq, Hkv, D, num_pages, max_pages, int(max_seq_len))
    tail = (float(k_scale), float(v_scale), float(softmax_scale), _ptr(o), _ptr(lse),
            _ptr(workspace), workspace.numel(), int(num_splits),
            FLAG_PARTIALS_ONLY if partials_only else 0, _stream(stream))
    if window is None:
        c = _invoke("wmtp_draft_attn_full_fp8", head + tail, prepare)
    else:
        c = _invoke("wmtp_draft_attn_window_paged_fp8",
                    head + (int(window[0]), int(window[1])) + tail, prepare)
    if prepare:
        return c
    return workspace if partials_only else (o, lse)


def paged_append(k_cache, v_cache, block_table, start_pos, k_new, v_new, stream=None,
                 prepare=False):
    """Write ``n_new`` positions per sequence at ``start_pos`` (``wmtp_paged_append``)."""
    torch = _torch()
    B, n_new, Hkv, D = k_new.shape
    num_pages = k_cache.shape[0]
    max_pages = block_table.shape[1]
    _need(k_cache, torch.bfloat16, k_cache_shape(num_pages, Hkv, D), "k_cache")
    _need(v_cache, torch.bfloat16, v_cache_shape(num_pages, Hkv, D), "v_cache")
    _need(block_table, torch.int32, (B, max_pages), "block_table")
    _need(start_pos, torch.int32, (B,), "start_pos")
    _need(k_new, torch.bfloat16, (B, n_new, Hkv, D), "k_new")
    _need(v_new, torch.bfloat16, (B, n_new, Hkv, D), "v_new")
    return _invoke("wmtp_paged_append", (_ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                         _ptr(start_pos), _ptr(k_new), _ptr(v_new), B, n_new,
                                         Hkv, D, num_pages, max_pages, _stream(stream)), prepare)


def split_combine(part_o, part_lse, B, Hkv, G, n_q, split_indptr=None, splits_per_group=0,
                  o=None, lse=None, stream=None, prepare=False):
    """Log-sum-exp merge of partials (``wmtp_split_combine``)."""
    torch = _torch()
    P, R, D = part_o.shape
    if R != n_q * G:
        raise ValueError("part_o rows must be n_q * G")
    _need(part_o, torch.float32, None, "part_o")
    _need(part_lse, torch.float32, (P, R), "part_lse")
    if split_indptr is not None:
        _need(split_indptr, torch.int32, (B * Hkv + 1,), "split_indptr")
    elif B * Hkv * splits_per_group > P:
        raise ValueError("fewer partials than B * Hkv * splits_per_group")
    o, lse = _outputs(o, lse, (B, n_q, Hkv * G, D), (B, n_q, Hkv * G), part_o.device)
    c = _invoke("wmtp_split_combine", (_ptr(part_o), _ptr(part_lse), P, _ptr(split_indptr),
                                       int(splits_per_group), B, Hkv, G, n_q, D, _ptr(o),
                                       _ptr(lse), _stream(stream)), prepare)
    return c if prepare else (o, lse)
