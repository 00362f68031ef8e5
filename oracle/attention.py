"""Plain float64 attention: the definition every GPU attention result must match.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the method computes.  The pages fix *which keys* each query reads, not a
new attention formula: the draft head's query attends over the draft KV
([ABSTRACT]; [VERDICT] key machinery), the windowed draft reads only the first
``n_sink`` positions plus the most recent ones ([VERDICT] key machinery; the
StreamingLLM sink-plus-window primitive named in [NOTES] and [ABSTRACT]), and the
target verifies the proposed positions with full attention over its own KV
([ABSTRACT]; [VERDICT] key machinery, where the verify term is untouched).  So the
oracle is ordinary scaled-dot-product softmax attention written out over an
explicit key set J:

    s_j = scale * sum_c q[c] * K[j, c]          (j in J)
    m   = max_j s_j
    w_j = exp(s_j - m)
    l   = sum_j w_j
    o   = sum_j w_j V[j, :] / l
    lse = m + ln(l)

computed in two passes (all logits first, then the max-subtracted exponentials),
which deliberately differs from the GPU's one-pass online softmax.

Readings taken where the pages are silent (each listed in the design notes):

* bf16 inputs are widened exactly to float64 before any arithmetic;
* grouped-query attention maps query head ``h`` to KV head ``h // G`` with
  ``G = Hq // Hkv``;
* the window is ``[0, min(n_sink, L)) U [max(n_sink, L - n_recent), L)``: the
  recent part includes the position just appended, and the two parts are joined
  without counting a key twice;
* draft step ``j`` (1-based) of a chain of gamma steps attends ``L = S + j``
  keys (the position appended at that step included);
* verify query ``i`` of ``n_q`` (0-based) sees the first ``L - n_q + i + 1``
  keys, where ``L`` already counts the ``n_q`` appended positions;
* the draft context pass (the draft head over the accepted positions, the
  draft-context term of the step cost in [VERDICT] referee report, major
  comment on Eq. 1) is causal like the verify: its query ``i`` sits at position
  ``L - n_q + i``; natively it reads every earlier draft key, windowed it reads
  the window of its own position, ``window_positions(L - n_q + i + 1, ...)``;
* ``lse`` is the natural-log log-sum-exp of the scaled logits.
"""

from __future__ import annotations

import numpy as np


def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly.

    A bf16 value is the upper half of an IEEE float32, so shifting the 16 bits
    into the high half of a 32-bit word and reading it as float32 is exact, and
    float32 -> float64 is exact too.
    """
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError("widen_bf16 expects uint16 bf16 bit patterns")
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def as_f64(x: np.ndarray) -> np.ndarray:
    """uint16 arrays are bf16 bit patterns and are widened; anything else is cast."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return widen_bf16(x)
    return x.astype(np.float64)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Softmax attention of query rows ``q`` [R, D] over keys ``K`` [N, D], values ``V`` [N, Dv].

    Returns ``(o [R, Dv], lse [R])`` in float64.  An empty key set (N == 0) has no
    defined output; it returns ``o = 0`` and ``lse = -inf`` (the identity element of
    the split combine).
    """
    q = as_f64(q)
    K = as_f64(K)
    V = as_f64(V)
    R = q.shape[0]
    if K.shape[0] == 0:
        return np.zeros((R, V.shape[1])), np.full(R, -np.inf)
    # pass 1: every logit, then the row maximum
    logits = float(scale) * (q @ K.T)                 # [R, N]
    m = logits.max(axis=1, keepdims=True)              # [R, 1]
    # pass 2: max-subtracted exponentials, their sum, the weighted value sum
    w = np.exp(logits - m)                             # [R, N]
    l = w.sum(axis=1, keepdims=True)                   # [R, 1]
    o = (w @ V) / l                                    # [R, Dv]
    lse = (m + np.log(l))[:, 0]
    return o, lse


def window_positions(L: int, n_sink: int, n_recent: int) -> np.ndarray:
    """Key positions the windowed draft reads at context length ``L``.

    [VERDICT] key machinery: the draft's per-request KV index keeps the first
    ``n_sink`` tokens and the last window of tokens.  Reading: the window is given
    as two counts, ``n_sink`` and ``n_recent`` (the pages' "4K" window is their sum,
    4 + 4092), the recent part ends at the newest position, and overlapping parts
    are joined without repeats.
    """
    if L < 0 or n_sink < 0 or n_recent < 0:
        raise ValueError("negative size")
    sink = np.arange(0, min(n_sink, L))
    recent = np.arange(max(n_sink, L - n_recent), L)
    return np.concatenate([sink, recent]).astype(np.int64)


def _group_rows(Hq: int, Hkv: int):
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    return G, [(g, np.arange(g * G, (g + 1) * G)) for g in range(Hkv)]


def draft_over(q, K, V, positions, scale):
    """One draft query per head over an explicit key-position list.

    q [Hq, D]; K, V [L_total, Hkv, D] (position-major, logical order);
    positions: int array of key positions.  Returns (o [Hq, D], lse [Hq]).
    """
    q = np.asarray(q)
    Hq, D = q.shape
    Hkv = K.shape[1]
    G, groups = _group_rows(Hq, Hkv)
    o = np.zeros((Hq, V.shape[2]))
    lse = np.zeros(Hq)
    pos = np.asarray(positions, dtype=np.int64)
    for g, heads in groups:
        Kg = K[pos, g, :]
        Vg = V[pos, g, :]
        o[heads], lse[heads] = attend(q[heads], Kg, Vg, scale)
    return o, lse


def draft_full(q, K, V, L: int, scale: float):
    """Native draft: the draft head's query reads every one of the ``L`` cached keys.

    [ABSTRACT]: a native MTP draft head runs full attention over the whole KV
    cache at every draft step, a read that grows linearly with context.
    """
    return draft_over(q, K, V, np.arange(L), scale)


def draft_window(q, K, V, L: int, n_sink: int, n_recent: int, scale: float):
    """Windowed draft: the same attention restricted to ``window_positions(L, ...)``.

    [VERDICT] key machinery; [ABSTRACT] (sliding window plus attention sink on the
    draft only).  Positions are the absolute ones; because the cached keys already
    carry their rotary positions ([VERDICT] key machinery), which slot a key sits
    in does not change its score, so reading the window in ring-slot order gives
    the same result as reading it in position order.
    """
    return draft_over(q, K, V, window_positions(L, n_sink, n_recent), scale)


def verify(q, K, V, L: int, scale: float):
    """Full-context causal verify of ``n_q`` proposed positions.

    q [n_q, Hq, D]; K, V [>= L, Hkv, D]; ``L`` counts the ``n_q`` appended positions.
    Query ``i`` sees keys ``[0, L - n_q + i + 1)``.  [ABSTRACT]: verification keeps
    full attention; [VERDICT] key machinery: the verify term of the step cost is
    untouched by the window.  Returns (o [n_q, Hq, D], lse [n_q, Hq]).
    """
    q = np.asarray(q)
    n_q = q.shape[0]
    if L < n_q:
        raise ValueError("L must count the n_q appended positions")
    o = np.zeros(q.shape[:2] + (V.shape[2],))
    lse = np.zeros(q.shape[:2])
    for i in range(n_q):
        o[i], lse[i] = draft_over(q[i], K, V, np.arange(L - n_q + i + 1), scale)
    return o, lse


def verify_tree(q, K, V, L: int, masks, scale: float):
    """Verify of a tree of ``n_q`` proposals ([VERDICT] forward implications: the
    window composes with tree-shaped speculation).

    q [n_q, Hq, D]; K, V [>= L, Hkv, D]; ``L`` counts the ``n_q`` appended positions;
    ``masks[i]`` (an int) has bit ``a`` set when query ``i`` sees the appended
    position ``L - n_q + a`` (its ancestors and itself).  Every query sees all keys
    before the appended ones.  Returns (o [n_q, Hq, D], lse [n_q, Hq]); a query
    with no key gets o = 0, lse = -inf.
    """
    q = np.asarray(q)
    n_q = q.shape[0]
    if L < n_q:
        raise ValueError("L must count the n_q appended positions")
    base = L - n_q
    o = np.zeros(q.shape[:2] + (V.shape[2],))
    lse = np.zeros(q.shape[:2])
    for i in range(n_q):
        seen = [base + a for a in range(n_q) if (int(masks[i]) >> a) & 1]
        o[i], lse[i] = draft_over(q[i], K, V, np.concatenate([np.arange(base), seen]).astype(np.int64),
                                  scale)
    return o, lse


def draft_context_window(q, K, V, L: int, n_sink: int, n_recent: int, scale: float):
    """Windowed draft context pass: ``n_q`` causal queries over the draft KV, query
    ``i`` (position ``L - n_q + i``) over the window of its own position.

    q [n_q, Hq, D]; K, V [>= L, Hkv, D].  The native form is ``verify`` over the
    draft KV.  Returns (o [n_q, Hq, D], lse [n_q, Hq]).
    """
    q = np.asarray(q)
    n_q = q.shape[0]
    if L < n_q:
        raise ValueError("L must count the n_q positions of the pass")
    o = np.zeros(q.shape[:2] + (V.shape[2],))
    lse = np.zeros(q.shape[:2])
    for i in range(n_q):
        o[i], lse[i] = draft_window(q[i], K, V, L - n_q + i + 1, n_sink, n_recent, scale)
    return o, lse


def combine(part_o: np.ndarray, part_lse: np.ndarray):
    """Merge attention results over disjoint key subsets (log-sum-exp combine).

    part_o [N, R, D] holds each subset's normalised output, part_lse [N, R] its
    log-sum-exp (``-inf`` for an empty subset).  The result equals attention over
    the union of the subsets:

        lse = ln sum_s exp(lse_s),   o = sum_s exp(lse_s - lse) * o_s.

    This identity is not on the pages; it is how a split over the key axis is put
    back together, and the tests check it against attention over the union.
    """
    part_o = np.asarray(part_o, dtype=np.float64)
    part_lse = np.asarray(part_lse, dtype=np.float64)
    M = part_lse.max(axis=0)                                 # [R]
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(part_lse), np.exp(part_lse - Ms), 0.0)   # [N, R]
    tot = w.sum(axis=0)                                      # [R]
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.einsum("nr,nrd->rd", w, part_o) / np.where(tot > 0, tot, 1.0)[:, None]
        lse = np.where(finite, Ms + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    o[~finite] = 0.0
    return o, lse
