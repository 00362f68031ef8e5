"""Draft-KV ring buffer: slot mapping and state after appends (pure Python).

TEST INFRASTRUCTURE ONLY (see the package docstring).

[VERDICT] referee minor comment on the App. A pseudocode: the windowed draft's KV
lives in a compact per-request ring, addressed as ``slot = ring_base(r) +
logical_pos``, with ``d`` slots of slack; the reviewer notes that the wrap rule and
the use of the slack are left unexplained.  [ABSTRACT]: the draft KV that the
window never reads is reclaimed by this ring.

Readings taken (the pages give the formula, not the wrap rule):

* a ring of capacity ``C`` keeps the ``n_sink`` sink positions in slots
  ``0 .. n_sink-1`` for good, and cycles every later position through the other
  ``C - n_sink`` slots:

      logical_pos(p) = p                                   if p < n_sink
                     = n_sink + (p - n_sink) mod (C - n_sink)  otherwise

  and ``ring_base(r) = r * C`` for request ``r``;
* the slack is capacity beyond ``n_sink + n_recent``: the window still reads only
  the last ``n_recent`` positions, so speculative positions that get rolled back
  never displace a position the window still needs.  The workloads here use no
  slack (``C = n_sink + n_recent``), where every filled slot is in the window;
* a slot never written holds position -1.
"""

from __future__ import annotations


def logical_pos(p: int, n_sink: int, C: int) -> int:
    """Ring-relative slot of absolute position ``p`` (reading above)."""
    if p < 0:
        raise ValueError("position must be >= 0")
    if not (0 <= n_sink < C):
        raise ValueError("need 0 <= n_sink < C")
    if p < n_sink:
        return p
    return n_sink + (p - n_sink) % (C - n_sink)


def slot(r: int, p: int, n_sink: int, C: int) -> int:
    """Global slot of position ``p`` of request ``r``: ring_base(r) + logical_pos(p)."""
    return r * C + logical_pos(p, n_sink, C)


class RingModel:
    """Step-by-step model of a batch of rings.

    ``pos[r][s]`` is the absolute position whose K/V sits in slot ``s`` of ring ``r``
    (-1 if never written); ``T[r]`` counts the positions appended so far.  The model
    stores positions only: the K/V payload of slot ``s`` is, by construction, the
    K/V of position ``pos[r][s]``.
    """

    def __init__(self, batch: int, C: int, n_sink: int):
        if not (0 <= n_sink < C):
            raise ValueError("need 0 <= n_sink < C")
        self.C = C
        self.n_sink = n_sink
        self.pos = [[-1] * C for _ in range(batch)]
        self.T = [0] * batch

    def append(self, r: int, n_new: int = 1) -> list:
        """Append positions ``T[r] .. T[r]+n_new-1`` to ring ``r`` one at a time.

        Returns the ring-relative slots written, in order.
        """
        written = []
        for _ in range(n_new):
            p = self.T[r]
            s = logical_pos(p, self.n_sink, self.C)
            self.pos[r][s] = p
            self.T[r] = p + 1
            written.append(s)
        return written

    def rollback(self, r: int, new_T: int) -> None:
        """Forget positions ``>= new_T`` (rejected speculative drafts).

        Only the count moves back; slots that held a forgotten position keep it and
        are excluded by :func:`window_valid` because their position is ``>= T``.
        """
        if not (0 <= new_T <= self.T[r]):
            raise ValueError("rollback target out of range")
        self.T[r] = new_T


def expected_pos_after(T: int, n_sink: int, C: int) -> list:
    """Closed form of a fresh ring's contents after ``T`` appends.

    Slot ``s`` holds the largest ``p < T`` with ``logical_pos(p) == s``, else -1.
    Written independently of :class:`RingModel` so that the two check each other.
    """
    out = [-1] * C
    for s in range(min(n_sink, T)):
        out[s] = s
    M = C - n_sink
    if T > n_sink:
        for s in range(n_sink, C):
            k = s - n_sink                      # residue class of (p - n_sink) mod M
            last = T - 1 - n_sink               # largest (p - n_sink)
            if last < k:
                continue
            out[s] = n_sink + last - ((last - k) % M)
    return out


def window_valid(pos: list, T: int, n_sink: int, n_recent: int) -> list:
    """Which slots the windowed draft reads: a filled slot whose position is a sink
    position or one of the last ``n_recent`` positions before ``T``."""
    return [0 <= p < T and (p < n_sink or p >= T - n_recent) for p in pos]
