"""Step-cost identity and KV accounting (closed forms).

TEST INFRASTRUCTURE ONLY (see the package docstring).

* Eq. 1 ([VERDICT] key machinery; referee major comment on App. B / Eq. 1): a
  decode step costs ``t_step = t_verify + t_ctx_draft + gamma * t_fwd_draft``;
  the two draft terms grow with context in the native arm and with the window in
  the windowed arm, while the verify term is the same in both.
* Eq. 3 ([VERDICT] referee minor comment on Eq. 3 / Table 1; [ABSTRACT]): per-token
  latency is step cost divided by acceptance length, so
  ``win/native = (step_native / step_window) * (AL_window / AL_native)``.
* [ABSTRACT]: the window drops about 99 % of KV entries at 1M context and the
  unread draft KV, 7.7-11 % of all KV at 1M, is reclaimed by the ring.

Readings: the pages print the per-step gain as "+28 % to +44 %" next to the verb
"cuts"; both ``t_native / t_window - 1`` and ``1 - t_window / t_native`` are
returned.  The reclaimed fraction counts one native draft-KV pool of ``T_draft``
positions beside ``n_layers`` target attention layers of ``T_target`` positions,
all with the same per-position KV size; the window keeps ``C`` ring slots.
"""

from __future__ import annotations


def step_cost(t_verify: float, t_ctx_draft: float, t_fwd_draft: float, gamma: int) -> float:
    """Eq. 1: t_step = t_verify + t_ctx_draft + gamma * t_fwd_draft."""
    if gamma < 0:
        raise ValueError("gamma must be >= 0")
    return t_verify + t_ctx_draft + gamma * t_fwd_draft


def cost_reduction(t_native: float, t_window: float):
    """Both readings of the per-step gain: (t_native/t_window - 1, 1 - t_window/t_native)."""
    if t_native <= 0 or t_window <= 0:
        raise ValueError("step times must be positive")
    return t_native / t_window - 1.0, 1.0 - t_window / t_native


def latency_ratio(step_native: float, step_window: float, al_native: float, al_window: float) -> float:
    """Eq. 3: win/native = (step_native / step_window) * (AL_window / AL_native)."""
    return (step_native / step_window) * (al_window / al_native)


def dropped_fraction(L: int, window: int) -> float:
    """Fraction of the L cached KV entries the windowed draft does not read."""
    if L <= 0:
        raise ValueError("L must be positive")
    return 1.0 - min(window, L) / L


def reclaimed_fraction(T_draft: int, C: int, n_layers: int, T_target: int) -> float:
    """Share of all KV freed when the native draft pool of ``T_draft`` positions
    shrinks to a ``C``-slot ring, next to ``n_layers`` target layers of ``T_target``."""
    total = n_layers * T_target + T_draft
    return (T_draft - min(C, T_draft)) / total


def kv_bytes(L: int, Hkv: int, D: int, elem_bytes: int = 2) -> int:
    """Bytes of K plus V for ``L`` positions of ``Hkv`` heads of width ``D``."""
    return 2 * L * Hkv * D * elem_bytes
