"""Comparing a GPU chunk with the oracle's: selections and tolerances.

TEST INFRASTRUCTURE ONLY (like the rest of this package): numpy only; it
imports nothing of the GPU path.  Used by the tests and by the benchmark's
CPU-baseline leg, which report near-ties and errors with the same rules.

Selections.  Both sides rank candidates best first by (value, then lower
slot); the GPU ranks in fp32, the oracle in float64, so where the oracle's
k-th and (k+1)-th best values lie within 1e-6 relative of each other (a
near-tie) the GPU may legitimately pick either.  Only there may the sets
differ, and only as validate_adopted_selection allows; the oracle then
adopts the GPU's set for that token so the rest of the step stays
comparable.

Tolerances.  Per chunk, teacher-forced (both sides from the same fp32
state): rtol 1e-4 / atol 1e-5; after chained chunks: rtol 1e-3 / atol 1e-4.
"""

from __future__ import annotations

import numpy as np

from . import fwpkm_oracle as O

RTOL_CHUNK, ATOL_CHUNK = 1e-4, 1e-5
RTOL_CHAIN, ATOL_CHAIN = 1e-3, 1e-4


def _tie_window(x, y):
    """Z17's near-tie width around two values (relative 1e-6, floor 1)."""
    return O.NEAR_TIE_REL * max(abs(x), abs(y), 1.0)


# Exact-tie enumeration gives up beyond this many candidate slots per token
# (then only the symmetric difference is checked for exact ties).
_MAX_WINDOW_SLOTS = 1 << 20


def validate_adopted_selection(r, t, chosen, n):
    """Check that `chosen`, a selection the GPU made for token t where it
    differs from the oracle's, is one an fp32 ranking may legitimately make.

    r is the oracle's (non-overridden) UnitChunkResult of the unit.  Raises
    AssertionError unless
      * chosen holds k distinct slots in [0, n*n);
      * every slot in the symmetric difference with the oracle's set has an
        oracle value within the near-tie window of the k-th best value (a
        slot the GPU dropped was not clearly better, one it took was not
        clearly worse);
      * where float64 values tie exactly, the lower slot was taken: no chosen
        slot has a left-out slot of exactly its value and a lower index
        (ties by lower slot, as both sides order candidates).
    """
    k = r.slots.shape[1]
    N = n * n
    chosen = [int(s) for s in chosen]
    assert len(chosen) == k and len(set(chosen)) == k, (
        f"token {t}: GPU selection {chosen} is not {k} distinct slots")
    assert all(0 <= s < N for s in chosen), f"token {t}: GPU selection {chosen} leaves [0, {N})"
    v1, v2 = r.half_values
    sign = 1.0 if r.mode == O.IDW else -1.0          # order key: ascending is best first

    def value(s):
        return float(v1[t, s // n] + v2[t, s % n])

    d_k = float(r.values[t, k - 1])                  # the oracle's k-th best value
    mine, theirs = set(chosen), set(int(s) for s in r.slots[t])
    for s in sorted(mine ^ theirs):
        d = value(s)
        assert abs(d - d_k) <= _tie_window(d, d_k), (
            f"token {t}: slot {s} ({'taken' if s in mine else 'dropped'} by the GPU) has value "
            f"{d!r}, outside the near-tie window of the k-th best {d_k!r}")
    # slots whose value could lie within the window: per half, the sub-keys
    # that can still reach it with the other half's best value
    o1, o2 = sign * v1[t], sign * v2[t]
    lim = sign * d_k + _tie_window(d_k, d_k) * 1.000001
    A = np.flatnonzero(o1 + o2.min() <= lim)
    B = np.flatnonzero(o2 + o1.min() <= lim)
    if A.size * B.size <= _MAX_WINDOW_SLOTS:
        cand = (A[:, None] * n + B[None, :]).reshape(-1)
        cval = (v1[t, A][:, None] + v2[t, B][None, :]).reshape(-1)
    else:
        cand = np.asarray(sorted(mine ^ theirs), dtype=np.int64)
        cval = np.asarray([value(s) for s in cand])
    left_out = ~np.isin(cand, np.asarray(chosen))
    for s in chosen:
        d = value(s)
        lower = cand[left_out & (cval == d) & (cand < s)]
        assert lower.size == 0, (
            f"token {t}: GPU took slot {s} over slot {int(lower[0])} of exactly the same value "
            f"{d!r} (ties go to the lower slot)")


def selection_overrides(results, gpu_slots, H, units, n=None):
    """Compare slot sets; returns ({u: {t: gpu set}}, near-tie count).

    A set may differ from the oracle's only at a near-tie (k-th and (k+1)-th
    best within 1e-6 relative), and then only as validate_adopted_selection
    allows; the oracle then adopts the GPU's set for that token."""
    overrides, ties = {}, 0
    for u in units:
        b, h = divmod(u, H)
        r = results[u]
        nn = n if n is not None else r.half_values[0].shape[1]
        g = gpu_slots[b, :, h]
        for t in range(g.shape[0]):
            gs = sorted(int(s) for s in g[t])
            os_ = sorted(int(s) for s in r.slots[t])
            if gs != os_:
                assert r.near_tie[t], (
                    f"unit {u} token {t}: GPU slots {gs} != oracle {os_} without a near-tie "
                    f"(k-th {r.values[t, -1]!r}, (k+1)-th {r.value_k1[t]!r})")
                validate_adopted_selection(r, t, gs, nn)
                overrides.setdefault(u, {})[t] = gs
                ties += 1
    return overrides, ties


def error_stats(got, want, rtol, atol):
    """Worst errors of `got` against `want`: the largest |got - want| over
    (atol + rtol |want|) (at most 1 within tolerance), the largest absolute
    error, and the largest relative error over entries with |want| >= 1e-3."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    if got.size == 0:
        return {"tol_used": 0.0, "max_abs_err": 0.0, "max_rel_err": 0.0}
    err = np.abs(got - want)
    big = np.abs(want) >= 1e-3
    return {"tol_used": float((err / (atol + rtol * np.abs(want))).max()),
            "max_abs_err": float(err.max()),
            "max_rel_err": float((err[big] / np.abs(want[big])).max()) if big.any() else 0.0}
