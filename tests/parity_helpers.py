"""Shared pieces of the GPU parity tests: run a chunk through the C ABI and
compare it with the CPU oracle on the same seeded inputs.

Protocol per chunk (teacher-forced): both sides start from the same fp32
state.  Selected slots are compared as sets per (unit, token); a difference
is allowed only where the oracle reports a near-tie (k-th and (k+1)-th best
within 1e-6 relative), and the oracle then adopts the GPU's set for that
token so the rest stays comparable.  Retrieved vectors and updated tables
must then agree within rtol 1e-4 / atol 1e-5.
"""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from oracle import fwpkm_oracle as O

RTOL_CHUNK, ATOL_CHUNK = 1e-4, 1e-5
RTOL_CHAIN, ATOL_CHAIN = 1e-3, 1e-4


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def say(*msg):
    print("[parity]", *msg, flush=True)
    sys.stdout.flush()


def mode_name(mode):
    return O.IDW if mode == "idw" else O.DOT


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def state_to_dev(st, B, H):
    """Oracle-layout state {k1: [U, n, dh], ...} -> per-sequence device State."""
    from sparse_weight_memory_amd import State
    U, n, dh = st["k1"].shape
    N, dv = st["v"].shape[1:]
    return State(to_dev(st["k1"].reshape(B, H, n, dh)),
                 to_dev(st["k2"].reshape(B, H, n, dh)),
                 to_dev(st["v"].reshape(B, H, N, dv)))


def state_to_host(s, units=None):
    """Device State -> oracle layout, optionally only some units."""
    B, H = s.k1.shape[:2]
    out = {}
    for name in ("k1", "k2", "v"):
        t = getattr(s, name)
        flat = t.reshape(B * H, *t.shape[2:])
        if units is not None:
            flat = flat[torch.as_tensor(units, device=flat.device)]
        out[name] = flat.cpu().numpy()
    return out


def oracle_units(state, q, y, lr, k, eps, mode, units, H, overrides=None, tw=None, addr=0.0):
    """Run the oracle on the given units only (state holds those units, in order).
    tw: token weights [B, C, H] or None; addr: addressing-loss weight.

    Returns (retrieved {u: [C, d_v]}, new state (same unit order), results).
    """
    rets, results = {}, {}
    new = {name: a.copy() for name, a in state.items()}
    for i, u in enumerate(units):
        b, h = divmod(u, H)
        ov = overrides.get(u) if overrides else None
        r = O.unit_chunk(state["k1"][i], state["k2"][i], state["v"][i], q[b, :, h], y[b, :, h],
                         lr, k, eps, mode, ov, None if tw is None else tw[b, :, h], addr)
        rets[u] = r.retrieved
        results[u] = r
        if r.updates:
            O.apply_updates(new["k1"][i], new["k2"][i], new["v"][i], r.updates)
    return rets, new, results


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


def assert_close(name, got, want, rtol, atol):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    err = np.abs(got - want)
    bound = atol + rtol * np.abs(want)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(
            f"{name}: {int(bad.sum())} of {bad.size} entries out of tolerance; worst at {i}: "
            f"got {got[i]!r} want {want[i]!r} (rtol {rtol}, atol {atol})")


def compare_chunk(mem, st_host, q, y, lr, units=None, rtol=RTOL_CHUNK, atol=ATOL_CHUNK,
                  label="", tw=None):
    """Teacher-forced parity of one chunk starting from st_host (all units);
    tw = token weights [B, C, H] (numpy) or None.

    Returns (oracle next state for `units`, near-tie count, GPU next State).
    """
    cfg = mem.cfg
    B, C, H = q.shape[0], q.shape[1], cfg.num_heads
    U = B * H
    units = list(range(U)) if units is None else list(units)
    dev_state = state_to_dev(st_host, B, H)
    qd, yd = to_dev(q), to_dev(y)
    say(label, "gpu chunk", dict(B=B, C=C, H=H, n=cfg.sqrt_slots, k=cfg.topk, lr=lr))
    ret, nxt, slots, weights = mem.forward_chunk(qd, yd, lr, dev_state, next=dev_state,
                                                 return_selection=True,
                                                 token_weights=None if tw is None else to_dev(tw))
    torch.cuda.synchronize()
    ret = ret.cpu().numpy()
    slots = slots.cpu().numpy()
    weights = weights.cpu().numpy()
    sub = {name: a[units] for name, a in st_host.items()}
    mode = mode_name(cfg.score_mode)
    say(label, "oracle on units", units[:8], "..." if len(units) > 8 else "")
    addr = getattr(cfg, "addr_weight", 0.0)
    rets, new, results = oracle_units(sub, q, y, lr, cfg.topk, cfg.eps, mode, units, H, tw=tw, addr=addr)
    overrides, ties = selection_overrides(results, slots, H, units)
    if overrides:
        rets, new, results = oracle_units(sub, q, y, lr, cfg.topk, cfg.eps, mode, units, H,
                                          overrides, tw=tw, addr=addr)
    for u in units:
        b, h = divmod(u, H)
        assert_close(f"{label} retrieved u{u}", ret[b, :, h], rets[u], rtol, atol)
        # weights, matched slot by slot
        r = results[u]
        go = np.argsort(slots[b, :, h], axis=1)
        oo = np.argsort(r.slots, axis=1)
        assert (np.take_along_axis(slots[b, :, h], go, 1) ==
                np.take_along_axis(r.slots, oo, 1)).all()
        assert_close(f"{label} weights u{u}", np.take_along_axis(weights[b, :, h], go, 1),
                     np.take_along_axis(r.weights, oo, 1), rtol, atol)
    got = state_to_host(nxt, units)
    for name in ("k1", "k2", "v"):
        assert_close(f"{label} next {name}", got[name], new[name], rtol, atol)
    return new, ties, nxt
