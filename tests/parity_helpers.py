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
from oracle.compare import (ATOL_CHAIN, ATOL_CHUNK, RTOL_CHAIN, RTOL_CHUNK,  # noqa: F401
                            error_stats, selection_overrides, validate_adopted_selection)


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


def mirror_units(dev_state, units):
    """Host copy (oracle layout, float32) of some units' tables on the GPU."""
    return state_to_host(dev_state, units)


def teacher_forced_step(mem, dev_state, mirror, units, q, y, lr, label="", tw=None):
    """One chunk on the GPU (every unit, in place, the launch the benchmark
    times) checked against the oracle on sampled units, teacher-forced: the
    oracle starts from `mirror`, a host copy of those units' tables equal to
    the GPU's before the chunk, and afterwards `mirror` is brought to the
    GPU's new state (sub-key tables copied whole, value rows at the slots the
    GPU selected: the only rows it writes).

    q, y [B, C, H, d] numpy.  Returns (near-ties, error stats dict)."""
    cfg = mem.cfg
    H = cfg.num_heads
    say(label, "gpu chunk (in place)")
    ret, _, slots, weights = mem.forward_chunk(to_dev(q), to_dev(y), lr, dev_state, next=dev_state,
                                               return_selection=True,
                                               token_weights=None if tw is None else to_dev(tw))
    torch.cuda.synchronize()
    ret = ret.cpu().numpy()
    slots_h = slots.cpu().numpy()
    weights_h = weights.cpu().numpy()
    mode = mode_name(cfg.score_mode)
    addr = getattr(cfg, "addr_weight", 0.0)
    rets, new, results = oracle_units(mirror, q, y, lr, cfg.topk, cfg.eps, mode, units, H, tw=tw,
                                      addr=addr)
    overrides, ties = selection_overrides(results, slots_h, H, units)
    if overrides:
        rets, new, results = oracle_units(mirror, q, y, lr, cfg.topk, cfg.eps, mode, units, H,
                                          overrides, tw=tw, addr=addr)
    worst = {"retrieved": 0.0, "weights": 0.0, "k1": 0.0, "k2": 0.0, "v": 0.0}
    for i, u in enumerate(units):
        b, h = divmod(u, H)
        assert_close(f"{label} retrieved u{u}", ret[b, :, h], rets[u], RTOL_CHUNK, ATOL_CHUNK)
        worst["retrieved"] = max(worst["retrieved"],
                                 error_stats(ret[b, :, h], rets[u], RTOL_CHUNK, ATOL_CHUNK)["tol_used"])
        r = results[u]
        go = np.argsort(slots_h[b, :, h], axis=1)
        oo = np.argsort(r.slots, axis=1)
        assert (np.take_along_axis(slots_h[b, :, h], go, 1) == np.take_along_axis(r.slots, oo, 1)).all()
        gw = np.take_along_axis(weights_h[b, :, h], go, 1)
        ow = np.take_along_axis(r.weights, oo, 1)
        assert_close(f"{label} weights u{u}", gw, ow, RTOL_CHUNK, ATOL_CHUNK)
        worst["weights"] = max(worst["weights"], error_stats(gw, ow, RTOL_CHUNK, ATOL_CHUNK)["tol_used"])
        if lr == 0.0:
            continue
        # sub-key tables whole; value rows where either side wrote
        for name in ("k1", "k2"):
            got = getattr(dev_state, name)[b, h].cpu().numpy()
            assert_close(f"{label} next {name} u{u}", got, new[name][i], RTOL_CHUNK, ATOL_CHUNK)
            worst[name] = max(worst[name], error_stats(got, new[name][i], RTOL_CHUNK, ATOL_CHUNK)["tol_used"])
            mirror[name][i] = got
        gpu_rows = np.unique(slots_h[b, :, h])
        rows = np.union1d(gpu_rows, r.updates["v"][0] if r.updates else gpu_rows)
        idx = torch.as_tensor(rows, device=dev_state.v.device, dtype=torch.long)
        got = dev_state.v[b, h].index_select(0, idx).cpu().numpy()
        assert_close(f"{label} next v u{u}", got, new["v"][i][rows], RTOL_CHUNK, ATOL_CHUNK)
        worst["v"] = max(worst["v"], error_stats(got, new["v"][i][rows], RTOL_CHUNK, ATOL_CHUNK)["tol_used"])
        mirror["v"][i][rows] = got
    return ties, worst
