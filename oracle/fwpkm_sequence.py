"""Sequence-level FwPKM layer, written out plainly in float64 on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring); it builds on the chunk
oracle in fwpkm_oracle and shares nothing with the GPU path.

What is computed for a batch of token sequences x [B, S, D] with H memory
heads, D = H * d_v (the memory's value width per head times the heads is
the model width):

  P1  per token, queries and values are linear projections of the token
      [PyPI page "fast-weight-product-key-memory", Usage: the module takes
      model-width tokens (dim 512) and has its own query/key and value
      widths; gist.science "Fast-weight Product Key Memory", section 2, Core
      Architecture: the target value comes from the input stream]:
        [q_t | v_t] = W_in x_t,  W_in [H*d_qk + H*d_v, D], rows ordered
        (queries of head 0, ..., head H-1, values of head 0, ..., H-1);
      both are rounded to fp32, the precision the memory step consumes.
  P2  lookahead targets: query q_t is paired with v_{t+1} [gist.science
      section 2, Key Technical Choices: Lookahead Targets]; the last token of
      a sequence has no successor, so it reads but does not write: token
      weight 0 (with a zero target), all other tokens weight 1.
  P3  the sequence is cut into chunks of C tokens (the last may be shorter);
      each chunk reads with the fast weights left by the chunks before it and
      then takes its own write step [gist.science section 2, Causality
      Preservation; PyPI page, Usage: memories are chained from one call to
      the next] -- the chunk step of fwpkm_oracle.forward_chunk.
  P4  a gate per token and head, g_t = sigmoid(w_gate[h] . x_t + b_gate[h]),
      interpolates between the memory read and the residual path
      [gist.science section 2, Core Architecture: Gated Residual Output;
      agifrontier tutorial, gating: a gate value decides between slow-weight
      knowledge and the fast-weight memory]:
        out_t[head h slice] = g * r_t[h] + (1 - g) * x_t[head h slice].

Readings: the pages name the gate and the lookahead pairing but give neither
the gate's input and form nor how the projections are shaped; the plainest
forms above are taken (one linear map per output, a sigmoid gate on the
token, a convex mix with the token itself).  No page prints a value that
pins them: parity unpinned for these choices; the composition is pinned by
closed forms and invariants in the tests.
"""

from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from .fwpkm_oracle import IDW, forward_chunk


def project(x: np.ndarray, w_in: np.ndarray, H: int, dqk: int, dv: int):
    """P1: queries [B, S, H, d_qk] and values [B, S, H, d_v], float64 products
    of the fp32 inputs, each rounded to fp32."""
    B, S, D = x.shape
    assert w_in.shape == (H * dqk + H * dv, D)
    p = np.einsum("bsd,nd->bsn", x.astype(np.float64), w_in.astype(np.float64))
    q = p[..., :H * dqk].reshape(B, S, H, dqk).astype(np.float32)
    v = p[..., H * dqk:].reshape(B, S, H, dv).astype(np.float32)
    return q, v


def lookahead(v: np.ndarray):
    """P2: targets y_t = v_{t+1} (zero for the last token) and token weights
    (1, with 0 on the last token)."""
    B, S, H, dv = v.shape
    y = np.zeros_like(v)
    y[:, :S - 1] = v[:, 1:]
    tw = np.ones((B, S, H), np.float32)
    tw[:, S - 1] = 0.0
    return y, tw


def gate(x: np.ndarray, w_gate: np.ndarray, b_gate: Optional[np.ndarray]) -> np.ndarray:
    """P4: g [B, S, H] = sigmoid(w_gate[h] . x_t + b_gate[h]), float64."""
    z = np.einsum("bsd,hd->bsh", x.astype(np.float64), w_gate.astype(np.float64))
    if b_gate is not None:
        z = z + b_gate.astype(np.float64)
    # sigmoid, with exp of a non-positive argument only
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def forward_sequence(state: dict, x: np.ndarray, w_in: np.ndarray, w_gate: np.ndarray,
                     b_gate: Optional[np.ndarray], lr: float, k: int, chunk: int,
                     eps: float = 1e-3, mode: str = IDW,
                     overrides: Optional[Dict[int, Dict[int, Dict[int, Sequence[int]]]]] = None,
                     addr_weight: float = 0.0):
    """P1-P4 over whole sequences.

    state: per-unit tables as in fwpkm_oracle.forward_chunk (unit u = b*H + h),
    advanced through every chunk (a new dict; the input is left as it was).
    overrides: {chunk index: {unit: {token in chunk: slot set}}}.
    Returns (out [B, S, D] float64, final state, [per-chunk unit results]).
    """
    B, S, D = x.shape
    U, n, dh = state["k1"].shape
    H = U // B
    dv = state["v"].shape[2]
    assert U == B * H and D == H * dv
    q, v = project(x, w_in, H, 2 * dh, dv)
    y, tw = lookahead(v)
    st = {key: val.copy() for key, val in state.items()}
    r = np.zeros((B, S, H, dv), np.float64)
    results = []
    for c, c0 in enumerate(range(0, S, chunk)):
        c1 = min(S, c0 + chunk)
        ov = overrides.get(c) if overrides else None
        ret, st, res = forward_chunk(st, q[:, c0:c1], y[:, c0:c1], lr, k, eps, mode, ov,
                                     inplace=True, token_weights=tw[:, c0:c1],
                                     addr_weight=addr_weight)
        r[:, c0:c1] = ret
        results.append(res)
    g = gate(x, w_gate, b_gate)[..., None]
    out = g * r + (1.0 - g) * x.astype(np.float64).reshape(B, S, H, dv)
    return out.reshape(B, S, D), st, results
