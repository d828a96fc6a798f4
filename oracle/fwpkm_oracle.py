"""FwPKM chunk step, written out plainly in float64 on the CPU.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  The GPU path never
imports this module; the two share nothing but the seeded inputs.

What is computed, per memory unit (one sequence x one head) and per chunk of
C tokens, with fast weights theta = (K1, K2, V):

Read (product-key top-k memory)
  R1  split each query q into q1 (first half) and q2 (second half)
      [agifrontier tutorial "Fast-weight Product Key Memory", section on
      efficient addressing (Product Key): the query is split into two
      sub-queries searched against two smaller sub-key matrices];
  R2  d1[i] = ||q1 - K1[i]||^2, d2[j] = ||q2 - K2[j]||^2: the IDW distance
      of the full key [K1[i]; K2[j]] splits into the two halves
      [gist.science "Fast-weight Product Key Memory", section 2,
      Key Technical Choices: IDW score -log(eps + ||q - K||^2) instead of a
      dot product];
  R3  per half, the k best sub-keys;
  R4  over the k x k Cartesian candidates, the k best slots, slot = a*n + b
      [same summary, section 2, Core Architecture: two codebooks K(1), K(2),
      top-k of about 10^6 slots with O(sqrt(N)) scoring; repo-explainer
      "FwPKM: The Memory Layer That Writes Back", section "Product keys give
      the model a huge address space"];
  R5  w = softmax(s) over the k selected scores s_m = -log(eps + D_m)
      [sciencestack.ai "Fast-weight Product Key Memory", contents entry
      "Top-k Key-value Memory"];
  R6  out_t = sum_m w_m V[slot_m]  (the retrieved vector).

Write (one local gradient step, applied after the chunk's read)
  W1  g_t = out_t - y_t with L = sum_t 1/2 ||out_t - y_t||^2
      [sciencestack.ai contents: "MSE loss", "Reducing MSE losses to a
      scalar by summation"; gist.science section 2: reconstruction (MSE)
      loss between the retrieved value and a target];
  W2  per-token gradients at the chunk's starting weights, with the top-k
      selection held fixed (it is piecewise constant):
        dL_t/dV[slot_m]  = w_m g_t                 ("weighting gradient by
                                                     row contribution")
        delta_m          = dL_t/ds_m = w_m (g_t.V[slot_m] - g_t.out_t)
        dL_t/dK1[a]      = sum_{m: a_m = a} 2 delta_m (q1 - K1[a]) / (eps + D_m)
        dL_t/dK2[b]      likewise with q2;
  W3  a row touched by several tokens of the chunk gets the mean of their
      gradients: the sum over tokens divided by the number of tokens that
      touched it [gist.science section 2, Key Technical Choices: gradient
      aggregation by averaging];
  W4  theta_r <- fp32(theta_r - eta * mean gradient), for all touched rows at
      once; no clipping, momentum or decay [agifrontier tutorial:
      theta' = theta - eta grad L_MSE; sciencestack.ai contents: "No gradient
      clipping"].  eta = 0 leaves the state untouched.
The next chunk reads the new weights [gist.science section 2, Causality
Preservation: updates applied after the chunk; predictions inside a chunk use
only earlier chunks' fast weights].

Token importance (optional) [sciencestack.ai contents: "Weighting MSE loss by
token importance"; how the weights are produced is not on the pages]: with
per-token weights lambda_t the loss is L = sum_t lambda_t/2 ||out_t - y_t||^2,
so every gradient of token t is scaled by lambda_t (g_t -> lambda_t g_t), and
a token with lambda_t = 0 reads but does not write: it is left out of the row
sums and of the token counts W3 divides by (a masked token, such as the last
one of a sequence, which has no lookahead target).  All weights 1 is the
unweighted step.

Addressing loss (optional) [gist.science section 2, Core Architecture: an
auxiliary loss based on negative entropy, applied to the key matrices, keeps
slot usage balanced across a chunk; sciencestack.ai contents: "Addressing
Optimization", "Marginal entropy loss"; repo-explainer: marginal entropy
pressure against falling back to the same few addresses].  Reading taken
(the pages give no formula): per half h, P_h[t, :] = softmax over all n
sub-keys of the token's scores s_h[t, i] (the same scores R3 ranks), the
chunk's marginal p_h = (1/C) sum_t P_h[t, :], and
  L_addr = lambda_addr * sum_h sum_i p_h[i] log p_h[i]   (negative entropy).
Its gradient reaches every sub-key (not only the selected ones), at the
chunk's starting weights, and joins the same SGD step:
  K_h[i] <- fp32(K_h[i] - eta * (mean MSE gradient of row i, if touched,
                                  + dL_addr/dK_h[i])).
lambda_addr = 0 (default) is the step without it.

Dot-product scoring, the standard-PKM alternative the summary contrasts IDW
with, is also provided: s = q1.K1[a] + q2.K2[b], best = largest, and
ds/dK1[a] = q1.

Ordering and ties: best-first by (distance ascending, index ascending) for
IDW, (score descending, index ascending) for dot product, both per half and
for slots.

Readings of points the pages leave open (each discussed in the design notes):
the IDW formula is applied to the concatenated key (D = d1 + d2); eps = 1e-3
by default; averaging divides by the count of distinct tokens that touched a
row (for K rows: candidates of one token sharing a row are summed first);
targets arrive already aligned with the queries.  No page prints a number
that separates these readings from their alternatives: parity unpinned for
those choices (the functions themselves are pinned by brute force, closed
forms and finite differences in the tests).

Arithmetic is float64; tables are stored in fp32 and each updated entry is
rounded to fp32 once.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Sequence

import numpy as np

IDW = "idw"
DOT = "dot"

# Two candidates whose distances differ by at most this (relative) are a
# near-tie: an fp32 implementation may order them either way.
NEAR_TIE_REL = 1e-6


# --------------------------------------------------------------------- read


def split_query(q: np.ndarray, half: int):
    """R1: q -> (first half, second half)."""
    return q[..., :half], q[..., half:]


def sq_distances(x: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """R2: [T, n] matrix of ||x_t - keys_i||^2, from the difference, float64."""
    x = np.asarray(x, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    out = np.empty((x.shape[0], keys.shape[0]), dtype=np.float64)
    for t in range(x.shape[0]):
        diff = keys - x[t][None, :]
        out[t] = np.einsum("id,id->i", diff, diff)
    return out


def dot_scores(x: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """Dot-product score x_t . keys_i, [T, n], float64."""
    return np.asarray(x, np.float64) @ np.asarray(keys, np.float64).T


def _order_key(values: np.ndarray, mode: str) -> np.ndarray:
    """A key whose ascending order is best-first for the scoring mode."""
    return values if mode == IDW else -values


def best_k(values: np.ndarray, k: int, mode: str = IDW) -> np.ndarray:
    """R3: indices of the k best entries of each row, best first, ties by index."""
    order = np.argsort(_order_key(values, mode), axis=-1, kind="stable")
    return order[..., :k]


def cartesian_best(vA: np.ndarray, A: np.ndarray, vB: np.ndarray, B: np.ndarray,
                   n: int, k: int, mode: str = IDW):
    """R4: best k of the |A| x |B| candidates per token.

    vA, A: [T, kA] half-1 values and indices; vB, B: [T, kB] for half 2.
    Candidate (a, b) has value vA + vB (a distance D for IDW, a score for dot
    product) and slot a*n + b.  Returns (slots [T, k], values [T, k]) ordered
    best first, ties by slot.
    """
    T = vA.shape[0]
    val = (vA[:, :, None] + vB[:, None, :]).reshape(T, -1)
    slot = (A[:, :, None].astype(np.int64) * n + B[:, None, :]).reshape(T, -1)
    order = np.lexsort((slot, _order_key(val, mode)), axis=-1)[:, :k]
    return (np.take_along_axis(slot, order, axis=-1),
            np.take_along_axis(val, order, axis=-1))


def score_weights(values: np.ndarray, eps: float, mode: str = IDW) -> np.ndarray:
    """R5: softmax over the k selected scores (IDW: s = -log(eps + D))."""
    s = -np.log(eps + values) if mode == IDW else np.asarray(values, np.float64)
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=-1, keepdims=True)


def near_tie(v_k: np.ndarray, v_k1: np.ndarray) -> np.ndarray:
    """True where the k-th and (k+1)-th best values are within NEAR_TIE_REL."""
    scale = np.maximum(np.maximum(np.abs(v_k), np.abs(v_k1)), 1.0)
    return np.abs(v_k1 - v_k) <= NEAR_TIE_REL * scale


@dataclasses.dataclass
class UnitChunkResult:
    retrieved: np.ndarray        # [C, d_v] float64
    slots: np.ndarray            # [C, k] int64, best first
    values: np.ndarray           # [C, k] distances D (IDW) or scores (dot)
    weights: np.ndarray          # [C, k] float64
    value_k1: np.ndarray         # [C] (k+1)-th best value over all N slots
    near_tie: np.ndarray         # [C] bool
    overridden: np.ndarray       # [C] bool: selection taken from the caller
    updates: Optional[dict]      # {"k1"|"k2"|"v": (rows, new fp32 rows)} or None
    half_values: Optional[tuple] = None   # R2 values (d1 [C, n], d2 [C, n]) or dot scores
    mode: str = IDW


def _weighted_rows(w: np.ndarray, vsel: np.ndarray) -> np.ndarray:
    """R6: out_t = sum_m w[t, m] vsel[t, m], summed in rank order."""
    out = np.zeros((vsel.shape[0], vsel.shape[2]), dtype=np.float64)
    for m in range(vsel.shape[1]):
        out += w[:, m, None] * vsel[:, m, :]
    return out


def _half_values(q, K, mode):
    return sq_distances(q, K) if mode == IDW else dot_scores(q, K)


def read_unit(k1, k2, v, q, k, eps, mode=IDW, override: Optional[Dict[int, Sequence[int]]] = None):
    """R1-R6 for one unit: returns (retrieved, slots, values, weights, extras)."""
    n, half = k1.shape
    q1, q2 = split_query(np.asarray(q, np.float64), half)
    v1 = _half_values(q1, k1, mode)
    v2 = _half_values(q2, k2, mode)
    A = best_k(v1, k, mode)
    B = best_k(v2, k, mode)
    slots, vals = cartesian_best(np.take_along_axis(v1, A, -1), A,
                                 np.take_along_axis(v2, B, -1), B, n, k, mode)
    # selection margin: the (k+1)-th best value over all n*n slots lies in the
    # Cartesian product of the per-half (k+1)-best lists
    N = n * n
    C = q.shape[0]
    vk1 = np.full(C, np.inf if mode == IDW else -np.inf)
    if N > k:
        kk = min(k + 1, n)
        A1 = best_k(v1, kk, mode)
        B1 = best_k(v2, kk, mode)
        _, vals1 = cartesian_best(np.take_along_axis(v1, A1, -1), A1,
                                  np.take_along_axis(v2, B1, -1), B1, n, k + 1, mode)
        vk1 = vals1[:, k]
    tie = near_tie(vals[:, k - 1], vk1) if N > k else np.zeros(C, bool)
    overridden = np.zeros(C, dtype=bool)
    if override:
        for t, chosen in override.items():
            chosen = np.asarray(sorted(int(s) for s in chosen), dtype=np.int64)
            # an imposed selection is still k distinct slots of the memory
            if (chosen.size != k or np.unique(chosen).size != k
                    or chosen.min() < 0 or chosen.max() >= N):
                raise ValueError(f"override of token {t} is not {k} distinct slots in [0, {N}): "
                                 f"{chosen.tolist()}")
            a, b = chosen // n, chosen % n
            cv = v1[t, a] + v2[t, b]
            order = np.lexsort((chosen, _order_key(cv, mode)))
            slots[t] = chosen[order]
            vals[t] = cv[order]
            overridden[t] = True
    w = score_weights(vals, eps, mode)
    out = _weighted_rows(w, np.asarray(v, np.float64)[slots])
    return out, slots, vals, w, dict(value_k1=vk1, near_tie=tie, overridden=overridden,
                                     half_values=(v1, v2))


# -------------------------------------------------------------------- write


def _sum_by_row(rows: np.ndarray, tokens: np.ndarray, contrib: np.ndarray):
    """Per distinct row: the sum of contributions over its pairs, and the
    number of distinct tokens among those pairs.  Pairs arrive in (token,
    rank) order, so each row's sum runs over ascending tokens."""
    uniq, inv = np.unique(rows, return_inverse=True)
    sums = np.zeros((uniq.size, contrib.shape[1]), dtype=np.float64)
    np.add.at(sums, inv, contrib)
    row_tok = np.unique(np.stack([inv, tokens]), axis=1)
    counts = np.bincount(row_tok[0], minlength=uniq.size)
    return uniq, sums, counts


def chunk_gradients(k1, k2, v, q, y, slots, values, weights, eps=1e-3, mode=IDW,
                    token_weights=None):
    """W1-W2 summed per row, with the token counts W3 divides by.

    Returns {"v"|"k1"|"k2": (rows, summed gradient [rows, d], token counts)}
    where the summed gradient is dL/dtheta_r for
    L = sum_t lambda_t/2 ||out_t - y_t||^2 at the given (fixed) selection
    (lambda = token_weights [C], default all 1); tokens with lambda_t = 0 are
    left out of the sums and the counts.
    """
    n, half = k1.shape
    C, k = slots.shape
    q64 = np.asarray(q, np.float64)
    q1, q2 = split_query(q64, half)
    vsel = np.asarray(v, np.float64)[slots]                    # [C, k, d_v]
    w = weights
    out = _weighted_rows(w, vsel)
    g = out - np.asarray(y, np.float64)                        # W1
    lam = np.ones(C) if token_weights is None else np.asarray(token_weights, np.float64)
    g = lam[:, None] * g                                       # dL/d out_t
    gv = np.einsum("cd,ckd->ck", g, vsel)
    gout = np.einsum("cd,cd->c", g, out)
    delta = w * (gv - gout[:, None])                           # dL_t/ds_m
    a = slots // n
    b = slots % n
    k1_64 = np.asarray(k1, np.float64)
    k2_64 = np.asarray(k2, np.float64)
    tok = np.repeat(np.arange(C), k)                           # pair -> token
    # W2: per-pair contributions in (token, rank) order
    gV = (w[:, :, None] * g[:, None, :]).reshape(C * k, -1)
    if mode == IDW:
        coef = 2.0 * delta / (eps + values)                    # ds/dD = -1/(eps+D)
        gK1 = (coef[:, :, None] * (q1[:, None, :] - k1_64[a])).reshape(C * k, -1)
        gK2 = (coef[:, :, None] * (q2[:, None, :] - k2_64[b])).reshape(C * k, -1)
    else:
        gK1 = (delta[:, :, None] * np.broadcast_to(q1[:, None, :], (C, k, half))).reshape(C * k, -1)
        gK2 = (delta[:, :, None] * np.broadcast_to(q2[:, None, :], (C, k, half))).reshape(C * k, -1)
    keep = lam[tok] != 0.0                                     # pairs of writing tokens
    return {
        "v": _sum_by_row(slots.reshape(-1)[keep], tok[keep], gV[keep]),
        "k1": _sum_by_row(a.reshape(-1)[keep], tok[keep], gK1[keep]),
        "k2": _sum_by_row(b.reshape(-1)[keep], tok[keep], gK2[keep]),
    }


def addressing_gradients(k1, k2, q, eps=1e-3, mode=IDW, lam_addr=1.0):
    """dL_addr/dK1, dL_addr/dK2 [n, d_h] (float64) for
    L_addr = lam_addr * sum_h sum_i p_h[i] log p_h[i],
    p_h = mean over the chunk's tokens of softmax_i(s_h[t, i]) over all n
    sub-keys, s_h the R2/R3 scores.  With l_i = log p_i, the chain rule gives
    dL/ds_h[t, j] = lam/C * P[t, j] (l_j - sum_i P[t, i] l_i)."""
    n, half = k1.shape
    q64 = np.asarray(q, np.float64)
    C = q64.shape[0]
    out = []
    for h, K in enumerate((k1, k2)):
        K64 = np.asarray(K, np.float64)
        qh = q64[:, h * half:(h + 1) * half]
        if mode == IDW:
            d = sq_distances(qh, K64)                              # [C, n]
            S = -np.log(eps + d)
        else:
            S = dot_scores(qh, K64)
        E = np.exp(S - S.max(axis=1, keepdims=True))
        P = E / E.sum(axis=1, keepdims=True)                       # per-token softmax
        p = P.mean(axis=0)                                         # chunk marginal
        ell = np.log(p)
        G = lam_addr / C * P * (ell[None, :] - (P * ell[None, :]).sum(axis=1, keepdims=True))
        if mode == IDW:
            coef = G * 2.0 / (eps + d)                             # ds/dK_i = 2 (q - K_i) / (eps + d)
            dK = coef.T @ qh - coef.sum(axis=0)[:, None] * K64
        else:
            dK = G.T @ qh                                          # ds/dK_i = q
        out.append(dK)
    return out[0], out[1]


def unit_chunk(k1, k2, v, q, y, lr, k, eps=1e-3, mode=IDW, override=None,
               token_weights=None, addr_weight=0.0) -> UnitChunkResult:
    """Read, then (if lr != 0) the aggregated SGD step, for one unit.

    k1, k2 [n, d_h] fp32; v [n*n, d_v] fp32; q [C, 2 d_h]; y [C, d_v];
    token_weights [C] or None (all 1); addr_weight = lambda_addr of the
    addressing loss (0: none; otherwise every K row is updated).
    The tables are not modified; the new values of every touched row are
    returned in ``updates`` (rounded to fp32).
    """
    out, slots, vals, w, ex = read_unit(k1, k2, v, q, k, eps, mode, override)
    res = UnitChunkResult(retrieved=out, slots=slots, values=vals, weights=w,
                          value_k1=ex["value_k1"], near_tie=ex["near_tie"],
                          overridden=ex["overridden"], updates=None,
                          half_values=ex["half_values"], mode=mode)
    if lr == 0.0:
        return res
    grads = chunk_gradients(k1, k2, v, q, y, slots, vals, w, eps, mode, token_weights)
    updates = {}
    addr = {}
    if addr_weight != 0.0:
        addr["k1"], addr["k2"] = addressing_gradients(k1, k2, q, eps, mode, addr_weight)
    for name, table in (("v", v), ("k1", k1), ("k2", k2)):
        rows, sums, counts = grads[name]
        mean = sums / counts[:, None]                          # W3
        if name in addr:
            grad = addr[name].copy()                           # every row: addressing
            grad[rows] += mean                                 # touched rows: + MSE mean
            rows = np.arange(table.shape[0])
            new = (np.asarray(table, np.float64) - lr * grad).astype(np.float32)
        else:
            new = (np.asarray(table[rows], np.float64) - lr * mean).astype(np.float32)  # W4
        updates[name] = (rows, new)
    res.updates = updates
    return res


def apply_updates(k1, k2, v, updates) -> None:
    """Write a unit's new rows into its tables (in place)."""
    if not updates:
        return
    for name, table in (("k1", k1), ("k2", k2), ("v", v)):
        rows, new = updates[name]
        table[rows] = new


# ------------------------------------------------------------- whole chunk


def forward_chunk(state: dict, queries: np.ndarray, targets: np.ndarray, lr: float,
                  k: int, eps: float = 1e-3, mode: str = IDW,
                  overrides: Optional[Dict[int, Dict[int, Sequence[int]]]] = None,
                  inplace: bool = False, token_weights: Optional[np.ndarray] = None,
                  addr_weight: float = 0.0):
    """One chunk over every unit.

    state: {"k1": [U, n, d_h], "k2": [U, n, d_h], "v": [U, n*n, d_v]} fp32,
           unit u = b*H + h.
    queries [B, C, H, d_qk], targets [B, C, H, d_v], token_weights [B, C, H]
    or None (all 1); addr_weight = lambda_addr (0: no addressing loss).
    overrides: {u: {t: slot set}} selections imposed on given tokens.
    Returns (retrieved [B, C, H, d_v] float64, next state, per-unit results).
    With inplace=False the input state is left as it was.
    """
    B, C, H, _ = queries.shape
    nxt = state if inplace else {key: val.copy() for key, val in state.items()}
    retrieved = np.zeros((B, C, H, targets.shape[-1]), dtype=np.float64)
    results = []
    for b in range(B):
        for h in range(H):
            u = b * H + h
            ov = overrides.get(u) if overrides else None
            # every unit reads the state as it was before this chunk
            tw = None if token_weights is None else token_weights[b, :, h]
            r = unit_chunk(state["k1"][u], state["k2"][u], state["v"][u],
                           queries[b, :, h], targets[b, :, h], lr, k, eps, mode, ov, tw,
                           addr_weight)
            retrieved[b, :, h] = r.retrieved
            results.append(r)
    if lr != 0.0:
        for u, r in enumerate(results):
            apply_updates(nxt["k1"][u], nxt["k2"][u], nxt["v"][u], r.updates)
    return retrieved, nxt, results
