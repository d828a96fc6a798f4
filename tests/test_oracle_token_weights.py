"""Pins of the oracle's token-importance weights (per-token lambda_t on the
MSE loss; lambda_t = 0 reads but does not write).

The pages name the weighting only (sciencestack.ai contents, "Weighting MSE
loss by token importance"); the reading implemented is
L = sum_t lambda_t/2 ||out_t - y_t||^2, with each row's mean taken over the
tokens with lambda_t != 0 that touch it.  These tests pin it against the
unweighted step, one-token chunks, a closed form and finite differences.
"""

import numpy as np
import pytest

from oracle import fwpkm_oracle as O


def _unit(rng, n, half, dv, C, dtype=np.float32):
    k1 = (rng.standard_normal((n, half)) / np.sqrt(half)).astype(dtype)
    k2 = (rng.standard_normal((n, half)) / np.sqrt(half)).astype(dtype)
    v = (rng.standard_normal((n * n, dv)) * 0.14).astype(dtype)
    q = rng.standard_normal((C, 2 * half)).astype(dtype)
    y = rng.standard_normal((C, dv)).astype(dtype)
    return k1, k2, v, q, y


def _state(k1, k2, v):
    return {"k1": k1[None].copy(), "k2": k2[None].copy(), "v": v[None].copy()}


def _run(k1, k2, v, q, y, lr, k, tw=None, mode=O.IDW):
    tw_b = None if tw is None else np.asarray(tw, np.float32)[None, :, None]
    return O.forward_chunk(_state(k1, k2, v), q[None, :, None], y[None, :, None], lr, k,
                           mode=mode, token_weights=tw_b)


@pytest.mark.parametrize("mode", [O.IDW, O.DOT])
def test_unit_weights_are_the_unweighted_step(mode):
    rng = np.random.default_rng(601)
    k1, k2, v, q, y = _unit(rng, 8, 4, 6, 12)
    r0, n0, _ = _run(k1, k2, v, q, y, 1.0, 3, None, mode)
    r1, n1, _ = _run(k1, k2, v, q, y, 1.0, 3, np.ones(12), mode)
    assert r0.tobytes() == r1.tobytes()
    for name in ("k1", "k2", "v"):
        assert n0[name].tobytes() == n1[name].tobytes()


def test_all_masked_reads_but_writes_nothing():
    rng = np.random.default_rng(602)
    k1, k2, v, q, y = _unit(rng, 8, 4, 6, 10)
    r0, _, _ = _run(k1, k2, v, q, y, 1.0, 3)
    r1, n1, _ = _run(k1, k2, v, q, y, 1.0, 3, np.zeros(10))
    assert r0.tobytes() == r1.tobytes()
    for name, a in (("k1", k1), ("k2", k2), ("v", v)):
        assert n1[name][0].tobytes() == a.tobytes()


@pytest.mark.parametrize("t", [0, 4, 9])
def test_single_writer_equals_a_one_token_chunk(t):
    """Only token t writes: the step equals the step of the chunk [t] alone
    (each token's gradient depends on its own read only)."""
    rng = np.random.default_rng(603 + t)
    k1, k2, v, q, y = _unit(rng, 8, 4, 6, 10)
    q[7] = q[t] if t != 7 else q[7]          # another token reading the same rows
    mask = np.zeros(10)
    mask[t] = 1.0
    _, n_mask, _ = _run(k1, k2, v, q, y, 1.0, 3, mask)
    _, n_one, _ = _run(k1, k2, v, q[t:t + 1], y[t:t + 1], 1.0, 3)
    for name in ("k1", "k2", "v"):
        assert n_mask[name].tobytes() == n_one[name].tobytes(), name


def test_weight_scales_a_single_token_step_like_the_learning_rate():
    rng = np.random.default_rng(604)
    k1, k2, v, q, y = _unit(rng, 8, 4, 6, 1)
    lam, lr = 0.37, 0.8
    _, n_w, _ = _run(k1, k2, v, q, y, lr, 3, [lam])
    _, n_lr, _ = _run(k1, k2, v, q, y, lr * lam, 3)
    for name in ("k1", "k2", "v"):
        np.testing.assert_allclose(n_w[name], n_lr[name], rtol=1e-6, atol=1e-7)
    assert not np.array_equal(n_w["v"], v[None])


def test_two_weighted_tokens_on_one_slot_closed_form():
    """k = 1, two identical queries (same slot, w = 1, out = V[slot]):
    V' = V - lr * (l1 (V - y1) + l2 (V - y2)) / 2 -- the mean runs over the
    two writing tokens, each gradient scaled by its weight."""
    rng = np.random.default_rng(605)
    k1, k2, v, q, y = _unit(rng, 8, 4, 6, 2, dtype=np.float64)
    q[1] = q[0]
    l1, l2, lr = 1.0, 3.0, 1.0
    _, nxt, res = _run(k1.astype(np.float32), k2.astype(np.float32), v.astype(np.float32),
                       q.astype(np.float32), y.astype(np.float32), lr, 1, [l1, l2])
    hit = int(res[0].slots[0, 0])
    V = v.astype(np.float32).astype(np.float64)[hit]
    y1, y2 = (y.astype(np.float32).astype(np.float64)[i] for i in (0, 1))
    expect = V - lr * (l1 * (V - y1) + l2 * (V - y2)) / 2.0
    np.testing.assert_allclose(nxt["v"][0, hit], expect, rtol=1e-6, atol=1e-6)


def _weighted_loss(k1, k2, v, q, y, slots, eps, lam):
    n, half = k1.shape
    L = 0.0
    for t in range(q.shape[0]):
        a, b = slots[t] // n, slots[t] % n
        D = ((q[t, :half] - k1[a]) ** 2).sum(1) + ((q[t, half:] - k2[b]) ** 2).sum(1)
        s = -np.log(eps + D)
        e = np.exp(s - s.max())
        w = e / e.sum()
        out = (w[:, None] * v[slots[t]]).sum(0)
        L += lam[t] * 0.5 * ((out - y[t]) ** 2).sum()
    return L


def test_weighted_gradients_match_central_differences():
    rng = np.random.default_rng(606)
    n, half, dv, C, k, eps = 5, 3, 4, 6, 3, 0.05
    k1, k2, v, q, y = _unit(rng, n, half, dv, C, dtype=np.float64)
    k1 *= 0.6 * np.sqrt(half)
    k2 *= 0.6 * np.sqrt(half)
    q *= 0.8
    q[4] = q[1]
    lam = rng.uniform(0.2, 2.0, C)
    _, slots, vals, w, _ = O.read_unit(k1, k2, v, q, k, eps)
    grads = O.chunk_gradients(k1, k2, v, q, y, slots, vals, w, eps, O.IDW, lam)
    tables = {"k1": k1, "k2": k2, "v": v}
    checked = 0
    for name, (rows, sums, counts) in grads.items():
        tab = tables[name]
        for ri, r in enumerate(rows):
            for d in range(tab.shape[1]):
                h = 1e-6 * max(1.0, abs(tab[r, d]))
                orig = tab[r, d]
                tab[r, d] = orig + h
                if not np.array_equal(O.read_unit(k1, k2, v, q, k, eps)[1], slots):
                    tab[r, d] = orig
                    continue
                Lp = _weighted_loss(k1, k2, v, q, y, slots, eps, lam)
                tab[r, d] = orig - h
                Lm = _weighted_loss(k1, k2, v, q, y, slots, eps, lam)
                tab[r, d] = orig
                fd = (Lp - Lm) / (2 * h)
                assert abs(fd - sums[ri, d]) <= 1e-6 * max(1.0, abs(fd)), (name, r, d)
                checked += 1
    assert checked > 50
