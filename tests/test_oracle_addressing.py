"""Pins of the oracle's marginal-entropy addressing loss.

L_addr = lambda * sum_h sum_i p_h[i] log p_h[i], p_h the chunk mean of the
per-token softmax over all n sub-keys of half h (the pages name a negative-
entropy loss on the key matrices that balances slot usage; the marginal form
is the reading taken).  Pinned by central differences of the loss written
out here, the uniform case, permutation equivariance, the direction it
moves usage in, and how it joins the chunk step.
"""

import numpy as np
import pytest

from oracle import fwpkm_oracle as O


def _keys(rng, n, half, C, spread=0.7):
    k1 = rng.standard_normal((n, half)) * spread
    k2 = rng.standard_normal((n, half)) * spread
    q = rng.standard_normal((C, 2 * half))
    return k1, k2, q


def _neg_entropy(k1, k2, q, eps, mode, lam):
    """The loss from its definition, token by token."""
    n, half = k1.shape
    C = q.shape[0]
    total = 0.0
    for h, K in enumerate((k1, k2)):
        p = np.zeros(n)
        for t in range(C):
            x = q[t, h * half:(h + 1) * half]
            if mode == O.IDW:
                s = np.array([-np.log(eps + np.sum((x - K[i]) ** 2)) for i in range(n)])
            else:
                s = np.array([np.dot(x, K[i]) for i in range(n)])
            e = np.exp(s - s.max())
            p += e / e.sum()
        p /= C
        total += np.sum(p * np.log(p))
    return lam * total


@pytest.mark.parametrize("mode", [O.IDW, O.DOT])
def test_addressing_gradient_matches_central_differences(mode):
    rng = np.random.default_rng(701 if mode == O.IDW else 702)
    n, half, C, eps, lam = 6, 3, 9, 0.05, 0.7
    k1, k2, q = _keys(rng, n, half, C)
    g1, g2 = O.addressing_gradients(k1, k2, q, eps, mode, lam)
    for K, G in ((k1, g1), (k2, g2)):
        for i in range(n):
            for d in range(half):
                h = 1e-6
                orig = K[i, d]
                K[i, d] = orig + h
                Lp = _neg_entropy(k1, k2, q, eps, mode, lam)
                K[i, d] = orig - h
                Lm = _neg_entropy(k1, k2, q, eps, mode, lam)
                K[i, d] = orig
                fd = (Lp - Lm) / (2 * h)
                assert abs(fd - G[i, d]) <= 1e-7 + 1e-6 * abs(fd), (i, d, fd, G[i, d])


def test_uniform_usage_has_zero_gradient():
    """Every sub-key equally far from every query: usage is uniform, the
    entropy is at its maximum and the gradient vanishes."""
    rng = np.random.default_rng(703)
    n, half, C = 8, 4, 5
    k1 = np.zeros((n, half))
    k2 = np.zeros((n, half))
    q = rng.standard_normal((C, 2 * half))
    g1, g2 = O.addressing_gradients(k1, k2, q, 1e-3, O.IDW, 1.0)
    assert np.abs(g1).max() < 1e-14 and np.abs(g2).max() < 1e-14


def test_gradient_follows_a_permutation_of_the_sub_keys():
    rng = np.random.default_rng(704)
    n, half, C = 7, 3, 6
    k1, k2, q = _keys(rng, n, half, C)
    perm = rng.permutation(n)
    g1, g2 = O.addressing_gradients(k1, k2, q, 1e-3, O.IDW, 1.0)
    h1, h2 = O.addressing_gradients(k1[perm], k2[perm], q, 1e-3, O.IDW, 1.0)
    np.testing.assert_allclose(h1, g1[perm], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(h2, g2[perm], rtol=1e-12, atol=1e-15)


def test_a_small_step_spreads_usage():
    """Descending the loss raises the entropy of the marginal usage."""
    rng = np.random.default_rng(705)
    n, half, C = 8, 4, 12
    k1, k2, q = _keys(rng, n, half, C, spread=1.0)
    g1, g2 = O.addressing_gradients(k1, k2, q, 1e-3, O.IDW, 1.0)
    before = _neg_entropy(k1, k2, q, 1e-3, O.IDW, 1.0)
    after = _neg_entropy(k1 - 1e-3 * g1, k2 - 1e-3 * g2, q, 1e-3, O.IDW, 1.0)
    assert after < before


def _unit(rng, n, half, dv, C):
    k1 = (rng.standard_normal((n, half)) / np.sqrt(half)).astype(np.float32)
    k2 = (rng.standard_normal((n, half)) / np.sqrt(half)).astype(np.float32)
    v = (rng.standard_normal((n * n, dv)) * 0.14).astype(np.float32)
    q = rng.standard_normal((C, 2 * half)).astype(np.float32)
    y = rng.standard_normal((C, dv)).astype(np.float32)
    return k1, k2, v, q, y


def test_zero_weight_is_the_plain_step():
    rng = np.random.default_rng(706)
    k1, k2, v, q, y = _unit(rng, 8, 4, 6, 10)
    a = O.unit_chunk(k1, k2, v, q, y, 1.0, 3)
    b = O.unit_chunk(k1, k2, v, q, y, 1.0, 3, addr_weight=0.0)
    for name in ("v", "k1", "k2"):
        assert np.array_equal(a.updates[name][0], b.updates[name][0])
        assert a.updates[name][1].tobytes() == b.updates[name][1].tobytes()


def test_addressing_joins_the_chunk_step():
    """With lambda != 0 every K row moves by -lr * lambda dK_addr; rows the
    MSE touched move by their mean gradient as well; V is unaffected."""
    rng = np.random.default_rng(707)
    n, half, dv, C, k, lr, lam = 8, 4, 6, 10, 3, 0.5, 0.3
    k1, k2, v, q, y = _unit(rng, n, half, dv, C)
    plain = O.unit_chunk(k1, k2, v, q, y, lr, k)
    both = O.unit_chunk(k1, k2, v, q, y, lr, k, addr_weight=lam)
    g1, g2 = O.addressing_gradients(k1, k2, q, 1e-3, O.IDW, lam)
    for name, K, G in (("k1", k1, g1), ("k2", k2, g2)):
        rows, new = both.updates[name]
        assert rows.tolist() == list(range(n))
        # the MSE part, read back from the plain step (rounding ~1 ulp of fp32)
        mse = np.zeros_like(G)
        prow, pnew = plain.updates[name]
        mse[prow] = (K[prow].astype(np.float64) - pnew.astype(np.float64)) / lr
        expect = K.astype(np.float64) - lr * (mse + G)
        np.testing.assert_allclose(new, expect, rtol=0, atol=4e-7)
    assert np.array_equal(plain.updates["v"][0], both.updates["v"][0])
    assert plain.updates["v"][1].tobytes() == both.updates["v"][1].tobytes()
