"""The near-tie exemption of the parity check must not accept any selection.

Where the oracle certifies a near-tie, the GPU path may rank the k-th and
(k+1)-th candidates either way, and the oracle then adopts the GPU's set.
These CPU tests feed the validity check selections that are wrong in the ways a
broken top-k would be (wrong slots, repeated slots, slots out of range, an
exact tie broken toward the higher index) and require it to fail, and feed
it legitimate near-tie swaps and require it to pass.  No GPU is involved:
the "GPU" selections are made up here from the oracle's own values.
"""

import numpy as np
import pytest

from oracle import fwpkm_oracle as O
from parity_helpers import selection_overrides, validate_adopted_selection


def _mass_tie_unit(k, seed, T=249, n=256, half=16, dv=16):
    """The mass-tie shape of the two-token selection GPU test: the first
    sub-key table is 4 distinct rows repeated n/4 times, so every token's
    best first-half value is shared by n/4 sub-keys exactly."""
    rng = np.random.default_rng(seed)
    k1 = (rng.standard_normal((n, half)) / np.sqrt(half)).astype(np.float32)
    k1 = np.ascontiguousarray(np.tile(k1[:4], (n // 4, 1)))
    k2 = (rng.standard_normal((n, half)) / np.sqrt(half)).astype(np.float32)
    v = (rng.standard_normal((n * n, dv)) * 0.14).astype(np.float32)
    q = rng.standard_normal((T, 2 * half)).astype(np.float32)
    y = rng.standard_normal((T, dv)).astype(np.float32)
    r = O.unit_chunk(k1, k2, v, q, y, 0.0, k)
    return r, n


def _as_gpu(slots_per_token):
    """[T, k] selections -> the [B=1, T, H=1, k] layout the validity check reads."""
    return np.asarray(slots_per_token)[None, :, None, :]


@pytest.mark.parametrize("k", [8, 16])
def test_mass_ties_are_certified_and_the_oracle_set_passes(k):
    r, n = _mass_tie_unit(k, 4343 + k)
    assert r.near_tie.all()          # exact ties at the k-th value, every token
    ov, ties = selection_overrides({0: r}, _as_gpu(r.slots), 1, [0])
    assert ov == {} and ties == 0


@pytest.mark.parametrize("k", [8, 16])
def test_highest_slots_are_rejected_at_every_token(k):
    """The selection the old check let through: the k highest slot indices."""
    r, n = _mass_tie_unit(k, 4343 + k)
    N = n * n
    wrong = np.tile(np.arange(N - k, N), (r.slots.shape[0], 1))
    with pytest.raises(AssertionError):
        selection_overrides({0: r}, _as_gpu(wrong), 1, [0])
    for t in range(r.slots.shape[0]):
        with pytest.raises(AssertionError):
            validate_adopted_selection(r, t, wrong[t], n)


@pytest.mark.parametrize("k", [8, 16])
def test_repeated_and_out_of_range_slots_are_rejected(k):
    r, n = _mass_tie_unit(k, 4343 + k)
    t = 5
    with pytest.raises(AssertionError):                 # k copies of the best slot
        validate_adopted_selection(r, t, [int(r.slots[t, 0])] * k, n)
    dup = [int(s) for s in r.slots[t]]
    dup[-1] = dup[0]                                    # one slot twice
    with pytest.raises(AssertionError):
        validate_adopted_selection(r, t, dup, n)
    out = [int(s) for s in r.slots[t]]
    out[-1] = n * n                                     # one past the last slot
    with pytest.raises(AssertionError):
        validate_adopted_selection(r, t, out, n)
    with pytest.raises(AssertionError):                 # too few slots
        validate_adopted_selection(r, t, [int(s) for s in r.slots[t, :-1]], n)


@pytest.mark.parametrize("k", [8, 16])
def test_exact_tie_broken_toward_a_higher_index_is_rejected(k):
    """Replace a selected slot by a copy of exactly the same value (same
    second-half row, a higher-index copy of the first-half row): the values
    are equal, so the near-tie window alone would accept it; the lower-index
    rule must not."""
    r, n = _mass_tie_unit(k, 4343 + k)
    for t in (0, 7, 100, 248):
        sel = [int(s) for s in r.slots[t]]
        taken_a = {s // n for s in sel}
        s_last = sel[-1]
        a, b = divmod(s_last, n)
        # copies of row a are a + 4j; take the first one above every selected row
        copy = next(c for c in range(a % 4, n, 4) if c > max(taken_a))
        swapped = sel[:-1] + [copy * n + b]
        v1, v2 = r.half_values
        assert v1[t, copy] + v2[t, b] == v1[t, a] + v2[t, b]   # exactly the same value
        with pytest.raises(AssertionError, match="exactly the same value"):
            validate_adopted_selection(r, t, swapped, n)
        with pytest.raises(AssertionError):
            selection_overrides({0: r}, _as_gpu(np.where(np.arange(r.slots.shape[0])[:, None] == t,
                                                         np.asarray(swapped)[None, :], r.slots)),
                                1, [0])


def _near_tie_unit(seed=11, T=64, n=32, half=8, dv=8, k=5):
    """Second-half sub-keys in pairs one fp32 ulp apart in one coordinate:
    candidates sharing a first-half row then differ by ~1e-8 relative, a
    near-tie that is not an exact one (k odd, so twins straddle the k-th
    place)."""
    rng = np.random.default_rng(seed)
    k1 = (rng.standard_normal((n, half)) / np.sqrt(half)).astype(np.float32)
    base = (rng.standard_normal((n // 2, half)) / np.sqrt(half)).astype(np.float32)
    twin = base.copy()
    twin[:, 0] = np.nextafter(twin[:, 0], np.float32(np.inf))
    k2 = np.ascontiguousarray(np.stack([base, twin], 1).reshape(n, half))
    v = (rng.standard_normal((n * n, dv)) * 0.14).astype(np.float32)
    q = rng.standard_normal((T, 2 * half)).astype(np.float32)
    y = rng.standard_normal((T, dv)).astype(np.float32)
    return O.unit_chunk(k1, k2, v, q, y, 0.0, k), n, k


def _brute_order(r, t, n):
    """All n*n slots of token t best first (value, then slot)."""
    v1, v2 = r.half_values
    val = (v1[t][:, None] + v2[t][None, :]).reshape(-1)
    return np.lexsort((np.arange(n * n), val))


def test_near_tie_swap_of_k_th_and_next_passes():
    r, n, k = _near_tie_unit()
    tokens = np.flatnonzero(r.near_tie)
    assert tokens.size > 0
    for t in tokens:
        order = _brute_order(r, t, n)
        swapped = [int(s) for s in order[:k - 1]] + [int(order[k])]
        v1, v2 = r.half_values
        d = [v1[t, s // n] + v2[t, s % n] for s in order[k - 1:k + 1]]
        if d[0] == d[1]:
            continue                   # an exact tie: only the lower slot is allowed
        validate_adopted_selection(r, t, swapped, n)
    gpu = r.slots.copy()
    t = int(next(t for t in tokens if (lambda o: r.half_values[0][t, o[k - 1] // n] +
                                        r.half_values[1][t, o[k - 1] % n] !=
                                        r.half_values[0][t, o[k] // n] +
                                        r.half_values[1][t, o[k] % n])(_brute_order(r, t, n))))
    order = _brute_order(r, t, n)
    gpu[t] = np.concatenate([order[:k - 1], order[k:k + 1]])
    ov, ties = selection_overrides({0: r}, _as_gpu(gpu), 1, [0])
    assert ties == 1 and sorted(ov[0][t]) == sorted(int(s) for s in gpu[t])


def test_swap_without_a_near_tie_is_rejected():
    # k even: twins fill places (1, 2), (3, 4), ..., so the k-th and the next
    # are not twins and no token is a near-tie
    r, n, k = _near_tie_unit(k=4)
    assert not r.near_tie.any()
    t = int(np.flatnonzero(~r.near_tie)[0])
    order = _brute_order(r, t, n)
    gpu = r.slots.copy()
    gpu[t] = np.concatenate([order[:k - 1], order[k:k + 1]])
    with pytest.raises(AssertionError, match="without a near-tie"):
        selection_overrides({0: r}, _as_gpu(gpu), 1, [0])


def test_swap_beyond_the_window_at_a_near_tie_is_rejected():
    """A near-tie at k licenses swapping the tied candidates, not taking a
    clearly worse slot in their place."""
    r, n, k = _near_tie_unit()
    for t in np.flatnonzero(r.near_tie):
        order = _brute_order(r, t, n)
        v1, v2 = r.half_values
        val = np.array([v1[t, s // n] + v2[t, s % n] for s in order])
        d_k = val[k - 1]
        far = np.flatnonzero(np.abs(val - d_k) > 1e-6 * max(abs(d_k), 1.0))
        far = far[far >= k]
        if far.size == 0:
            continue
        bad = [int(s) for s in order[:k - 1]] + [int(order[far[0]])]
        with pytest.raises(AssertionError, match="outside the near-tie window"):
            validate_adopted_selection(r, t, bad, n)
        return
    pytest.fail("no near-tie token with a slot outside the window")


def test_oracle_rejects_a_malformed_override():
    r, n = _mass_tie_unit(8, 11)
    rng = np.random.default_rng(3)
    k1 = (rng.standard_normal((8, 4)) / 2).astype(np.float32)
    k2 = (rng.standard_normal((8, 4)) / 2).astype(np.float32)
    v = rng.standard_normal((64, 4)).astype(np.float32)
    q = rng.standard_normal((2, 8)).astype(np.float32)
    for bad in ([1, 1, 2], [1, 2], [1, 2, 64], [-1, 2, 3]):
        with pytest.raises(ValueError):
            O.read_unit(k1, k2, v, q, 3, 1e-3, override={0: bad})
