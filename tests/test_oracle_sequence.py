"""Pins of the sequence-level oracle (projections, lookahead targets, chunk
loop, gate) against closed forms and invariants that do not restate it.
"""

import numpy as np
import pytest

from oracle import fwpkm_oracle as O
from oracle import fwpkm_sequence as OS


def _state(rng, U, n, dh, dv):
    return {"k1": (rng.standard_normal((U, n, dh)) / np.sqrt(dh)).astype(np.float32),
            "k2": (rng.standard_normal((U, n, dh)) / np.sqrt(dh)).astype(np.float32),
            "v": (rng.standard_normal((U, n * n, dv)) * 0.14).astype(np.float32)}


def _layer(rng, H, dqk, dv):
    D = H * dv
    w_in = (rng.standard_normal((H * dqk + H * dv, D)) / np.sqrt(D)).astype(np.float32)
    w_gate = (rng.standard_normal((H, D)) / np.sqrt(D)).astype(np.float32)
    b_gate = rng.standard_normal(H).astype(np.float32)
    return w_in, w_gate, b_gate


def test_lookahead_write_is_read_by_the_next_chunk():
    """Two tokens, one-token chunks, k = 1, lr = 1, one head with d_qk = 2,
    d_v = D = 4.  Queries read coordinates 0 and 1 of the token, values are
    2x the token.  Token 1 shares token 0's query but not its value, so:
      chunk 0: token 0 reads V0[s] and writes its target v_1 = 2 x_1 there
               (with one candidate the weight is 1: V <- V - (V - y) = y);
      chunk 1: token 1 (the last: reads only) finds 2 x_1 in slot s.
    out_1 = g_1 * 2 x_1 + (1 - g_1) x_1 = (1 + g_1) x_1."""
    rng = np.random.default_rng(901)
    n, D = 3, 4
    st = _state(rng, 1, n, 1, D)
    x = np.zeros((1, 2, D), np.float32)
    x[0, 0] = [0.3, -0.2, 0.5, 0.25]
    x[0, 1] = [0.3, -0.2, -0.75, 1.5]
    w_in = np.zeros((2 + D, D), np.float32)
    w_in[0, 0] = 1.0
    w_in[1, 1] = 1.0
    w_in[2:, :] = 2.0 * np.eye(D, dtype=np.float32)
    w_gate = np.array([[0.5, -1.0, 0.25, 0.125]], np.float32)
    b_gate = np.array([0.1], np.float32)
    out, nxt, res = OS.forward_sequence(st, x, w_in, w_gate, b_gate, 1.0, 1, chunk=1)
    s = int(res[0][0].slots[0, 0])
    assert int(res[1][0].slots[0, 0]) == s
    g = 1.0 / (1.0 + np.exp(-(w_gate[0].astype(np.float64) @ x[0].T.astype(np.float64)
                              + np.float64(b_gate[0]))))
    x64 = x[0].astype(np.float64)
    np.testing.assert_allclose(out[0, 0], g[0] * st["v"][0, s] + (1 - g[0]) * x64[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out[0, 1], (1 + g[1]) * x64[1], rtol=1e-12, atol=1e-12)
    # state: slot s holds v_1, nothing else moved (one candidate: no key gradient)
    want_v = st["v"].copy()
    want_v[0, s] = 2.0 * x[0, 1]
    assert np.array_equal(nxt["v"], want_v)
    assert np.array_equal(nxt["k1"], st["k1"]) and np.array_equal(nxt["k2"], st["k2"])


@pytest.mark.parametrize("res_head", [0, 1])
def test_saturated_gates_pick_one_path_per_head(res_head):
    """One head's gate saturates at 0, the other's at 1: that head's slice of
    the output is exactly the token slice, the other's exactly the memory
    read (lr = 0, so every read uses the initial tables)."""
    rng = np.random.default_rng(902)
    B, S, H, dqk, dv, n, k = 2, 7, 2, 4, 3, 4, 2
    st = _state(rng, B * H, n, dqk // 2, dv)
    w_in, w_gate, _ = _layer(rng, H, dqk, dv)
    x = rng.standard_normal((B, S, H * dv)).astype(np.float32)
    b_gate = np.full(H, 1e4, np.float32)
    b_gate[res_head] = -1e4
    out, _, _ = OS.forward_sequence(st, x, w_in, w_gate, b_gate, 0.0, k, chunk=3)
    q, _ = OS.project(x, w_in, H, dqk, dv)
    x64 = x.astype(np.float64).reshape(B, S, H, dv)
    out = out.reshape(B, S, H, dv)
    mem_head = 1 - res_head
    for b in range(B):
        assert np.array_equal(out[b, :, res_head], x64[b, :, res_head])
        u = b * H + mem_head
        r = O.read_unit(st["k1"][u], st["k2"][u], st["v"][u], q[b, :, mem_head], k, 1e-3)[0]
        assert np.array_equal(out[b, :, mem_head], r)


def test_projection_rows_are_query_heads_then_value_heads():
    """W_in rows that copy distinct coordinates: each head's query and value
    are the coordinates its rows select."""
    B, S, H, dqk, dv = 1, 3, 2, 2, 3
    D = H * dv
    x = np.arange(B * S * D, dtype=np.float32).reshape(B, S, D) / 8.0
    w_in = np.zeros((H * dqk + H * dv, D), np.float32)
    picks = [5, 0, 3, 1] + [2, 4, 1, 0, 5, 3]     # q(h0), q(h1), v(h0), v(h1)
    for r, c in enumerate(picks):
        w_in[r, c] = 1.0
    q, v = OS.project(x, w_in, H, dqk, dv)
    assert np.array_equal(q[0, :, 0], x[0][:, [5, 0]]) and np.array_equal(q[0, :, 1], x[0][:, [3, 1]])
    assert np.array_equal(v[0, :, 0], x[0][:, [2, 4, 1]]) and np.array_equal(v[0, :, 1], x[0][:, [0, 5, 3]])


@pytest.mark.parametrize("chunk", [1, 3, 5, 11])
def test_without_writes_the_output_does_not_depend_on_chunking(chunk):
    rng = np.random.default_rng(903)
    B, S, H, dqk, dv, n, k = 2, 11, 1, 6, 5, 6, 3
    st = _state(rng, B * H, n, dqk // 2, dv)
    w_in, w_gate, b_gate = _layer(rng, H, dqk, dv)
    x = rng.standard_normal((B, S, H * dv)).astype(np.float32)
    ref, nxt_ref, _ = OS.forward_sequence(st, x, w_in, w_gate, b_gate, 0.0, k, chunk=S)
    out, nxt, _ = OS.forward_sequence(st, x, w_in, w_gate, b_gate, 0.0, k, chunk=chunk)
    assert np.array_equal(out, ref)
    for name in ("k1", "k2", "v"):
        assert np.array_equal(nxt[name], st[name])


def test_one_chunk_reads_only_the_starting_tables():
    """Inside a chunk no token sees the chunk's own writes: one chunk with
    lr = 1 reads exactly what lr = 0 reads."""
    rng = np.random.default_rng(904)
    B, S, H, dqk, dv, n, k = 1, 9, 2, 4, 3, 5, 2
    st = _state(rng, B * H, n, dqk // 2, dv)
    w_in, w_gate, b_gate = _layer(rng, H, dqk, dv)
    x = rng.standard_normal((B, S, H * dv)).astype(np.float32)
    out0, _, _ = OS.forward_sequence(st, x, w_in, w_gate, b_gate, 0.0, k, chunk=S)
    out1, nxt, _ = OS.forward_sequence(st, x, w_in, w_gate, b_gate, 1.0, k, chunk=S)
    assert np.array_equal(out0, out1)
    assert not np.array_equal(nxt["v"], st["v"])


def test_last_token_does_not_write():
    """The step of a one-chunk sequence equals the chunk step of its first
    S-1 tokens with their lookahead targets: the last token adds nothing."""
    rng = np.random.default_rng(905)
    B, S, H, dqk, dv, n, k = 2, 8, 1, 4, 4, 5, 3
    st = _state(rng, B * H, n, dqk // 2, dv)
    w_in, w_gate, b_gate = _layer(rng, H, dqk, dv)
    x = rng.standard_normal((B, S, H * dv)).astype(np.float32)
    _, nxt, _ = OS.forward_sequence(st, x, w_in, w_gate, b_gate, 0.7, k, chunk=S)
    q, v = OS.project(x, w_in, H, dqk, dv)
    _, want, _ = O.forward_chunk(st, q[:, :S - 1], v[:, 1:], 0.7, k)
    for name in ("k1", "k2", "v"):
        assert np.array_equal(nxt[name], want[name]), name


def test_later_chunks_read_earlier_writes():
    """Chunking changes the output once there are writes (the second chunk
    reads what the first wrote), and the two-chunk state is the chunk step
    applied twice by hand."""
    rng = np.random.default_rng(906)
    B, S, H, dqk, dv, n, k = 1, 8, 1, 4, 4, 3, 2
    st = _state(rng, B * H, n, dqk // 2, dv)
    w_in, w_gate, b_gate = _layer(rng, H, dqk, dv)
    x = rng.standard_normal((B, S, H * dv)).astype(np.float32)
    one, _, _ = OS.forward_sequence(st, x, w_in, w_gate, b_gate, 1.0, k, chunk=S)
    two, nxt, _ = OS.forward_sequence(st, x, w_in, w_gate, b_gate, 1.0, k, chunk=4)
    assert np.array_equal(one[:, :4], two[:, :4])
    assert not np.allclose(one[:, 4:], two[:, 4:])
    q, v = OS.project(x, w_in, H, dqk, dv)
    y = np.zeros_like(v)
    y[:, :-1] = v[:, 1:]
    tw = np.ones((B, S, H), np.float32)
    tw[:, -1] = 0
    _, s1, _ = O.forward_chunk(st, q[:, :4], y[:, :4], 1.0, k)
    _, s2, _ = O.forward_chunk(s1, q[:, 4:], y[:, 4:], 1.0, k, token_weights=tw[:, 4:])
    for name in ("k1", "k2", "v"):
        assert np.array_equal(nxt[name], s2[name]), name
