"""GPU parity of the token-weighted chunk (fwpkm_forward_chunk_weighted)
against the oracle's token-importance reading, through the C ABI.

Weights mix zeros (read-only tokens), fractions and values above 1; some
queries repeat so that rows are written by several tokens with different
weights, through both the short and the long segment paths of the update.
"""

import numpy as np
import pytest
import torch

from parity_helpers import (ATOL_CHAIN, RTOL_CHAIN, assert_close, compare_chunk, need_gpu,
                            oracle_units, say, state_to_dev, state_to_host, to_dev)
from oracle import fwpkm_oracle as O

pytestmark = pytest.mark.gpu


def _mem(**kw):
    from sparse_weight_memory_amd import Config, Memory
    return Memory(Config(**kw))


def _case(seed, B, H, C, n, half, dv, repeat_every=0):
    rng = np.random.default_rng(seed)
    U = B * H
    st = {"k1": (rng.standard_normal((U, n, half)) / np.sqrt(half)).astype(np.float32),
          "k2": (rng.standard_normal((U, n, half)) / np.sqrt(half)).astype(np.float32),
          "v": (rng.standard_normal((U, n * n, dv)) * 0.14).astype(np.float32)}
    q = rng.standard_normal((B, C, H, 2 * half)).astype(np.float32)
    if repeat_every:
        # a few distinct queries repeated across the chunk: long segments
        base = q[:, :repeat_every].copy()
        for t in range(C):
            q[:, t] = base[:, t % repeat_every] + 0.01 * rng.standard_normal(q[:, t].shape).astype(np.float32)
    y = rng.standard_normal((B, C, H, dv)).astype(np.float32)
    tw = rng.uniform(0.0, 2.0, (B, C, H)).astype(np.float32)
    tw[rng.random((B, C, H)) < 0.25] = 0.0
    return st, q, y, tw


@pytest.mark.parametrize("mode", ["idw", "dot"])
def test_weighted_chunk_matches_oracle(mode):
    need_gpu()
    B, H, C, n, half, dv, k = 3, 2, 64, 32, 16, 64, 4
    mem = _mem(sqrt_slots=n, dim_qk=2 * half, dim_v=dv, topk=k, chunk_size=C, num_heads=H,
               max_batch=B, score_mode=mode)
    st, q, y, tw = _case(71 if mode == "idw" else 72, B, H, C, n, half, dv)
    compare_chunk(mem, st, q, y, 1.0, label=f"weighted-{mode}", tw=tw)


def test_weighted_long_segments_match_oracle():
    need_gpu()
    B, H, C, n, half, dv, k = 2, 1, 256, 64, 32, 128, 8
    mem = _mem(sqrt_slots=n, dim_qk=2 * half, dim_v=dv, topk=k, chunk_size=C, num_heads=H, max_batch=B)
    st, q, y, tw = _case(73, B, H, C, n, half, dv, repeat_every=5)
    compare_chunk(mem, st, q, y, 0.5, label="weighted-long", tw=tw)


def test_unit_weights_are_bitwise_the_plain_call():
    need_gpu()
    B, H, C, n, half, dv, k = 3, 2, 64, 32, 16, 64, 4
    mem = _mem(sqrt_slots=n, dim_qk=2 * half, dim_v=dv, topk=k, chunk_size=C, num_heads=H, max_batch=B)
    st, q, y, _ = _case(74, B, H, C, n, half, dv)
    d0 = state_to_dev(st, B, H)
    r0, n0 = mem.forward_chunk(to_dev(q), to_dev(y), 1.0, d0, next=d0)
    d1 = state_to_dev(st, B, H)
    ones = torch.ones((B, C, H), device="cuda")
    r1, n1 = mem.forward_chunk(to_dev(q), to_dev(y), 1.0, d1, next=d1, token_weights=ones)
    torch.cuda.synchronize()
    assert torch.equal(r0, r1)
    for a, b in zip(n0, n1):
        assert torch.equal(a, b)


def test_zero_weights_read_without_writing():
    need_gpu()
    B, H, C, n, half, dv, k = 2, 2, 48, 32, 16, 64, 4
    mem = _mem(sqrt_slots=n, dim_qk=2 * half, dim_v=dv, topk=k, chunk_size=C, num_heads=H, max_batch=B)
    st, q, y, _ = _case(75, B, H, C, n, half, dv)
    d0 = state_to_dev(st, B, H)
    r0, _ = mem.forward_chunk(to_dev(q), to_dev(y), 0.0, d0, next=d0)
    d1 = state_to_dev(st, B, H)
    before = [t.clone() for t in d1]
    zeros = torch.zeros((B, C, H), device="cuda")
    r1, n1 = mem.forward_chunk(to_dev(q), to_dev(y), 1.0, d1, next=d1, token_weights=zeros)
    torch.cuda.synchronize()
    assert torch.equal(r0, r1)
    for a, b in zip(before, n1):
        assert torch.equal(a, b)


def test_weighted_chain_with_masked_last_token():
    """Four chained chunks where the last token of each sequence has weight 0
    (it has no lookahead target) and the rest weight 1."""
    need_gpu()
    B, H, C, n, half, dv, k, chunks = 2, 1, 32, 32, 16, 64, 4, 4
    mem = _mem(sqrt_slots=n, dim_qk=2 * half, dim_v=dv, topk=k, chunk_size=C, num_heads=H, max_batch=B)
    rng = np.random.default_rng(76)
    st, _, _, _ = _case(76, B, H, C, n, half, dv)
    dev = state_to_dev(st, B, H)
    host = {name: a.copy() for name, a in st.items()}
    units = list(range(B * H))
    for c in range(chunks):
        q = rng.standard_normal((B, C, H, 2 * half)).astype(np.float32)
        y = rng.standard_normal((B, C, H, dv)).astype(np.float32)
        tw = np.ones((B, C, H), np.float32)
        if c == chunks - 1:
            tw[:, -1] = 0.0
        say("weighted chain chunk", c)
        ret, dev = mem.forward_chunk(to_dev(q), to_dev(y), 1.0, dev, next=dev, token_weights=to_dev(tw))
        rets, host, _ = oracle_units(host, q, y, 1.0, k, mem.cfg.eps, O.IDW, units, H, tw=tw)
    torch.cuda.synchronize()
    got = state_to_host(dev)
    for name in ("k1", "k2", "v"):
        assert_close(f"weighted chain {name}", got[name], host[name], RTOL_CHAIN, ATOL_CHAIN)
