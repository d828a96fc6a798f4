"""GPU parity of the marginal-entropy addressing loss (addr_weight != 0)
against the oracle, through the C ABI: the score kernel's full score tiles,
the statistics kernel, the key-gradient contraction on the matrix cores and
the key step after the update must reproduce the oracle's single step
K <- K - lr (mean MSE gradient + dL_addr/dK) on every key row.
"""

import numpy as np
import pytest
import torch

from parity_helpers import compare_chunk, need_gpu, state_to_dev, to_dev

pytestmark = pytest.mark.gpu


def _mem(**kw):
    from sparse_weight_memory_amd import Config, Memory
    return Memory(Config(**kw))


def _case(seed, B, H, C, n, half, dv, q_std=1.0):
    rng = np.random.default_rng(seed)
    U = B * H
    st = {"k1": (rng.standard_normal((U, n, half)) / np.sqrt(half)).astype(np.float32),
          "k2": (rng.standard_normal((U, n, half)) / np.sqrt(half)).astype(np.float32),
          "v": (rng.standard_normal((U, n * n, dv)) * 0.14).astype(np.float32)}
    q = (rng.standard_normal((B, C, H, 2 * half)) * q_std).astype(np.float32)
    y = rng.standard_normal((B, C, H, dv)).astype(np.float32)
    return st, q, y


@pytest.mark.parametrize("mode,q_std", [("idw", 1.0), ("dot", 0.25)])
def test_addressing_step_matches_oracle(mode, q_std):
    need_gpu()
    B, H, C, n, half, dv, k = 2, 2, 64, 32, 16, 64, 4
    mem = _mem(sqrt_slots=n, dim_qk=2 * half, dim_v=dv, topk=k, chunk_size=C, num_heads=H,
               max_batch=B, score_mode=mode, addr_weight=0.5)
    st, q, y = _case(81 if mode == "idw" else 82, B, H, C, n, half, dv, q_std)
    compare_chunk(mem, st, q, y, 1.0, label=f"addr-{mode}")


def test_addressing_ragged_shapes():
    """Sub-keys, dims and tokens that fill no tile evenly."""
    need_gpu()
    B, H, C, n, half, dv, k = 2, 1, 64, 40, 20, 36, 5
    mem = _mem(sqrt_slots=n, dim_qk=2 * half, dim_v=dv, topk=k, chunk_size=C, num_heads=H,
               max_batch=B, addr_weight=2.0)
    st, q, y = _case(83, B, H, 50, n, half, dv)
    compare_chunk(mem, st, q, y, 0.7, label="addr-ragged")


def test_addressing_at_the_chained_workload_shape():
    """n 256, d_qk 512, d_v 512, top-8, 256 tokens: one 64-key block per
    score workgroup, four gradient tiles per half."""
    need_gpu()
    B, H, C, n, half, dv, k = 1, 1, 256, 256, 256, 512, 8
    mem = _mem(sqrt_slots=n, dim_qk=2 * half, dim_v=dv, topk=k, chunk_size=C, num_heads=H,
               max_batch=B, addr_weight=0.1)
    st, q, y = _case(84, B, H, C, n, half, dv)
    compare_chunk(mem, st, q, y, 1.0, label="addr-wide")


def test_zero_addressing_weight_is_the_plain_step():
    need_gpu()
    B, H, C, n, half, dv, k = 2, 2, 48, 32, 16, 64, 4
    kw = dict(sqrt_slots=n, dim_qk=2 * half, dim_v=dv, topk=k, chunk_size=C, num_heads=H, max_batch=B)
    st, q, y = _case(85, B, H, C, n, half, dv)
    outs = []
    for mem in (_mem(**kw), _mem(addr_weight=0.0, **kw)):
        d = state_to_dev(st, B, H)
        r, nxt = mem.forward_chunk(to_dev(q), to_dev(y), 1.0, d, next=d)
        torch.cuda.synchronize()
        outs.append((r, nxt))
    assert torch.equal(outs[0][0], outs[1][0])
    for a, b in zip(outs[0][1], outs[1][1]):
        assert torch.equal(a, b)


def test_addressing_with_wide_sub_key_tables():
    """n = 1024 sub-keys (four 256-wide load batches per score row), 4 heads
    of d_h 64, top-16: the statistics kernels' row loops and the gradient
    tiles at more than one block per dimension."""
    need_gpu()
    B, H, C, n, half, dv, k = 1, 4, 96, 1024, 64, 32, 16
    mem = _mem(sqrt_slots=n, dim_qk=2 * half, dim_v=dv, topk=k, chunk_size=C, num_heads=H,
               max_batch=B, addr_weight=0.3)
    rng = np.random.default_rng(86)
    U = B * H
    st = {"k1": (rng.standard_normal((U, n, half)) / np.sqrt(half)).astype(np.float32),
          "k2": (rng.standard_normal((U, n, half)) / np.sqrt(half)).astype(np.float32),
          "v": (rng.standard_normal((U, n * n, dv)) * 0.14).astype(np.float32)}
    q = rng.standard_normal((B, C, H, 2 * half)).astype(np.float32)
    y = rng.standard_normal((B, C, H, dv)).astype(np.float32)
    compare_chunk(mem, st, q, y, 1.0, label="addr-n1024")
