"""fwpkm_forward_chunk_noalloc: the chunk step on the library's fixed device
workspace, for callers that cannot allocate.

It runs the same kernels as fwpkm_forward_chunk, so on the GPU its results
must equal that entry point's bit for bit: two calls in a row (the second
with fewer sequences and tokens, so it reuses the array the first call
left), in place and in copy mode.  On the CPU: a call whose workspace would
exceed the fixed array is refused before anything is enqueued.
"""

import ctypes

import numpy as np
import pytest
import torch

from sparse_weight_memory_amd import _lib


def _case(seed, B, H, C, n, half, dv):
    rng = np.random.default_rng(seed)
    U = B * H
    st = [(rng.standard_normal((B, H, n, half)) / np.sqrt(half)).astype(np.float32),
          (rng.standard_normal((B, H, n, half)) / np.sqrt(half)).astype(np.float32),
          (rng.standard_normal((B, H, n * n, dv)) * 0.14).astype(np.float32)]
    q = rng.standard_normal((B, C, H, 2 * half)).astype(np.float32)
    y = rng.standard_normal((B, C, H, dv)).astype(np.float32)
    assert U == B * H
    return st, q, y


def _run(mem, st, q, y, lr, noalloc, copy_mode):
    from sparse_weight_memory_amd import State
    past = State(*(torch.from_numpy(a).cuda() for a in st))
    nxt = State(*(torch.empty_like(t) for t in past)) if copy_mode else past
    B, T, H = q.shape[0], q.shape[1], mem.cfg.num_heads
    ret = torch.full((B, T, H, mem.cfg.dim_v), float("nan"), device="cuda")
    print(f"[no-alloc] {'noalloc' if noalloc else 'plain'} call B={B} T={T} copy={copy_mode}",
          flush=True)
    r, n, slots, w = mem.forward_chunk(torch.from_numpy(q).cuda(), torch.from_numpy(y).cuda(), lr,
                                       past, next=nxt, retrieved=ret, return_selection=True,
                                       noalloc=noalloc)
    torch.cuda.synchronize()
    return r.cpu(), [t.cpu() for t in n], slots.cpu(), w.cpu()


def _compare(i, got, ref):
    assert torch.equal(got[2], ref[2]), f"call {i}: selected slots differ"
    assert torch.equal(got[3], ref[3]), f"call {i}: weights differ"
    assert torch.equal(got[0], ref[0]), f"call {i}: retrieved differs"
    for name, a, b in zip(("k1", "k2", "v"), got[1], ref[1]):
        assert torch.equal(a, b), f"call {i}: next {name} differs"


@pytest.mark.gpu
@pytest.mark.parametrize("mode", ["idw", "dot"])
def test_noalloc_equals_the_allocating_entry_point(mode):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from sparse_weight_memory_amd import Config, Memory
    # two key blocks with a ragged second one (n = 96), a ragged token tile,
    # d_v spanning two float4 rounds per lane
    n, half, dv, k, C, H = 96, 64, 320, 8, 80, 2
    mem = Memory(Config(sqrt_slots=n, dim_qk=2 * half, dim_v=dv, topk=k, chunk_size=C,
                        num_heads=H, max_batch=3, score_mode=mode))
    calls = [(3, 80, 1.0, False), (2, 37, 0.5, False), (3, 80, 1.0, True), (1, 5, 1.0, True)]
    for i, (B, T, lr, copy_mode) in enumerate(calls):
        st, q, y = _case(100 * i + (mode == "dot"), B, H, T, n, half, dv)
        ref = _run(mem, st, q, y, lr, noalloc=False, copy_mode=copy_mode)
        got = _run(mem, st, q, y, lr, noalloc=True, copy_mode=copy_mode)
        _compare(i, got, ref)
    mem.close()


@pytest.mark.gpu
def test_noalloc_with_the_separate_grouping_kernel():
    """More than 2,048 pairs per unit: the grouping runs as its own kernel on
    the fixed array too.  The first call's tokens mostly ask one query, so
    its hot regions are renamed to ranks (one radix pass); the second, with
    fewer and random tokens, sorts every region by its rows."""
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from sparse_weight_memory_amd import Config, Memory
    n, half, dv, k, C, H = 512, 8, 16, 8, 1024, 1
    mem = Memory(Config(sqrt_slots=n, dim_qk=2 * half, dim_v=dv, topk=k, chunk_size=C,
                        num_heads=H, max_batch=1))
    for i, (T, lr, copy_mode, hot) in enumerate([(1024, 1.0, False, True), (600, 0.5, True, False)]):
        st, q, y = _case(500 + i, 1, H, T, n, half, dv)
        if hot:
            q[:] = q[:, [t if t % 8 == 0 else 0 for t in range(T)]]
        ref = _run(mem, st, q, y, lr, noalloc=False, copy_mode=copy_mode)
        got = _run(mem, st, q, y, lr, noalloc=True, copy_mode=copy_mode)
        _compare(i, got, ref)
    mem.close()


def test_noalloc_refuses_a_workspace_beyond_the_fixed_array(fwpkm_lib):
    """A 4-head, 512-token, top-16 configuration over 16 sequences needs
    ~160 MiB of workspace: refused with FWPKM_ERR_UNSUPPORTED before any HIP
    call (so this runs without a GPU), while 2 sequences fit."""
    c = _lib.CConfig(512, 256, 256, 16, 512, 4, 16, 1e-3, _lib.SCORE_IDW, 0.0)
    h = ctypes.c_void_p()
    assert fwpkm_lib.fwpkm_create(ctypes.byref(c), ctypes.byref(h)) == _lib.OK
    assert fwpkm_lib.fwpkm_workspace_bytes(ctypes.byref(c)) > _lib.NOALLOC_SCRATCH_BYTES
    st = _lib.CState(0x40_0000_0000, 0x50_0000_0000, 0x60_0000_0000, 4 * 512 * 128, 4 * 512 * 512 * 256)
    args = (0x10_0000_0000, 0x20_0000_0000)
    rc = fwpkm_lib.fwpkm_forward_chunk_noalloc(h, *args, 16, 512, 1.0, ctypes.byref(st),
                                               ctypes.byref(st), 0x30_0000_0000, None, None, None)
    assert rc == _lib.ERR_UNSUPPORTED
    assert "fixed array" in fwpkm_lib.fwpkm_last_error().decode()
    if not torch.cuda.is_available():
        # within the limit the call passes validation and only then needs a device
        rc = fwpkm_lib.fwpkm_forward_chunk_noalloc(h, *args, 2, 512, 1.0, ctypes.byref(st),
                                                   ctypes.byref(st), 0x30_0000_0000, None, None,
                                                   None)
        assert rc == _lib.ERR_HIP
    fwpkm_lib.fwpkm_destroy(h)
