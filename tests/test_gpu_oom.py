"""Out of device memory: the workspace allocation fails cleanly.

A handle allocates its workspace at its first chunk call.  Here the device's
free memory is first taken by another allocation, so that call must return
FWPKM_ERR_OOM before anything is enqueued: the retrieved output, the next
state (copy mode) and the past state keep the values they had.  Once the
memory is released the same handle works.
"""

import numpy as np
import pytest
import torch

from sparse_weight_memory_amd import _lib


@pytest.mark.gpu
def test_workspace_oom_leaves_outputs_untouched():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from sparse_weight_memory_amd import Config, Memory, State
    from sparse_weight_memory_amd.memory import FwPKMError
    # a configuration whose workspace (sized by max_batch) is about 1.1 GiB,
    # called with 2 sequences
    B, H, C, n, half, dv, k = 2, 1, 512, 64, 64, 2048, 16
    mem = Memory(Config(sqrt_slots=n, dim_qk=2 * half, dim_v=dv, topk=k, chunk_size=C, num_heads=H,
                        max_batch=256))
    need = mem.workspace_bytes
    assert need > 1 << 30
    rng = np.random.default_rng(7)
    past = State(*(torch.from_numpy(a).cuda() for a in (
        (rng.standard_normal((B, H, n, half)) / 8).astype(np.float32),
        (rng.standard_normal((B, H, n, half)) / 8).astype(np.float32),
        (rng.standard_normal((B, H, n * n, dv)) * 0.1).astype(np.float32))))
    nxt = State(*(torch.full_like(t, 5.0) for t in past))
    before = [t.clone() for t in past]
    q = torch.from_numpy(rng.standard_normal((B, C, H, 2 * half)).astype(np.float32)).cuda()
    y = torch.from_numpy(rng.standard_normal((B, C, H, dv)).astype(np.float32)).cuda()
    ret = torch.full((B, C, H, dv), 7.0, device="cuda")
    torch.cuda.synchronize()

    # hold all but half a workspace of the free memory (in 1 GiB blocks, then
    # the rest rounded down to 2 MiB)
    hog = []
    try:
        gib = 1 << 30
        free, _ = torch.cuda.mem_get_info()
        while free - need // 2 > 2 * gib:
            hog.append(torch.empty(gib, dtype=torch.uint8, device="cuda"))
            free, _ = torch.cuda.mem_get_info()
        rest = (free - need // 2) // (2 << 20) * (2 << 20)
        if rest > 0:
            hog.append(torch.empty(rest, dtype=torch.uint8, device="cuda"))
        free, _ = torch.cuda.mem_get_info()
        print(f"[oom] holding {sum(h.numel() for h in hog) / gib:.1f} GiB, {free / gib:.2f} GiB free, "
              f"workspace {need / gib:.2f} GiB", flush=True)
        assert free < need
        with pytest.raises(FwPKMError) as err:
            mem.forward_chunk(q, y, 1.0, past, next=nxt, retrieved=ret)
        assert err.value.code == _lib.ERR_OOM, str(err.value)
        torch.cuda.synchronize()
        assert bool((ret == 7.0).all()), "retrieved was written"
        for t in nxt:
            assert bool((t == 5.0).all()), "next state was written"
        for t, b in zip(past, before):
            assert torch.equal(t, b), "past state was written"
    finally:
        hog.clear()
        torch.cuda.empty_cache()
    print("[oom] memory released; calling again", flush=True)
    r, _ = mem.forward_chunk(q, y, 1.0, past, next=nxt, retrieved=ret)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(r).all()) and not bool((r == 7.0).all())
    mem.close()
