"""Chunk-step cases run on the product library and on the checked build.

Run as a script (``python tests/checked_cases.py OUT.npz``) it executes every
case on whichever library ``FWPKM_LIB_PATH`` names and saves the outputs, the
error code of each call (0 = success) and its message; tests/test_gpu_checked.py
runs it in a child process against libfwpkm_checked.so and compares with the
same cases run on the product library in its own process.

The cases cover the paths whose indexing the device checks watch: two key
blocks with a ragged second one and a ragged token tile, both score modes,
a chunk of more than 2048 pairs per unit (separate grouping kernel and
batched update), sub-keys that all tie (whole-wave selection fallback), the
addressing loss, one query asked by 1,024 tokens (hot rows renamed in
the grouping kernel), and 16 units whose value lists are each one hash
group of ~2,000 distinct rows (too many for the update's per-row token
masks: the radix sort groups them).  The last case feeds NaN queries in dot mode, whose
softmax weights are then NaN: a checked build must report it.
"""

import json
import sys

import numpy as np
import torch

CASES = {
    # name: (B, H, C, n, half, dv, k, mode, addr_weight, calls, special)
    "ragged_idw": (3, 2, 80, 96, 64, 320, 8, "idw", 0.0, 2, None),
    "ragged_dot": (3, 2, 80, 96, 64, 320, 8, "dot", 0.0, 2, None),
    "unfused_k16": (2, 1, 300, 64, 64, 128, 16, "idw", 0.0, 2, None),
    "mass_ties": (2, 1, 48, 64, 32, 64, 8, "idw", 0.0, 1, "tied_keys"),
    "addressing": (2, 2, 64, 48, 32, 96, 4, "idw", 0.1, 2, None),
    "nan_dot": (1, 1, 32, 32, 32, 64, 4, "dot", 0.0, 1, "nan_queries"),
    "hot_rows": (1, 1, 1024, 512, 8, 16, 8, "idw", 0.0, 1, "one_query"),
    "many_rows": (16, 1, 256, 256, 512, 64, 8, "idw", 0.0, 1, None),
}


def run(name):
    """Outputs of one case: dict of numpy arrays, plus (code, message) of the
    first failing call (0, "") if every call succeeded."""
    from sparse_weight_memory_amd import Config, Memory, State
    from sparse_weight_memory_amd.memory import FwPKMError
    B, H, C, n, half, dv, k, mode, addr, calls, special = CASES[name]
    rng = np.random.default_rng(sum(map(ord, name)))
    k1 = (rng.standard_normal((B, H, n, half)) / np.sqrt(half)).astype(np.float32)
    k2 = (rng.standard_normal((B, H, n, half)) / np.sqrt(half)).astype(np.float32)
    if special == "tied_keys":
        k1[:] = k1[:, :, :1]
        k2[:] = k2[:, :, :1]
    v = (rng.standard_normal((B, H, n * n, dv)) * 0.14).astype(np.float32)
    mem = Memory(Config(sqrt_slots=n, dim_qk=2 * half, dim_v=dv, topk=k, chunk_size=C, num_heads=H,
                        max_batch=B, score_mode=mode, addr_weight=addr))
    st = State(*(torch.from_numpy(a).cuda() for a in (k1, k2, v)))
    out = {}
    code, msg = 0, ""
    for c in range(calls):
        q = rng.standard_normal((B, C, H, 2 * half)).astype(np.float32)
        if special == "nan_queries":
            q[:] = np.nan
        if special == "one_query":
            q[:] = q[:, :1]
        y = rng.standard_normal((B, C, H, dv)).astype(np.float32)
        print(f"[checked-cases] {name} call {c}", flush=True)
        try:
            r, st, slots, w = mem.forward_chunk(torch.from_numpy(q).cuda(), torch.from_numpy(y).cuda(), 1.0,
                                                st, next=st, return_selection=True)
            torch.cuda.synchronize()
        except FwPKMError as e:
            code, msg = e.code, str(e)
            break
        out[f"retrieved{c}"] = r.cpu().numpy()
        out[f"slots{c}"] = slots.cpu().numpy()
        out[f"weights{c}"] = w.cpu().numpy()
    if code == 0:
        for nm, t in zip(("k1", "k2", "v"), st):
            out[nm] = t.cpu().numpy()
    mem.close()
    return out, code, msg


def main(path):
    from sparse_weight_memory_amd import _lib
    lib = _lib.load()
    arrays, status = {}, {"checked_build": int(lib.fwpkm_checked_build())}
    for name in CASES:
        out, code, msg = run(name)
        status[name] = {"code": code, "message": msg}
        arrays.update({f"{name}/{key}": val for key, val in out.items()})
    np.savez(path, **arrays)
    with open(path + ".json", "w") as f:
        json.dump(status, f)


if __name__ == "__main__":
    import os
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    main(sys.argv[1])
