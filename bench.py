#!/usr/bin/env python3
"""Throughput of the chained FwPKM read+update chunk on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME|INDEX]

A step is one pass of the whole hot path over one batch of synthetic input:
score -> per-half top-k -> Cartesian top-k -> softmax -> gather -> backward
-> sort -> segmented SGD update, chained through the memory state (each
chunk reads the tables the previous one wrote).  For a single-chunk workload
a step is one chunk call; for a streamed workload it is every chunk of the
pass.  Every step starts from the workload's initial tables: a pristine
device copy is restored before each step, untimed and outside the step's own
event pair, so each timed step is the same first pass and the figures
describe one state.  Inputs and tables sit in HBM before the timed region
starts.  The chunk calls of one step are captured once into a HIP graph and
the graph is replayed for every timed step (--eager launches each chunk from
Python); each step is timed with its own pair of events and the median is
reported.

Prints one JSON line: tokens/s, the roofline of the dominant kernel (timed
with HIP events recorded around each kernel on its own stream), the gather
and scatter kernels' bandwidth against the HBM peak (algorithmic bytes, and
the counted HBM bytes where a fresh counter summary exists), and the CPU
oracle: timed on a bounded sample of the same workload with one thread and
with every host core, and compared chunk by chunk with the GPU's first pass
on two units (near-ties, errors against the tolerances, distinct rows).
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
FP32_MFMA_PEAK_TFLOPS = 157.3   # MI355X dense fp32 matrix
DEFAULT_WORKLOAD = 3            # 65,536 slots, d_v 512, top-8: 8 x 4096 tokens in 16 chained chunks
# the memory state every figure of a run describes; a counter summary taken
# on another state is not used
STATE = "first pass from the initial tables (restored before every step)"
KERNEL_SOURCES = {              # the sources that fix each kernel's code
    "score": ["ka_score.hip", "fwpkm_device.h"],
    "read": ["kb_read.hip", "fwpkm_device.h"],
    "sort": ["kc_sort.hip", "fwpkm_device.h"],
    "update": ["kd_update.hip", "fwpkm_device.h"],
    "addr_stats": ["ke_addr.hip", "fwpkm_device.h"],
    "addr_grad": ["ke_addr.hip", "fwpkm_device.h"],
    "addr_apply": ["ke_addr.hip", "fwpkm_device.h"],
}


def measured_traffic(workload):
    """HBM bytes per launch of each kernel, from the rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary committed under profiles/ (already scaled by the plain
    copy calibration), for kernels whose sources are unchanged since the
    counters were taken; None where there is no summary or it is stale."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"hbm_counters_{workload}.md")
    if not os.path.exists(path):
        return {}
    text = open(path).read()
    try:
        block = text.split("```json", 1)[1].split("```", 1)[0]
        data = json.loads(block)
    except (IndexError, ValueError):
        return {}
    if data.get("state") != STATE:
        return {}
    out = {}
    for name, entry in data.get("kernels", {}).items():
        h = hashlib.sha256()
        for f in entry.get("sources", KERNEL_SOURCES.get(name, [])):
            fp = os.path.join(ROOT, "sparse_weight_memory_amd", "csrc", f)
            if not os.path.exists(fp):
                h = None
                break
            h.update(open(fp, "rb").read())
        fresh = h is not None and h.hexdigest()[:16] == entry.get("source_sha256_16")
        out[name] = entry["bytes_per_launch"] if fresh else None
    return out


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=str(DEFAULT_WORKLOAD))
    ap.add_argument("--batch", type=int, default=0,
                    help="run the workload's per-unit shape with this many sequences "
                         "(the workload name records it); 0 keeps the workload's own")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="approximate CPU time spent timing the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle leg (its timing and its parity check)")
    ap.add_argument("--weighted", action="store_true",
                    help="run the token-weighted step (fwpkm_forward_chunk_weighted): weight 1 "
                         "everywhere except 0 on the last token of every sequence, which has "
                         "no lookahead target")
    ap.add_argument("--addr-weight", type=float, default=0.0,
                    help="weight of the marginal-entropy addressing loss on the sub-keys "
                         "(0: the plain step)")
    ap.add_argument("--sequence", action="store_true",
                    help="time the sequence layer instead (fwpkm_forward_sequence): model-width "
                         "tokens projected to queries and lookahead targets, the chained chunk "
                         "step, and the gated output, with random stand-in layer weights")
    ap.add_argument("--eager", action="store_true",
                    help="launch every chunk from Python instead of replaying a HIP graph")
    ap.add_argument("--no-profile-pass", action="store_true",
                    help="skip the per-kernel event pass (for external profilers)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB, 5 times (to "
                         "calibrate HBM byte counters against a known size), then exit")
    return ap.parse_args()


def copy_probe(mib):
    """A plain device-to-device copy of `mib` MiB, 5 times: the calibration
    for the HBM byte counters, and (timed with events on the copy's stream)
    the bandwidth such a copy achieves, as context for the 8 TB/s peak."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    ms = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        e1.synchronize()
        ms.append(e0.elapsed_time(e1))
    torch.cuda.synchronize()
    med = statistics.median(ms)
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4,
                      "copies": 5, "ms_per_copy": ms,
                      "read_plus_write_gbps_median": 2 * n * 4 / (med * 1e6)}))


def algorithmic_cost(cfg, kernel, tokens, uniq_v, uniq_k, addr=False):
    """Compulsory bytes (and flops) one launch of `kernel` must move.

    tokens  = units * tokens per chunk in the launch
    uniq_v  = distinct value rows the launch updates
    uniq_k  = distinct K1 plus K2 rows the launch updates
    addr    = the addressing loss is on (the score kernel also writes every
              score, 2 halves x n per token)
    """
    f = 4  # fp32
    U = cfg.units
    n, half = cfg.sqrt_slots, cfg.half
    scores = f * tokens * 2 * n              # one fp32 score per (token, half, sub-key)
    keys = f * U * 2 * n * half              # both sub-key tables
    if kernel == "score":
        byts = f * tokens * cfg.dim_qk + keys + (scores if addr else 0)
        flops = 2.0 * tokens * n * cfg.dim_qk
        return byts, flops
    if kernel == "addr_stats":
        # scores in, coefficients out (same buffer)
        return 2 * scores, 0.0
    if kernel == "addr_grad":
        # coefficients and queries in, key tables in (IDW), key gradients out
        return scores + f * tokens * cfg.dim_qk + 2 * keys, 2.0 * tokens * n * cfg.dim_qk
    if kernel == "addr_apply":
        # key gradients in, key tables read and written
        return 3 * keys, 0.0
    D = cfg.heads * cfg.dim_v
    Nf = cfg.heads * (cfg.dim_qk + cfg.dim_v)
    if kernel == "project":
        # tokens and projection rows in, queries and targets out; launched once
        # per sequence call, so `tokens` is every token of the call here
        return f * (tokens * D + Nf * D + tokens * Nf), 2.0 * tokens * D * Nf
    if kernel == "gate":
        # tokens and memory reads in, outputs out (gate rows stay in cache)
        return f * 3 * tokens * D, 2.0 * tokens * D * cfg.heads
    if kernel == "read":
        # k gathered value rows + the target row read + the retrieved row written
        return f * tokens * (cfg.topk * cfg.dim_v + 2 * cfg.dim_v), 0.0
    if kernel == "update":
        # read-modify-write of every touched V, K1 and K2 row
        return f * 2 * (uniq_v * cfg.dim_v + uniq_k * cfg.half), 0.0
    if kernel == "sort":
        # three key lists read, three index lists written
        return f * 2 * 3 * tokens * cfg.topk, 0.0
    return 0.0, 0.0


def _timed_legs(run_once, seconds):
    """Time `run_once()` (returns tokens done) repeatedly for ~seconds, once
    with one BLAS/OpenMP thread and once with every host core this process
    may use.  Returns (one-thread leg, all-cores leg); each records the rate,
    the threads allowed and the cores actually kept busy (CPU time / wall)."""
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    cores = len(os.sched_getaffinity(0))
    legs = []
    for threads in (1, cores):
        ctx = threadpool_limits(limits=threads) if threadpool_limits else None
        tokens = reps = 0
        c0 = time.process_time()
        t0 = time.perf_counter()
        try:
            while True:
                tokens += run_once()
                reps += 1
                if time.perf_counter() - t0 >= seconds:
                    break
        finally:
            if ctx is not None:
                ctx.__exit__(None, None, None)
        dt = time.perf_counter() - t0
        legs.append({"value": tokens / dt, "threads": threads, "reps": reps, "seconds": dt,
                     "cores_busy": (time.process_time() - c0) / dt})
    return legs[0], legs[1]


def cpu_baseline(cfg, tables, Q, Y, seconds):
    """The oracle as it stands on whole chained chunks of unit 0, one thread
    and all cores."""
    import numpy as np

    from oracle import fwpkm_oracle as O

    st = {"k1": tables.k1[:1].copy(), "k2": tables.k2[:1].copy(), "v": tables.v[:1].copy()}
    pos = [0]

    def one_chunk():
        c = pos[0] % cfg.chunks
        q = np.ascontiguousarray(Q[:1, c * cfg.chunk:(c + 1) * cfg.chunk, :1])
        y = np.ascontiguousarray(Y[:1, c * cfg.chunk:(c + 1) * cfg.chunk, :1])
        O.forward_chunk(st, q, y, cfg.lr, cfg.topk, cfg.eps, inplace=True)
        pos[0] += 1
        return cfg.chunk

    one, every = _timed_legs(one_chunk, seconds / 2)
    return {"value": every["value"], "unit": "tokens/s", "cores": every["threads"], "kind": "oracle",
            "cores_busy": every["cores_busy"], "one_thread": one,
            "sample": f"{one['reps'] + every['reps']} chained chunk(s) of {cfg.chunk} tokens on one "
                      f"memory unit (1 of {cfg.units}; units are independent), float64 numpy: "
                      f"{one['reps']} with 1 thread ({one['seconds']:.1f} s), then "
                      f"{every['reps']} with {every['threads']} BLAS threads allowed "
                      f"({every['seconds']:.1f} s; the oracle's element-wise work runs on one "
                      f"core, cores_busy says how many it kept busy)"}


def cpu_baseline_sequence(cfg, tables, x, lw, seconds):
    """The oracle's sequence layer on sequence 0, one thread and all cores."""
    from oracle import fwpkm_sequence as OS

    state = [{"k1": tables.k1[:1].copy(), "k2": tables.k2[:1].copy(), "v": tables.v[:1].copy()}]

    def one_pass():
        _, state[0], _ = OS.forward_sequence(state[0], x[:1], lw.w_in, lw.w_gate, lw.b_gate, cfg.lr,
                                             cfg.topk, cfg.chunk, cfg.eps)
        return x.shape[1]

    one, every = _timed_legs(one_pass, seconds / 2)
    return {"value": every["value"], "unit": "tokens/s", "cores": every["threads"], "kind": "oracle",
            "cores_busy": every["cores_busy"], "one_thread": one,
            "sample": f"{one['reps'] + every['reps']} pass(es) of sequence 0 ({x.shape[1]} tokens, "
                      f"1 of {cfg.batch} sequences; sequences are independent), float64 numpy: "
                      f"{one['reps']} with 1 thread, {every['reps']} with {every['threads']} "
                      f"BLAS threads allowed"}


def parity_leg(cfg, tables, Q, Y, mem, st, restore, qd, yd, units):
    """The GPU's first pass (every chunk, all units, in place, from the
    initial tables: the timed state) against the oracle on `units`, both
    teacher-forced (the oracle restarts every chunk from a host copy of the
    GPU's tables, value rows refreshed where the GPU wrote) and chained (the
    oracle runs its own chain).  Reports near-ties, the worst error as a
    fraction of the tolerance (at most 1 passes), the largest absolute and
    relative errors, and distinct value rows per unit and chunk."""
    import numpy as np
    import torch

    from oracle import fwpkm_oracle as O
    from oracle.compare import (ATOL_CHAIN, ATOL_CHUNK, RTOL_CHAIN, RTOL_CHUNK, error_stats,
                                selection_overrides)

    H, C, k = cfg.heads, cfg.chunk, cfg.topk
    restore()
    torch.cuda.synchronize()
    mirror = {u: {n: getattr(tables, n)[u % H].copy() for n in ("k1", "k2", "v")} for u in units}
    chain = {u: {n: getattr(tables, n)[u % H].copy() for n in ("k1", "k2", "v")} for u in units}
    out = {"units": list(units), "chunks": cfg.chunks, "tokens_checked": 0, "near_ties": 0,
           "teacher_forced": {}, "chained": {}, "unique_v_rows_per_unit_chunk": None, "ok": True}

    def worst(bucket, name, got, want, rtol, atol):
        e = error_stats(got, want, rtol, atol)
        b = out[bucket].setdefault(name, {"tol_used": 0.0, "max_abs_err": 0.0, "max_rel_err": 0.0})
        for key in b:
            b[key] = max(b[key], e[key])

    uniq = []
    try:
        for c in range(cfg.chunks):
            ret, _, slots, weights = mem.forward_chunk(qd[c], yd[c], cfg.lr, st, next=st,
                                                       return_selection=True)
            torch.cuda.synchronize()
            ret_h, slots_h, w_h = ret.cpu().numpy(), slots.cpu().numpy(), weights.cpu().numpy()
            q = Q[:, c * C:(c + 1) * C]
            y = Y[:, c * C:(c + 1) * C]
            for u in range(cfg.units):
                b, h = divmod(u, H)
                uniq.append(np.unique(slots_h[b, :, h]).size)
            for u in units:
                b, h = divmod(u, H)
                m = mirror[u]
                r = O.unit_chunk(m["k1"], m["k2"], m["v"], q[b, :, h], y[b, :, h], cfg.lr, k, cfg.eps)
                ov, nt = selection_overrides({u: r}, slots_h, H, [u])
                if ov:
                    r = O.unit_chunk(m["k1"], m["k2"], m["v"], q[b, :, h], y[b, :, h], cfg.lr, k,
                                     cfg.eps, override=ov[u])
                out["near_ties"] += nt
                out["tokens_checked"] += C
                worst("teacher_forced", "retrieved", ret_h[b, :, h], r.retrieved, RTOL_CHUNK, ATOL_CHUNK)
                go = np.argsort(slots_h[b, :, h], axis=1)
                oo = np.argsort(r.slots, axis=1)
                if not (np.take_along_axis(slots_h[b, :, h], go, 1) ==
                        np.take_along_axis(r.slots, oo, 1)).all():
                    raise AssertionError(f"chunk {c} unit {u}: adopted selection not applied")
                worst("teacher_forced", "weights", np.take_along_axis(w_h[b, :, h], go, 1),
                      np.take_along_axis(r.weights, oo, 1), RTOL_CHUNK, ATOL_CHUNK)
                if r.updates:
                    for name in ("k1", "k2"):
                        rows, new = r.updates[name]
                        want = m[name].copy()
                        want[rows] = new
                        got = getattr(st, name)[b, h].cpu().numpy()
                        worst("teacher_forced", name, got, want, RTOL_CHUNK, ATOL_CHUNK)
                        m[name] = got
                    rows, new = r.updates["v"]
                    want = dict(zip(rows.tolist(), new))
                    allrows = np.union1d(rows, np.unique(slots_h[b, :, h]))
                    idx = torch.as_tensor(allrows, device=st.v.device, dtype=torch.long)
                    got = st.v[b, h].index_select(0, idx).cpu().numpy()
                    ref = np.stack([want.get(int(rr), m["v"][rr]) for rr in allrows])
                    worst("teacher_forced", "v", got, ref, RTOL_CHUNK, ATOL_CHUNK)
                    m["v"][allrows] = got
                # the oracle's own chain
                ch = chain[u]
                rc = O.unit_chunk(ch["k1"], ch["k2"], ch["v"], q[b, :, h], y[b, :, h], cfg.lr, k, cfg.eps)
                ov, _ = selection_overrides({u: rc}, slots_h, H, [u])
                if ov:
                    rc = O.unit_chunk(ch["k1"], ch["k2"], ch["v"], q[b, :, h], y[b, :, h], cfg.lr,
                                      k, cfg.eps, override=ov[u])
                worst("chained", "retrieved", ret_h[b, :, h], rc.retrieved, RTOL_CHAIN, ATOL_CHAIN)
                O.apply_updates(ch["k1"], ch["k2"], ch["v"], rc.updates)
        for u in units:
            b, h = divmod(u, H)
            for name in ("k1", "k2", "v"):
                got = getattr(st, name)[b, h].cpu().numpy()
                worst("chained", name, got, chain[u][name], RTOL_CHAIN, ATOL_CHAIN)
                if name == "v" and not np.array_equal(got, mirror[u]["v"]):
                    raise AssertionError(f"unit {u}: the GPU wrote value rows it did not select")
    except AssertionError as e:
        out["ok"] = False
        out["error"] = str(e)[:400]
    for bucket in ("teacher_forced", "chained"):
        if any(v["tol_used"] > 1.0 for v in out[bucket].values()):
            out["ok"] = False
    out["unique_v_rows_per_unit_chunk"] = (float(np.mean(uniq)) if uniq else None)
    out["unique_v_rows_max"] = int(max(uniq)) if uniq else None
    return out


def main():
    args = parse()
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return
    if args.gpus != 1:
        print(f"bench.py: the FwPKM step here runs on one GPU only (asked for --gpus {args.gpus}); "
              "memory units are independent, so N GPUs would each run this step on "
              "their own share of the batch.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from sparse_weight_memory_amd import Config, Memory, State, _lib
    from workloads import (draw_queries, draw_targets, draw_tokens, get_config, initial_tables,
                           layer_weights)

    key = int(args.workload) if args.workload.isdigit() else args.workload
    cfg = get_config(key)
    if args.batch:
        import dataclasses
        import re
        cfg = dataclasses.replace(cfg, batch=args.batch,
                                  name=re.sub(r"-\d+x", f"-{args.batch}x", cfg.name, count=1))
    if not os.path.exists(_lib.LIB_PATH):
        from sparse_weight_memory_amd import build as _build
        _build.build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")

    print(f"[bench] workload {cfg.name}: drawing inputs", file=sys.stderr, flush=True)
    tables = initial_tables(cfg)
    Q = draw_queries(cfg)
    Y = draw_targets(cfg)
    B, H, C = cfg.batch, cfg.heads, cfg.chunk

    mem = Memory(Config(sqrt_slots=cfg.sqrt_slots, dim_qk=cfg.dim_qk, dim_v=cfg.dim_v,
                        topk=cfg.topk, chunk_size=C, num_heads=H, max_batch=B, eps=cfg.eps,
                        addr_weight=args.addr_weight))
    # per-sequence tables expanded from the shared initial ones (untimed),
    # and a pristine device copy restored before every step
    st = State(*(torch.from_numpy(a).to(dev).unsqueeze(0).repeat(B, *([1] * a.ndim)).contiguous()
                 for a in (tables.k1, tables.k2, tables.v)))
    pristine = st.clone()

    def restore():
        for dst, src in zip(st, pristine):
            dst.copy_(src)

    # each chunk's inputs contiguous in HBM: [chunks, B, C, H, d]
    qd = torch.from_numpy(np.ascontiguousarray(
        Q.reshape(B, cfg.chunks, C, H, cfg.dim_qk).transpose(1, 0, 2, 3, 4))).to(dev)
    yd = torch.from_numpy(np.ascontiguousarray(
        Y.reshape(B, cfg.chunks, C, H, cfg.dim_v).transpose(1, 0, 2, 3, 4))).to(dev)
    ret = torch.empty((B, C, H, cfg.dim_v), device=dev)
    tokens_per_step = B * C * cfg.chunks

    tw = None
    if args.weighted:
        # [chunks, B, C, H]: every token weighs 1 except each sequence's last
        tw = torch.ones((cfg.chunks, B, C, H), device=dev)
        tw[-1, :, -1, :] = 0.0

    def step(select=False):
        out = []
        for c in range(cfg.chunks):
            r = mem.forward_chunk(qd[c], yd[c], cfg.lr, st, next=st, retrieved=ret,
                                  return_selection=select,
                                  token_weights=None if tw is None else tw[c])
            if select:
                out.append(r[2])
        return out

    X = lw = None
    if args.sequence:
        # the sequence layer: model-width tokens [B, S, D] instead of ready
        # queries and targets, random stand-in layer weights
        X = draw_tokens(cfg)
        lw = layer_weights(cfg)
        xd = torch.from_numpy(X).to(dev)
        w_in, w_gate, b_gate = (torch.from_numpy(a).to(dev) for a in (lw.w_in, lw.w_gate, lw.b_gate))
        seq_out = torch.empty_like(xd)
        ws = torch.empty(mem.sequence_workspace_bytes(B, cfg.tokens_per_pass), dtype=torch.uint8,
                         device=dev)
        del qd, yd

        def step(select=False):  # noqa: F811
            r = mem.forward_sequence(xd, w_in, w_gate, b_gate, cfg.lr, st, next=st, out=seq_out,
                                     return_selection=select, workspace=ws)
            if not select:
                return []
            slots = r[2]
            return [slots[:, c * C:(c + 1) * C] for c in range(cfg.chunks)]

    print(f"[bench] warmup {args.warmup} step(s)", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        restore()
        step()
    torch.cuda.synchronize()

    # one step = the chain of all chunks, replayed from a HIP graph so the
    # host does not pace the kernels (the warmup above already allocated the
    # library's workspace, which must not happen under capture)
    graph = None
    if not args.eager:
        restore()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()

    def timed_step():
        if graph is not None:
            graph.replay()
        else:
            step()

    print(f"[bench] timing {args.steps} step(s) ({'eager' if graph is None else 'graph'}), "
          "tables restored before each", file=sys.stderr, flush=True)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in pairs:
        restore()                 # untimed: before the step's own start event
        e0.record()
        timed_step()
        e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [a.elapsed_time(b) for a, b in pairs]
    ms_step = statistics.median(step_ms)
    value = tokens_per_step / (ms_step * 1e-3)

    result = {
        "metric": ("tokens/s for the FwPKM sequence layer (projection, chained chunks, gate)"
                   if args.sequence else "tokens/s for chained FwPKM read+update chunk"),
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "step_ms": {"median": ms_step, "mean": statistics.fmean(step_ms), "min": min(step_ms),
                    "max": max(step_ms), "reps": len(step_ms)},
        "wall_s_timed": wall,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": {"workload": cfg.name, "batch": B, "heads": H, "chunk": C,
                   "chunks_per_step": cfg.chunks, "tokens_per_step": tokens_per_step,
                   "slots": cfg.num_slots, "dim_qk": cfg.dim_qk, "dim_v": cfg.dim_v,
                   "topk": cfg.topk, "lr": cfg.lr, "eps": cfg.eps,
                   "parallelism": "single GPU",
                   "launch": "eager" if graph is None else "hip graph of one step",
                   "state": STATE,
                   "token_weights": "last token of each sequence 0, others 1" if args.weighted else None,
                   "addr_weight": args.addr_weight,
                   "layer": ("sequence: tokens [B, S, H*d_v] -> fp32 projection to queries and "
                             "lookahead targets -> chunks -> gated output; random stand-in "
                             "weights") if args.sequence else None},
    }

    if not args.no_profile_pass:
        print("[bench] per-kernel event pass (same state)", file=sys.stderr, flush=True)
        mem.profile(True)
        sels = []
        for _ in range(args.steps):
            restore()
            sels = step(select=True)      # every step is the same first pass
        prof = mem.profile_read()
        mem.profile(False)
        # distinct rows each launch updates, from the selections of that pass
        uv = uk = 0
        for s in sels:
            flat = s.permute(0, 2, 1, 3).reshape(B * H, -1).long()
            for u in range(B * H):
                row = flat[u]
                uv += int(torch.unique(row).numel())
                uk += int(torch.unique(row // cfg.sqrt_slots).numel())
                uk += int(torch.unique(row % cfg.sqrt_slots).numel())
        launches = len(sels)
        uv /= launches
        uk /= launches
        # the committed counters were taken on the plain step, in this state
        plain = args.addr_weight == 0 and not args.weighted and not args.sequence
        traffic = measured_traffic(cfg.name) if plain else {}
        kernels = {}
        tokens_launch = B * H * C
        for name, (ms, n) in prof.items():
            if n == 0:
                continue
            avg_us = 1e3 * ms / n
            per_call = name in ("project", "gate")      # once per sequence call
            byts, flops = algorithmic_cost(cfg, name, B * cfg.tokens_per_pass if per_call else tokens_launch,
                                           uv, uk, args.addr_weight != 0)
            kernels[name] = {"avg_us": avg_us, "launches": n,
                             "alg_bytes": byts, "alg_gbps": byts / (avg_us * 1e3) if byts else None,
                             "alg_tflops": flops / (avg_us * 1e6) if flops else None,
                             "hbm_bytes_counted": traffic.get(name)}
        result["kernels"] = kernels
        result["unique_rows_per_launch"] = {"v": uv, "k1_plus_k2": uk,
                                            "pairs": B * H * C * cfg.topk}
        # the gather (read) and scatter (update) against the HBM peak:
        # algorithmic bytes, and counted HBM bytes beside them; where the
        # counters read fewer bytes than the algorithm names, caches served
        # the rest and the algorithmic figure is an "effective" bandwidth
        hbm = {}
        for role, name in (("gather", "read"), ("scatter", "update")):
            if name not in kernels:
                continue
            kd = kernels[name]
            e = {"kernel": name, "avg_us": kd["avg_us"], "alg_bytes": kd["alg_bytes"],
                 "alg_gbps": kd["alg_gbps"], "alg_frac": kd["alg_gbps"] / HBM_PEAK_GBPS}
            cnt = kd["hbm_bytes_counted"]
            if cnt is not None:
                e.update(counted_bytes=cnt, counted_gbps=cnt / (kd["avg_us"] * 1e3),
                         counted_frac=cnt / (kd["avg_us"] * 1e3) / HBM_PEAK_GBPS)
                e["alg_label"] = "effective" if cnt < kd["alg_bytes"] else "hbm"
            else:
                e["alg_label"] = "algorithmic (no fresh counters)"
            hbm[role] = e
        result["hbm"] = hbm
        dom = max(kernels, key=lambda k: kernels[k]["avg_us"])
        kd = kernels[dom]
        if kd["alg_tflops"] is not None and dom in ("score", "addr_grad", "project"):
            roof = {"bound": "mfma", "achieved": kd["alg_tflops"], "peak": FP32_MFMA_PEAK_TFLOPS,
                    "unit": "TFLOP/s"}
        else:
            roof = {"bound": "hbm", "achieved": kd["alg_gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s"}
        roof["frac"] = roof["achieved"] / roof["peak"]
        roof["traffic"] = traffic.get(dom)
        roof["kernel"] = dom
        result["roofline"] = roof

    if not args.no_cpu_baseline:
        print(f"[bench] CPU oracle baseline (~{args.cpu_seconds:.0f} s)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = (cpu_baseline_sequence(cfg, tables, X, lw, args.cpu_seconds)
                                  if args.sequence else cpu_baseline(cfg, tables, Q, Y, args.cpu_seconds))
        if not (args.sequence or args.weighted or args.addr_weight):
            units = sorted({0, cfg.units - 1})
            print(f"[bench] parity of the first pass against the oracle on units {units}",
                  file=sys.stderr, flush=True)
            result["parity"] = parity_leg(cfg, tables, Q, Y, mem, st, restore, qd, yd, units)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
