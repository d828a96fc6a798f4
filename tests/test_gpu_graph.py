"""Chunk calls captured into a HIP graph replay to exactly the eager results.

The benchmark times a step (every chunk of a pass, chained in place) as one
graph replay.  This test captures a three-chunk chain of a clustered
workload, restores the starting tables between replays with eager copies,
runs unrelated eager chunk calls and synchronisations between the replays,
and checks every replay bit for bit against the eager chain: the kernels are
deterministic, so a graph that replays correctly reproduces them exactly.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from workloads import WorkloadConfig, draw_queries, draw_targets, initial_tables

pytestmark = pytest.mark.gpu

CFG = WorkloadConfig(index=61, name="graph-2x384-n64-d128-k8-clustered", batch=2, heads=2,
                     chunk=128, chunks=3, passes=1, sqrt_slots=64, dim_qk=128, dim_v=96,
                     topk=8, query_kind="clustered", clusters=8)


def _inputs(cfg):
    tables = initial_tables(cfg)
    B, H, C = cfg.batch, cfg.heads, cfg.chunk
    Q = draw_queries(cfg).reshape(B, cfg.chunks, C, H, cfg.dim_qk).transpose(1, 0, 2, 3, 4)
    Y = draw_targets(cfg).reshape(B, cfg.chunks, C, H, cfg.dim_v).transpose(1, 0, 2, 3, 4)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    start = [dev(np.repeat(a[None], B, axis=0)) for a in (tables.k1, tables.k2, tables.v)]
    return start, dev(Q), dev(Y)


def test_graph_replays_match_eager(fwpkm_lib):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from sparse_weight_memory_amd import Config, Memory, State
    cfg = CFG
    B, H, C = cfg.batch, cfg.heads, cfg.chunk
    mem = Memory(Config(sqrt_slots=cfg.sqrt_slots, dim_qk=cfg.dim_qk, dim_v=cfg.dim_v,
                        topk=cfg.topk, chunk_size=C, num_heads=H, max_batch=B, eps=cfg.eps))
    start, qd, yd = _inputs(cfg)

    def chain(st, rets):
        for c in range(cfg.chunks):
            mem.forward_chunk(qd[c], yd[c], cfg.lr, st, next=st, retrieved=rets[c])

    # eager reference (also allocates the library workspace before capture)
    ref_st = State(*(t.clone() for t in start))
    ref_rets = [torch.empty((B, C, H, cfg.dim_v), device="cuda") for _ in range(cfg.chunks)]
    chain(ref_st, ref_rets)
    torch.cuda.synchronize()

    st = State(*(t.clone() for t in start))
    rets = [torch.empty_like(r) for r in ref_rets]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chain(st, rets)
    torch.cuda.synchronize()

    other = State(*(t.clone() for t in start))
    for rep in range(4):
        print(f"[graph] replay {rep}", flush=True)
        for dst, src in zip(st, start):
            dst.copy_(src)
        for r in rets:
            r.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for c in range(cfg.chunks):
            assert torch.equal(rets[c], ref_rets[c]), f"replay {rep}: chunk {c} retrieved differs"
        for name, a, b in zip(("k1", "k2", "v"), st, ref_st):
            assert torch.equal(a, b), f"replay {rep}: table {name} differs"
        # unrelated eager work on the same handle between replays
        mem.forward_chunk(qd[rep % cfg.chunks], yd[rep % cfg.chunks], cfg.lr, other, next=other)
        torch.cuda.synchronize()
