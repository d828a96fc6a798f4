"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (every unit of the batch in one call, state updated in place).

The oracle covers sampled units (units are independent memories, so a unit's
result does not depend on the others) for every chunk it can afford, chained
(each side runs its own chain) and teacher-forced (the oracle restarts every
chunk from a host copy of the GPU's tables); the streams are also checked
teacher-forced through their second pass, the state a repeated stream
leaves.
"""

import numpy as np
import pytest
import torch

from oracle import fwpkm_oracle as O
from parity_helpers import (ATOL_CHAIN, ATOL_CHUNK, RTOL_CHAIN, RTOL_CHUNK, assert_close,
                            compare_chunk, mirror_units, need_gpu, oracle_units, say,
                            selection_overrides, state_to_host, teacher_forced_step, to_dev)
from workloads import chunk_inputs, draw_queries, draw_targets, get_config, initial_tables

pytestmark = pytest.mark.gpu


def _mem_for(w):
    from sparse_weight_memory_amd import Config, Memory
    return Memory(Config(sqrt_slots=w.sqrt_slots, dim_qk=w.dim_qk, dim_v=w.dim_v, topk=w.topk,
                         chunk_size=w.chunk, num_heads=w.heads, max_batch=w.batch, eps=w.eps))


def _device_state(tables, B):
    from sparse_weight_memory_amd import State
    return State(*(torch.from_numpy(a).cuda().unsqueeze(0).repeat(B, *([1] * a.ndim)).contiguous()
                   for a in (tables.k1, tables.k2, tables.v)))


def _host_units(tables, units, H):
    """Oracle-layout state of the given units from the shared initial tables."""
    return {name: np.stack([getattr(tables, name)[u % H] for u in units])
            for name in ("k1", "k2", "v")}


def _chained(w, units, chunks, check_every_chunk=True):
    """Run `chunks` chunks on the GPU (all units) and the oracle (sampled units)."""
    mem = _mem_for(w)
    tables = initial_tables(w)
    Q, Y = draw_queries(w), draw_targets(w)
    dev = _device_state(tables, w.batch)
    ost = _host_units(tables, units, w.heads)
    ties = 0
    for c in range(chunks):
        ci = chunk_inputs(Q, Y, w, c % w.chunks)
        say(w.name, "chunk", c)
        ret, dev, slots, _ = mem.forward_chunk(to_dev(ci.queries), to_dev(ci.targets), w.lr, dev,
                                               next=dev, return_selection=True)
        slots = slots.cpu().numpy()
        rets, new, res = oracle_units(ost, ci.queries, ci.targets, w.lr, w.topk, w.eps, O.IDW,
                                      units, w.heads)
        ov, nt = selection_overrides(res, slots, w.heads, units)
        ties += nt
        if ov:
            rets, new, res = oracle_units(ost, ci.queries, ci.targets, w.lr, w.topk, w.eps, O.IDW,
                                          units, w.heads, ov)
        ost = new
        if check_every_chunk or c == chunks - 1:
            r = ret.cpu().numpy()
            for u in units:
                b, h = divmod(u, w.heads)
                assert_close(f"{w.name} c{c} retrieved u{u}", r[b, :, h], rets[u], RTOL_CHAIN, ATOL_CHAIN)
    got = state_to_host(dev, units)
    for name in ("k1", "k2", "v"):
        assert_close(f"{w.name} after {chunks} chunks: {name}", got[name], ost[name],
                     RTOL_CHAIN, ATOL_CHAIN)
    say(w.name, "near-ties", ties)
    return mem, dev, Q, Y


def test_library_default_shape_single_chunk_full():
    """65,536 slots, d_qk = d_v = 512, top-8, batch 2 x 256: every unit, every output."""
    need_gpu()
    w = get_config(2)
    mem = _mem_for(w)
    tables = initial_tables(w)
    st = _host_units(tables, range(w.units), w.heads)
    ci = chunk_inputs(draw_queries(w), draw_targets(w), w, 0)
    compare_chunk(mem, st, ci.queries, ci.targets, w.lr, label=w.name)


def _teacher_forced_pass(mem, dev, Q, Y, w, units, chunks, label):
    """Chunks 0..chunks-1 of a pass on the GPU (all units, in place), each
    checked teacher-forced on `units` from a host mirror of the GPU tables."""
    mirror = mirror_units(dev, units)
    ties, worst = 0, {}
    for c in range(chunks):
        ci = chunk_inputs(Q, Y, w, c)
        nt, wc = teacher_forced_step(mem, dev, mirror, units, ci.queries, ci.targets, w.lr,
                                     label=f"{label} c{c}")
        ties += nt
        for key, val in wc.items():
            worst[key] = max(worst.get(key, 0.0), val)
    say(label, "near-ties", ties, "worst error / tolerance", worst)
    return ties


def test_training_length_stream_sampled_units():
    """8 sequences x 4096 clustered tokens, 16 chained chunks; units 0 and 5
    chained, then every unit teacher-forced through the first pass from the
    initial tables (the benchmark's timed state) and through a second pass
    of the same stream."""
    need_gpu()
    w = get_config(3)
    _chained(w, units=[0, 5], chunks=w.chunks)
    mem = _mem_for(w)
    tables = initial_tables(w)
    Q, Y = draw_queries(w), draw_targets(w)
    dev = _device_state(tables, w.batch)
    units = list(range(w.units))
    _teacher_forced_pass(mem, dev, Q, Y, w, units, w.chunks, f"{w.name} pass1")
    _teacher_forced_pass(mem, dev, Q, Y, w, units, w.chunks, f"{w.name} pass2")


def test_multihead_stream_sampled_units():
    """4 heads x 262,144 slots, top-16, batch 4 x 8192 tokens; units (0,0)
    and (2,3) chained with every chunk's retrieved checked, then every unit
    (two per XCD, each through its own place in the separate grouping and
    update kernels' unit-major grids) teacher-forced through the first two
    chunks."""
    need_gpu()
    w = get_config(4)
    _chained(w, units=[0, 11], chunks=w.chunks, check_every_chunk=True)
    mem = _mem_for(w)
    Q, Y = draw_queries(w), draw_targets(w)
    dev = _device_state(initial_tables(w), w.batch)
    _teacher_forced_pass(mem, dev, Q, Y, w, list(range(w.units)), 2, f"{w.name} tf")


def test_long_context_two_passes():
    """1 x 131,072 tokens over 2^20 slots, read twice: the first 16 chunks
    chained, then the rest of the first pass on the GPU and the second
    pass's first 16 chunks teacher-forced from the GPU state."""
    need_gpu()
    w = get_config(5)
    mem, dev, Q, Y = _chained(w, units=[0], chunks=16)
    for c in range(16, w.chunks):
        ci = chunk_inputs(Q, Y, w, c)
        mem.forward_chunk(to_dev(ci.queries), to_dev(ci.targets), w.lr, dev, next=dev)
    torch.cuda.synchronize()
    say(w.name, "first pass done on the GPU; second pass, 16 chunks, teacher-forced")
    _teacher_forced_pass(mem, dev, Q, Y, w, [0], 16, f"{w.name} pass2")
