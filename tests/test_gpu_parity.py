"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Small and edge-case shapes, every chunk compared in full, plus GPU
properties: determinism, lr = 0, in-place vs copy, shared-state expansion,
unit independence and checkpoint/resume.
"""

import zlib

import numpy as np
import pytest
import torch

from oracle import fwpkm_oracle as O
from parity_helpers import (ATOL_CHAIN, ATOL_CHUNK, RTOL_CHAIN, RTOL_CHUNK, assert_close,
                            compare_chunk, need_gpu, oracle_units, say, selection_overrides,
                            state_to_dev, state_to_host, to_dev)
from workloads import chunk_inputs, draw_queries, draw_targets, get_config, initial_tables
from workloads.generate import expand_tables

pytestmark = pytest.mark.gpu


def _mem(**kw):
    from sparse_weight_memory_amd import Config, Memory
    return Memory(Config(**kw))


def _random_case(seed, B, H, C, n, half, dv, q_std=1.0):
    rng = np.random.default_rng(seed)
    U = B * H
    st = {"k1": (rng.standard_normal((U, n, half)) / np.sqrt(half)).astype(np.float32),
          "k2": (rng.standard_normal((U, n, half)) / np.sqrt(half)).astype(np.float32),
          "v": (rng.standard_normal((U, n * n, dv)) * 0.14).astype(np.float32)}
    q = (rng.standard_normal((B, C, H, 2 * half)) * q_std).astype(np.float32)
    y = rng.standard_normal((B, C, H, dv)).astype(np.float32)
    return st, q, y


def _workload_state(cfg):
    t = initial_tables(cfg)
    ex = expand_tables(t, cfg.batch)
    return {"k1": ex.k1, "k2": ex.k2, "v": ex.v}


# ------------------------------------------------------------ tiny workload

def test_tiny_workload_teacher_forced_every_chunk():
    need_gpu()
    w = get_config(1)
    mem = _mem(sqrt_slots=w.sqrt_slots, dim_qk=w.dim_qk, dim_v=w.dim_v, topk=w.topk,
               chunk_size=w.chunk, num_heads=w.heads, max_batch=w.batch, eps=w.eps)
    st = _workload_state(w)
    Q, Y = draw_queries(w), draw_targets(w)
    total_ties = 0
    for c in range(w.chunks):
        ci = chunk_inputs(Q, Y, w, c)
        st, ties, _ = compare_chunk(mem, st, ci.queries, ci.targets, w.lr, label=f"tiny c{c}")
        total_ties += ties
    say("tiny near-ties", total_ties)


def test_tiny_workload_chained():
    need_gpu()
    w = get_config(1)
    mem = _mem(sqrt_slots=w.sqrt_slots, dim_qk=w.dim_qk, dim_v=w.dim_v, topk=w.topk,
               chunk_size=w.chunk, num_heads=w.heads, max_batch=w.batch, eps=w.eps)
    st0 = _workload_state(w)
    Q, Y = draw_queries(w), draw_targets(w)
    dev = state_to_dev(st0, w.batch, w.heads)
    ost = {k: v.copy() for k, v in st0.items()}
    for c in range(w.chunks):
        ci = chunk_inputs(Q, Y, w, c)
        ret, dev, slots, _ = mem.forward_chunk(to_dev(ci.queries), to_dev(ci.targets), w.lr, dev,
                                               next=dev, return_selection=True)
        slots = slots.cpu().numpy()
        rets, new, res = oracle_units(ost, ci.queries, ci.targets, w.lr, w.topk, w.eps, O.IDW, [0], 1)
        ov, _ = selection_overrides(res, slots, 1, [0])
        if ov:
            rets, new, res = oracle_units(ost, ci.queries, ci.targets, w.lr, w.topk, w.eps, O.IDW, [0], 1, ov)
        ost = new
    got = state_to_host(dev)
    assert_close("chained retrieved", ret.cpu().numpy()[0, :, 0], rets[0], RTOL_CHAIN, ATOL_CHAIN)
    for name in ("k1", "k2", "v"):
        assert_close(f"chained {name}", got[name], ost[name], RTOL_CHAIN, ATOL_CHAIN)


# ------------------------------------------------------------ edge shapes

EDGE = [
    # (label, B, H, C_max, T, n, half, dv, k, mode)
    ("ragged-tail", 2, 1, 64, 37, 16, 8, 12, 3, "idw"),
    ("one-token", 1, 1, 64, 1, 8, 4, 8, 2, "idw"),
    ("k-equals-n", 1, 1, 32, 32, 6, 4, 8, 6, "idw"),
    ("k1", 2, 2, 40, 40, 12, 4, 8, 1, "idw"),
    ("n-not-multiple", 1, 2, 48, 48, 300, 20, 36, 5, "idw"),
    ("wide-dv", 1, 1, 32, 32, 16, 8, 1040, 4, "idw"),
    ("k16-two-blocks", 1, 1, 64, 64, 520, 16, 64, 16, "idw"),
    ("k24-fallback", 1, 1, 32, 32, 64, 8, 32, 24, "idw"),
    ("k32-max", 1, 1, 32, 32, 40, 4, 600, 32, "idw"),
    # per-block lists merged across the whole wave (2 KMAX = 64 lanes), four
    # 64-key blocks with a ragged last one; and k below KMAX, whose lanes
    # k..KMAX-1 must stay empty between merges
    ("k32-four-blocks", 1, 1, 32, 32, 200, 4, 64, 32, "idw"),
    ("k20-three-blocks-dot", 1, 1, 48, 48, 150, 8, 16, 20, "dot"),
    ("dot-small", 2, 1, 64, 64, 16, 8, 12, 4, "dot"),
    ("dot-k16", 1, 2, 64, 50, 64, 16, 32, 16, "dot"),
    # keys staged straight into LDS: 128-key blocks (two dim shares), and
    # 256-key blocks with a ragged last block and token tile
    ("direct-staging-blk128", 4, 1, 256, 256, 256, 256, 64, 8, "idw"),
    ("direct-staging-ragged-dot", 8, 1, 256, 200, 300, 128, 32, 8, "dot"),
    # work-item decompositions by divisors that are not powers of two: three
    # heads over 24 units (3 units per XCD, ragged token tiles and read
    # workgroups), two key blocks of a 100-key half, and five heads over 5
    # units (the plain unit order)
    ("heads3-units24", 8, 3, 64, 37, 64, 16, 32, 4, "idw"),
    ("heads3-two-blocks-dot", 8, 3, 64, 50, 100, 8, 16, 8, "dot"),
    ("heads5-units5", 1, 5, 80, 70, 40, 8, 24, 6, "idw"),
]


@pytest.mark.parametrize("case", EDGE, ids=[c[0] for c in EDGE])
def test_edge_shapes(case):
    need_gpu()
    label, B, H, Cmax, T, n, half, dv, k, mode = case
    mem = _mem(sqrt_slots=n, dim_qk=2 * half, dim_v=dv, topk=k, chunk_size=Cmax, num_heads=H,
               max_batch=B + 1, score_mode=mode)
    st, q, y = _random_case(zlib.crc32(label.encode()) % 1000, B, H, T, n, half, dv)
    for c, lr in enumerate((1.0, 0.5)):
        st, _, _ = compare_chunk(mem, st, q, y, lr, label=f"{label} step{c}")


@pytest.mark.parametrize("k", [8, 16])
def test_two_token_selection_odd_tail_and_mass_ties(k):
    """256-key blocks select two tokens per wave.  249 tokens leave a last
    tile of 9, so one wave serves a real token and one past the chunk.  With
    the first sub-key table made of 4 distinct rows repeated 64 times, each
    lane's candidates are copies of one row, the best values tie across 64
    keys, and a token's survivors (64 or 128) overflow the 32 lanes: it takes
    the whole-wave path.  Every token is then an exact float64 tie at the
    k-th place, and the validity check accepts only the lower-slot choice among
    exactly tied candidates, so the path's selection is checked bit for bit."""
    need_gpu()
    B, H, T, n, half, dv = 8, 1, 249, 256, 16, 16
    mem = _mem(sqrt_slots=n, dim_qk=2 * half, dim_v=dv, topk=k, chunk_size=256, num_heads=H, max_batch=B)
    st, q, y = _random_case(4242 + k, B, H, T, n, half, dv)
    compare_chunk(mem, st, q, y, 1.0, units=[0, 7], label=f"odd tail k{k}")
    st, q, y = _random_case(4343 + k, B, H, T, n, half, dv)
    st["k1"] = np.ascontiguousarray(np.tile(st["k1"][:, :4], (1, n // 4, 1)))
    compare_chunk(mem, st, q, y, 1.0, units=[0, 3, 7], label=f"mass ties k{k}")


@pytest.mark.parametrize("C", [32, 33])
def test_grouping_at_the_rank_sort_limit(C):
    """48 units leave one hash region per list, so every unit's V list holds
    exactly C*k entries: 256 (the largest region sorted by ranking) or 264
    (the radix sort); the K lists hold fewer entries, with 5-bit rows."""
    need_gpu()
    B, H, n, half, dv, k = 48, 1, 32, 8, 16, 8
    mem = _mem(sqrt_slots=n, dim_qk=2 * half, dim_v=dv, topk=k, chunk_size=C, num_heads=H, max_batch=B)
    st, q, y = _random_case(900 + C, B, H, C, n, half, dv)
    compare_chunk(mem, st, q, y, 1.0, units=[0, 11, 30, 47], label=f"rank-limit C{C}")


@pytest.mark.parametrize("mode", ["idw", "dot"])
def test_long_segments_split_into_pieces(mode):
    """Every token asks the same few queries, so each touched row is hit by
    dozens of tokens: its gradient is summed over several pieces."""
    need_gpu()
    B, H, C, n, half, dv, k = 2, 1, 200, 24, 8, 20, 6
    mem = _mem(sqrt_slots=n, dim_qk=2 * half, dim_v=dv, topk=k, chunk_size=C, num_heads=H,
               max_batch=B, score_mode=mode)
    st, q, y = _random_case(77, B, H, C, n, half, dv)
    q[:] = q[:, [t % 3 for t in range(C)]]             # three distinct queries per sequence
    for c, lr in enumerate((1.0, 0.3)):
        st, _, _ = compare_chunk(mem, st, q, y, lr, label=f"long-segments {mode} step{c}")


@pytest.mark.parametrize("C,mode", [(300, "idw"), (700, "idw"), (700, "dot")])
def test_update_geometry_at_wide_chunks(C, mode):
    """Chunks of more than 256 and 512 tokens narrow the update's column
    slices (32 and 16 floats); with 8 units and d_v 256 each workgroup then
    owns a whole list, whose 2,400 or 5,600 entries pass in batches cut at
    segment heads.  Half the tokens repeat 4 queries (rows touched by 38 or
    88 tokens: multi-piece segments summed across waves), the rest are
    distinct (one-token segments packed several to a wave pass)."""
    need_gpu()
    B, H, n, half, dv, k = 8, 1, 64, 64, 256, 8
    mem = _mem(sqrt_slots=n, dim_qk=2 * half, dim_v=dv, topk=k, chunk_size=C, num_heads=H,
               max_batch=B, score_mode=mode)
    st, q, y = _random_case(600 + C + (mode == "dot"), B, H, C, n, half, dv)
    rep = np.arange(C) % 2 == 0
    q[:, rep] = q[:, [t % 8 for t in range(C) if rep[t]]]
    compare_chunk(mem, st, q, y, 1.0, units=[0, 3, 7], label=f"wide C{C} {mode}")


@pytest.mark.parametrize("fresh", [0, 8])
def test_grouping_renames_hot_rows(fresh):
    """One sequence of 1,024 tokens, n = 512, k = 8: 8,192 pairs per unit take
    the separate grouping kernel, and with every token asking the same query
    (or all but every fresh-th token) each selected value slot (18 bits) and
    sub-key row (9 bits) is hit by hundreds of tokens.  Their regions hold
    hundreds of entries over a few distinct rows, which are renamed to their
    ranks and sorted in one radix pass; the fresh tokens' rows mix cold rows
    into the same regions."""
    need_gpu()
    B, H, C, n, half, dv, k = 1, 1, 1024, 512, 8, 16, 8
    mem = _mem(sqrt_slots=n, dim_qk=2 * half, dim_v=dv, topk=k, chunk_size=C, num_heads=H, max_batch=B)
    st, q, y = _random_case(1100 + fresh, B, H, C, n, half, dv)
    q[:] = q[:, [t if fresh and t % fresh == 0 else 0 for t in range(C)]]
    compare_chunk(mem, st, q, y, 1.0, label=f"hot rows, fresh every {fresh}")


@pytest.mark.parametrize("C,k", [(300, 4), (700, 2)])
def test_fused_update_at_narrow_slices(C, k):
    """At most 2,048 pairs per unit keep the grouping inside the update
    kernel while chunks of more than 256 and 512 tokens narrow its column
    slices to 32 and 16 floats: the sub-key lists (n = 64, one radix pass)
    take their segment tables straight from the digit counts there, and the
    value rows (12 bits) go through two passes.  Half the tokens repeat 4
    queries, as above."""
    need_gpu()
    B, H, n, half, dv = 8, 1, 64, 64, 256
    mem = _mem(sqrt_slots=n, dim_qk=2 * half, dim_v=dv, topk=k, chunk_size=C, num_heads=H,
               max_batch=B)
    st, q, y = _random_case(800 + C + k, B, H, C, n, half, dv)
    rep = np.arange(C) % 2 == 0
    q[:, rep] = q[:, [t % 8 for t in range(C) if rep[t]]]
    compare_chunk(mem, st, q, y, 1.0, units=[0, 3, 7], label=f"narrow C{C} k{k}")


@pytest.mark.parametrize("k,distinct,seed", [(1, 256, 3010), (2, 129, 3022)])
def test_fused_grouping_at_the_row_mask_limit(k, distinct, seed):
    """With 16 units, d_h = 512 and d_v = 64, one hash group per list already
    gives the update a workgroup per compute unit, so a unit's whole value
    list is one group.  256 tokens asking 256 distinct queries with k = 1 give
    unit 0 exactly 256 distinct value rows, the most the per-row token masks
    take (unit 15: 255); 129 distinct queries with k = 2 give 258 (unit 0) and
    257 (unit 15), which the radix sort groups instead, after the bitmap of
    the rows present has counted them."""
    need_gpu()
    B, H, C, n, half, dv = 16, 1, 256, 256, 512, 64
    units = [0, 15]
    mem = _mem(sqrt_slots=n, dim_qk=2 * half, dim_v=dv, topk=k, chunk_size=C, num_heads=H, max_batch=B)
    st, q, y = _random_case(seed, B, H, C, n, half, dv)
    q[:] = q[:, [t if t < distinct else t % distinct for t in range(C)]]
    rows = [len(np.unique(O.unit_chunk(st["k1"][u], st["k2"][u], st["v"][u], q[u, :, 0], y[u, :, 0],
                                       1.0, k, mem.cfg.eps, O.IDW).slots)) for u in units]
    assert rows == ([256, 255] if k == 1 else [258, 257]), rows
    compare_chunk(mem, st, q, y, 1.0, units=units, label=f"row-mask limit k{k} rows {rows}")


def test_closed_form_k1_single_token_writes_target():
    need_gpu()
    n, half, dv = 16, 8, 32
    mem = _mem(sqrt_slots=n, dim_qk=2 * half, dim_v=dv, topk=1, chunk_size=8)
    st, q, y = _random_case(5, 1, 1, 1, n, half, dv)
    dev = state_to_dev(st, 1, 1)
    _, nxt, slots, w = mem.forward_chunk(to_dev(q), to_dev(y), 1.0, dev, next=dev, return_selection=True)
    hit = int(slots[0, 0, 0, 0])
    assert float(w[0, 0, 0, 0]) == 1.0
    # in fp32 the step is V - (V - y): exact up to the rounding of V - y
    got = nxt.v[0, 0, hit].cpu().numpy().astype(np.float64)
    bound = 2 * np.finfo(np.float32).eps * (np.abs(y[0, 0, 0]) + np.abs(st["v"][0, hit]))
    assert np.all(np.abs(got - y[0, 0, 0]) <= bound)


# ------------------------------------------------------------ properties

def _small_mem_and_case(seed=11, B=3, H=2, C=64, n=32, half=16, dv=64, k=4):
    mem = _mem(sqrt_slots=n, dim_qk=2 * half, dim_v=dv, topk=k, chunk_size=C, num_heads=H, max_batch=B)
    return mem, _random_case(seed, B, H, C, n, half, dv)


def test_lr_zero_leaves_state_bitwise_and_reads_match():
    need_gpu()
    mem, (st, q, y) = _small_mem_and_case()
    dev = state_to_dev(st, 3, 2)
    before = [t.clone() for t in dev]
    ret, nxt = mem.forward_chunk(to_dev(q), to_dev(y), 0.0, dev, next=dev)
    for a, b in zip(before, nxt):
        assert torch.equal(a, b)
    compare_chunk(mem, st, q, y, 0.0, label="lr0")


def test_repeat_runs_are_bitwise_identical():
    need_gpu()
    mem, (st, q, y) = _small_mem_and_case(seed=12)
    outs = []
    for _ in range(3):
        dev = state_to_dev(st, 3, 2)
        ret, nxt = mem.forward_chunk(to_dev(q), to_dev(y), 1.0, dev, next=dev)
        torch.cuda.synchronize()
        outs.append((ret.cpu(), [t.cpu() for t in nxt]))
    for ret, tabs in outs[1:]:
        assert torch.equal(ret, outs[0][0])
        for a, b in zip(tabs, outs[0][1]):
            assert torch.equal(a, b)


def test_in_place_equals_copy_mode_and_shared_expansion():
    need_gpu()
    from sparse_weight_memory_amd import State
    mem, (st, q, y) = _small_mem_and_case(seed=13)
    # shared initial tables: make every sequence's tables equal to sequence 0's
    B, H = 3, 2
    for name in st:
        per = st[name].reshape(B, H, *st[name].shape[1:])
        per[:] = per[0:1]
    dev = state_to_dev(st, B, H)
    r1, n1 = mem.forward_chunk(to_dev(q), to_dev(y), 1.0, dev, next=dev)       # in place
    shared = State(to_dev(st["k1"].reshape(B, H, *st["k1"].shape[1:])[0]),
                   to_dev(st["k2"].reshape(B, H, *st["k2"].shape[1:])[0]),
                   to_dev(st["v"].reshape(B, H, *st["v"].shape[1:])[0]))
    keep = [t.clone() for t in shared]
    r2, n2 = mem.forward_chunk(to_dev(q), to_dev(y), 1.0, shared)              # copy + expand
    torch.cuda.synchronize()
    assert torch.equal(r1, r2)
    for a, b in zip(n1, n2):
        assert torch.equal(a, b)
    for a, b in zip(keep, shared):                                             # past untouched
        assert torch.equal(a, b)


def test_units_are_independent_on_gpu():
    need_gpu()
    mem, (st, q, y) = _small_mem_and_case(seed=14)
    dev1 = state_to_dev(st, 3, 2)
    r1, n1 = mem.forward_chunk(to_dev(q), to_dev(y), 1.0, dev1, next=dev1)
    q2, y2 = q.copy(), y.copy()
    q2[1, :, 1] += 0.5
    y2[1, :, 1] -= 1.0
    dev2 = state_to_dev(st, 3, 2)
    r2, n2 = mem.forward_chunk(to_dev(q2), to_dev(y2), 1.0, dev2, next=dev2)
    torch.cuda.synchronize()
    for (b, h) in [(0, 0), (0, 1), (1, 0), (2, 0), (2, 1)]:
        assert torch.equal(r1[b, :, h], r2[b, :, h])
        for a, c in zip(n1, n2):
            assert torch.equal(a[b, h], c[b, h])
    assert not torch.equal(r1[1, :, 1], r2[1, :, 1])


def test_checkpoint_resume_is_bitwise():
    need_gpu()
    from sparse_weight_memory_amd import State
    w = get_config(1)
    mem = _mem(sqrt_slots=w.sqrt_slots, dim_qk=w.dim_qk, dim_v=w.dim_v, topk=w.topk,
               chunk_size=w.chunk, max_batch=1)
    st0 = _workload_state(w)
    Q, Y = draw_queries(w), draw_targets(w)
    chunks = [chunk_inputs(Q, Y, w, c) for c in range(w.chunks)]
    a = state_to_dev(st0, 1, 1)
    for ci in chunks:
        ra, a = mem.forward_chunk(to_dev(ci.queries), to_dev(ci.targets), 1.0, a, next=a)
    b = state_to_dev(st0, 1, 1)
    for ci in chunks[:2]:
        rb, b = mem.forward_chunk(to_dev(ci.queries), to_dev(ci.targets), 1.0, b, next=b)
    saved = [t.cpu().numpy().copy() for t in b]                                 # "checkpoint"
    del b
    b = State(*[to_dev(x) for x in saved])
    for ci in chunks[2:]:
        rb, b = mem.forward_chunk(to_dev(ci.queries), to_dev(ci.targets), 1.0, b, next=b)
    torch.cuda.synchronize()
    assert torch.equal(ra, rb)
    for x, z in zip(a, b):
        assert torch.equal(x, z)


def test_errors_leave_outputs_untouched():
    need_gpu()
    from sparse_weight_memory_amd import FwPKMError
    mem, (st, q, y) = _small_mem_and_case(seed=15)
    dev = state_to_dev(st, 3, 2)
    ret = torch.full((3, 64, 2, 64), 7.0, device="cuda")
    with pytest.raises(FwPKMError) as ei:
        mem.forward_chunk(to_dev(q), to_dev(y), float("nan"), dev, next=dev, retrieved=ret)
    assert ei.value.code == -1
    torch.cuda.synchronize()
    assert bool((ret == 7.0).all())
