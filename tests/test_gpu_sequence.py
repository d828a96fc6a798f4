"""GPU parity of the sequence layer (fwpkm_forward_sequence) against the
oracle's sequence layer, through the C ABI.

Protocol: the GPU runs the whole sequence; the oracle runs it from the same
fp32 inputs.  Selected slots are compared per chunk; where they differ the
oracle must report a near-tie, and it then adopts the GPU's set for that
token and runs again (later chunks depend on it).  Outputs and final tables
must agree to the chained-step tolerance.  Memory units are independent, so
at the full benchmark shape the oracle follows one unit's whole chain.
"""

import numpy as np
import pytest
import torch

from oracle import fwpkm_sequence as OS
from parity_helpers import (ATOL_CHAIN, RTOL_CHAIN, assert_close, mode_name, need_gpu, say,
                            selection_overrides, state_to_dev, state_to_host, to_dev)

pytestmark = pytest.mark.gpu


def _mem(**kw):
    from sparse_weight_memory_amd import Config, Memory
    return Memory(Config(**kw))


def _case(seed, B, S, H, n, dqk, dv, x_std=1.0):
    rng = np.random.default_rng(seed)
    U, D = B * H, H * dv
    st = {"k1": (rng.standard_normal((U, n, dqk // 2)) / np.sqrt(dqk // 2)).astype(np.float32),
          "k2": (rng.standard_normal((U, n, dqk // 2)) / np.sqrt(dqk // 2)).astype(np.float32),
          "v": (rng.standard_normal((U, n * n, dv)) * 0.14).astype(np.float32)}
    x = (rng.standard_normal((B, S, D)) * x_std).astype(np.float32)
    w_in = (rng.standard_normal((H * (dqk + dv), D)) / np.sqrt(D)).astype(np.float32)
    w_gate = (rng.standard_normal((H, D)) / np.sqrt(D)).astype(np.float32)
    b_gate = rng.standard_normal(H).astype(np.float32)
    return st, x, w_in, w_gate, b_gate


def run_gpu(mem, st, x, w_in, w_gate, b_gate, lr):
    B, H = x.shape[0], mem.cfg.num_heads
    dev = state_to_dev(st, B, H)
    say("gpu sequence", dict(B=B, S=x.shape[1], H=H, D=x.shape[2], n=mem.cfg.sqrt_slots,
                             k=mem.cfg.topk, C=mem.cfg.chunk_size, lr=lr))
    out, nxt, slots, _ = mem.forward_sequence(
        to_dev(x), to_dev(w_in), to_dev(w_gate), None if b_gate is None else to_dev(b_gate),
        lr, dev, next=dev, return_selection=True)
    torch.cuda.synchronize()
    return out.cpu().numpy(), state_to_host(nxt), slots.cpu().numpy()


def oracle_with_ties(cfg, st, x, w_in, w_gate, b_gate, lr, gpu_slots):
    """The oracle's sequence, adopting the GPU's selection at near-ties."""
    B, S, _ = x.shape
    H, C = cfg.num_heads, cfg.chunk_size
    units = list(range(B * H))
    overrides, ties = {}, 0
    for _ in range((S + C - 1) // C + 1):
        out, nxt, results = OS.forward_sequence(st, x, w_in, w_gate, b_gate, lr, cfg.topk, C,
                                                cfg.eps, mode_name(cfg.score_mode), overrides)
        changed = False
        for c, res in enumerate(results):
            ov, nt = selection_overrides(res, gpu_slots[:, c * C:(c + 1) * C], H, units)
            if ov:
                for u, toks in ov.items():
                    overrides.setdefault(c, {}).setdefault(u, {}).update(toks)
                ties += nt
                changed = True
                break          # later chunks depend on this one: run again
        if not changed:
            return out, nxt, ties
    raise AssertionError("near-tie adoption did not settle")


def compare_sequence(mem, st, x, w_in, w_gate, b_gate, lr, label):
    out, nxt, slots = run_gpu(mem, st, x, w_in, w_gate, b_gate, lr)
    say(label, "oracle")
    o_out, o_nxt, ties = oracle_with_ties(mem.cfg, st, x, w_in, w_gate, b_gate, lr, slots)
    say(label, "near-ties adopted:", ties)
    assert_close(f"{label} out", out, o_out, RTOL_CHAIN, ATOL_CHAIN)
    for name in ("k1", "k2", "v"):
        assert_close(f"{label} next {name}", nxt[name], o_nxt[name], RTOL_CHAIN, ATOL_CHAIN)
    return out, nxt


@pytest.mark.parametrize("mode,x_std", [("idw", 1.0), ("dot", 0.5)])
def test_sequence_matches_oracle(mode, x_std):
    """Three chunks (64, 64, 22 tokens), two heads; every projection tile
    ragged (300 tokens, 56 features, 24 input features)."""
    need_gpu()
    B, S, H, n, dqk, dv, k, C = 2, 150, 2, 32, 16, 12, 4, 64
    mem = _mem(sqrt_slots=n, dim_qk=dqk, dim_v=dv, topk=k, chunk_size=C, num_heads=H,
               max_batch=B, score_mode=mode)
    st, x, w_in, w_gate, b_gate = _case(1101 if mode == "idw" else 1102, B, S, H, n, dqk, dv, x_std)
    compare_sequence(mem, st, x, w_in, w_gate, b_gate, 1.0, f"seq-{mode}")


@pytest.mark.parametrize("S", [1, 2, 64, 65, 129])
def test_sequence_lengths_around_the_chunk(S):
    """One token (reads only), exactly one chunk, one token over, and two
    chunks plus one; no gate bias."""
    need_gpu()
    B, H, n, dqk, dv, k, C = 2, 1, 32, 32, 64, 4, 64
    mem = _mem(sqrt_slots=n, dim_qk=dqk, dim_v=dv, topk=k, chunk_size=C, num_heads=H, max_batch=B)
    st, x, w_in, w_gate, _ = _case(1110 + S, B, S, H, n, dqk, dv)
    out, nxt = compare_sequence(mem, st, x, w_in, w_gate, None, 0.8, f"seq-S{S}")
    if S == 1:
        for name in ("k1", "k2", "v"):
            assert np.array_equal(nxt[name], st[name])


def test_closed_gate_returns_the_tokens():
    """b_gate = -1e4: g is 0 in fp32, so the output is the tokens bit for bit
    while the memory still takes its steps."""
    need_gpu()
    B, S, H, n, dqk, dv, k, C = 2, 100, 2, 32, 16, 8, 4, 32
    mem = _mem(sqrt_slots=n, dim_qk=dqk, dim_v=dv, topk=k, chunk_size=C, num_heads=H, max_batch=B)
    st, x, w_in, w_gate, _ = _case(1120, B, S, H, n, dqk, dv)
    b_gate = np.full(H, -1e4, np.float32)
    out, nxt = compare_sequence(mem, st, x, w_in, w_gate, b_gate, 1.0, "seq-closed-gate")
    assert np.array_equal(out, x)
    assert not np.array_equal(nxt["v"], st["v"])


def test_sequence_at_the_chained_workload_shape():
    """8 sequences x 4096 tokens, D = d_qk = d_v = 512, n = 256, top-8,
    chunks of 256 (the benchmark's sequence shape, clustered tokens): the
    GPU runs all 8 memories; the oracle follows sequence 0's whole chain."""
    need_gpu()
    from workloads import draw_tokens, get_config, initial_tables, layer_weights
    cfg = get_config(3)
    B, S, C = cfg.batch, cfg.tokens_per_pass, cfg.chunk
    mem = _mem(sqrt_slots=cfg.sqrt_slots, dim_qk=cfg.dim_qk, dim_v=cfg.dim_v, topk=cfg.topk,
               chunk_size=C, num_heads=1, max_batch=B, eps=cfg.eps)
    tab = initial_tables(cfg)
    x = draw_tokens(cfg)
    lw = layer_weights(cfg)
    st = {name: np.repeat(getattr(tab, name), B, axis=0) for name in ("k1", "k2", "v")}
    out, nxt, slots = run_gpu(mem, st, x, lw.w_in, lw.w_gate, lw.b_gate, cfg.lr)
    st0 = {name: a[:1] for name, a in st.items()}
    say("chained shape: oracle on sequence 0")
    o_out, o_nxt, ties = oracle_with_ties(mem.cfg, st0, x[:1], lw.w_in, lw.w_gate, lw.b_gate,
                                          cfg.lr, slots[:1])
    say("near-ties adopted:", ties)
    assert_close("chained out", out[:1], o_out, RTOL_CHAIN, ATOL_CHAIN)
    for name in ("k1", "k2", "v"):
        assert_close(f"chained next {name}", nxt[name][:1], o_nxt[name], RTOL_CHAIN, ATOL_CHAIN)
    # the other sequences took their own steps
    assert not np.array_equal(nxt["v"][1], st["v"][1])


def test_sequence_with_four_heads():
    """Four heads of d_qk 64 / d_v 32 (D = 128, 384 projection rows over
    three column tiles), chunks of 48, 2 x 200 tokens."""
    need_gpu()
    B, S, H, n, dqk, dv, k, C = 2, 200, 4, 64, 64, 32, 8, 48
    mem = _mem(sqrt_slots=n, dim_qk=dqk, dim_v=dv, topk=k, chunk_size=C, num_heads=H, max_batch=B)
    st, x, w_in, w_gate, b_gate = _case(1130, B, S, H, n, dqk, dv)
    compare_sequence(mem, st, x, w_in, w_gate, b_gate, 1.0, "seq-4heads")
