"""Seeded random draws for the FwPKM workloads (no method arithmetic here).

Every array comes from numpy's PCG64 generator seeded with
``1000 * config.index + stream``; streams are

    0 = K1 sub-keys, 1 = K2 sub-keys, 2 = V, 3 = queries, 4 = targets,
    5 = cluster centres, 6 = cluster assignment then cluster noise,
    7 = sequence-layer tokens (centres, then assignment and noise),
    8 = sequence-layer projection rows, 9 = gate weights then gate biases.

Values are drawn in float64 in C order, scaled in float64 and cast to fp32
once.  Large arrays are drawn block by block from one generator, which
yields the same numbers as a single draw.

Layouts:
  * initial tables: one set per head, shared by every sequence of the batch
    (k1, k2: [H, n, d_qk/2]; v: [H, n*n, d_v]);
  * queries [B, T, H, d_qk], targets [B, T, H, d_v], T = tokens per pass;
  * sequence layer: tokens [B, T, D] with D = H * d_v, projection rows
    [H*d_qk + H*d_v, D], gate weights [H, D] and biases [H].
Targets stand in for the lookahead value vectors (each query paired with
the next token's value); the caller would shift them, so here they are
simply independent N(0, 1) draws aligned with the queries.
"""

from __future__ import annotations

import dataclasses

import numpy as np

from .configs import WorkloadConfig

STREAM_K1 = 0
STREAM_K2 = 1
STREAM_V = 2
STREAM_Q = 3
STREAM_Y = 4
STREAM_CENTRES = 5
STREAM_ASSIGN = 6
STREAM_TOKENS = 7
STREAM_W_IN = 8
STREAM_GATE = 9

_BLOCK = 1 << 22  # elements per block when drawing large arrays


def make_rng(cfg: WorkloadConfig, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * cfg.index + stream))


def draw_normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) in float64, C order, block by block, cast to fp32."""
    shape = tuple(int(s) for s in shape)
    total = int(np.prod(shape, dtype=np.int64))
    out = np.empty(total, dtype=np.float32)
    pos = 0
    while pos < total:
        m = min(_BLOCK, total - pos)
        block = rng.standard_normal(m)  # float64
        if std != 1.0:
            block *= std
        out[pos:pos + m] = block
        pos += m
    return out.reshape(shape)


@dataclasses.dataclass
class InitialTables:
    k1: np.ndarray  # [H, n, d_h] fp32
    k2: np.ndarray  # [H, n, d_h] fp32
    v: np.ndarray   # [H, N, d_v] fp32


def initial_tables(cfg: WorkloadConfig) -> InitialTables:
    n, dh, N, dv, H = cfg.sqrt_slots, cfg.half, cfg.num_slots, cfg.dim_v, cfg.heads
    k1 = draw_normal(make_rng(cfg, STREAM_K1), (H, n, dh), cfg.key_std)
    k2 = draw_normal(make_rng(cfg, STREAM_K2), (H, n, dh), cfg.key_std)
    v = draw_normal(make_rng(cfg, STREAM_V), (H, N, dv), cfg.value_std)
    return InitialTables(k1=k1, k2=k2, v=v)


def draw_queries(cfg: WorkloadConfig) -> np.ndarray:
    """Queries for one pass, [B, T, H, d_qk] fp32."""
    B, T, H, d = cfg.batch, cfg.tokens_per_pass, cfg.heads, cfg.dim_qk
    if cfg.query_kind == "normal":
        return draw_normal(make_rng(cfg, STREAM_Q), (B, T, H, d))
    if cfg.query_kind != "clustered":
        raise ValueError(cfg.query_kind)
    # unit-norm centres; per-coordinate noise sigma/sqrt(d), so the noise
    # vector has norm close to sigma
    crng = make_rng(cfg, STREAM_CENTRES)
    centres = crng.standard_normal((cfg.clusters, d))
    centres /= np.linalg.norm(centres, axis=1, keepdims=True)
    arng = make_rng(cfg, STREAM_ASSIGN)
    assign = arng.integers(0, cfg.clusters, size=(B, T, H))
    out = np.empty((B, T, H, d), dtype=np.float32)
    flat_assign = assign.reshape(-1)
    flat_out = out.reshape(-1, d)
    noise_std = cfg.cluster_sigma / np.sqrt(d)
    rows_per_block = max(1, _BLOCK // d)
    for r0 in range(0, flat_out.shape[0], rows_per_block):
        r1 = min(flat_out.shape[0], r0 + rows_per_block)
        noise = arng.standard_normal((r1 - r0, d)) * noise_std
        flat_out[r0:r1] = centres[flat_assign[r0:r1]] + noise
    return out


def draw_targets(cfg: WorkloadConfig) -> np.ndarray:
    """Targets for one pass, [B, T, H, d_v] fp32, N(0, 1)."""
    B, T, H, d = cfg.batch, cfg.tokens_per_pass, cfg.heads, cfg.dim_v
    return draw_normal(make_rng(cfg, STREAM_Y), (B, T, H, d))


@dataclasses.dataclass
class ChunkInputs:
    queries: np.ndarray  # [B, C, H, d_qk] fp32, C-contiguous
    targets: np.ndarray  # [B, C, H, d_v] fp32, C-contiguous


def chunk_inputs(queries: np.ndarray, targets: np.ndarray, cfg: WorkloadConfig,
                 c: int) -> ChunkInputs:
    """The c-th chunk (0-based, within one pass) of a pass's inputs."""
    t0, t1 = c * cfg.chunk, (c + 1) * cfg.chunk
    return ChunkInputs(
        queries=np.ascontiguousarray(queries[:, t0:t1]),
        targets=np.ascontiguousarray(targets[:, t0:t1]),
    )


def expand_tables(tables: InitialTables, batch: int) -> InitialTables:
    """Per-sequence copies of the shared initial tables, [B*H, ...]."""
    def rep(a):
        return np.repeat(a[None], batch, axis=0).reshape((-1,) + a.shape[1:])
    return InitialTables(k1=rep(tables.k1), k2=rep(tables.k2), v=rep(tables.v))


def draw_tokens(cfg: WorkloadConfig) -> np.ndarray:
    """Model-width tokens for the sequence layer, [B, T, D] fp32, D = H*d_v.

    Clustered workloads: unit-norm centres in D dimensions, per-coordinate
    noise sigma/sqrt(D) (the query recipe, one level up); otherwise N(0, 1/D)
    per coordinate (unit expected norm)."""
    B, T, D = cfg.batch, cfg.tokens_per_pass, cfg.heads * cfg.dim_v
    rng = make_rng(cfg, STREAM_TOKENS)
    if cfg.query_kind != "clustered":
        return draw_normal(rng, (B, T, D), 1.0 / np.sqrt(D))
    centres = rng.standard_normal((cfg.clusters, D))
    centres /= np.linalg.norm(centres, axis=1, keepdims=True)
    assign = rng.integers(0, cfg.clusters, size=B * T)
    out = np.empty((B * T, D), dtype=np.float32)
    noise_std = cfg.cluster_sigma / np.sqrt(D)
    rows_per_block = max(1, _BLOCK // D)
    for r0 in range(0, B * T, rows_per_block):
        r1 = min(B * T, r0 + rows_per_block)
        out[r0:r1] = centres[assign[r0:r1]] + rng.standard_normal((r1 - r0, D)) * noise_std
    return out.reshape(B, T, D)


@dataclasses.dataclass
class LayerWeights:
    w_in: np.ndarray    # [H*d_qk + H*d_v, D] fp32, N(0, 1/D)
    w_gate: np.ndarray  # [H, D] fp32, N(0, 1/D)
    b_gate: np.ndarray  # [H] fp32, N(0, 1)


def layer_weights(cfg: WorkloadConfig) -> LayerWeights:
    """Stand-in (random, untrained) weights of the sequence layer."""
    H, D = cfg.heads, cfg.heads * cfg.dim_v
    w_in = draw_normal(make_rng(cfg, STREAM_W_IN), (H * (cfg.dim_qk + cfg.dim_v), D), 1.0 / np.sqrt(D))
    grng = make_rng(cfg, STREAM_GATE)
    w_gate = draw_normal(grng, (H, D), 1.0 / np.sqrt(D))
    b_gate = draw_normal(grng, (H,))
    return LayerWeights(w_in=w_in, w_gate=w_gate, b_gate=b_gate)
