"""The seeded input generators: determinism, shapes and block drawing."""

import numpy as np

from workloads import CONFIGS, draw_normal, draw_queries, draw_targets, get_config, initial_tables
from workloads import generate as G


def test_block_draw_equals_single_draw(monkeypatch):
    rng_a = np.random.Generator(np.random.PCG64(5))
    one = (rng_a.standard_normal(1000) * 0.5).astype(np.float32)
    monkeypatch.setattr(G, "_BLOCK", 37)
    rng_b = np.random.Generator(np.random.PCG64(5))
    blocks = draw_normal(rng_b, (10, 100), 0.5)
    assert blocks.reshape(-1).tobytes() == one.tobytes()


def test_tiny_workload_is_deterministic_and_shaped():
    cfg = get_config(1)
    t1, t2 = initial_tables(cfg), initial_tables(cfg)
    assert t1.v.tobytes() == t2.v.tobytes()
    assert t1.k1.shape == (1, 32, 32) and t1.v.shape == (1, 1024, 64)
    q, y = draw_queries(cfg), draw_targets(cfg)
    assert q.shape == (1, 256, 1, 64) and y.shape == (1, 256, 1, 64)
    assert q.dtype == np.float32 and y.dtype == np.float32
    assert q.tobytes() == draw_queries(cfg).tobytes()
    # distinct streams
    assert not np.array_equal(t1.k1, t1.k2)


def test_scales_match_the_configs():
    cfg = get_config(1)
    t = initial_tables(cfg)
    assert abs(t.k1.std() - np.sqrt(1 / 32)) < 0.01
    assert abs(t.v.std() - np.sqrt(0.02)) < 0.005


def test_clustered_queries_sit_near_unit_centres():
    cfg = get_config(3)
    q = draw_queries(cfg)
    norms = np.linalg.norm(q.reshape(-1, cfg.dim_qk)[:4096], axis=1)
    assert abs(norms.mean() - np.sqrt(1 + 0.3 ** 2)) < 0.02


def test_config_table():
    assert [c.num_slots for c in CONFIGS.values()] == [1024, 65536, 65536, 262144, 1048576]
    assert [c.units for c in CONFIGS.values()] == [1, 2, 8, 16, 1]
    assert get_config(3).tokens_per_pass == 4096
    assert get_config(5).passes == 2
