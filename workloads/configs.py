"""The five synthetic workloads the FwPKM chunk step is checked and timed on.

Shapes follow the pages:
  * the PyPI page "fast-weight-product-key-memory 0.2.2", Usage: a memory of
    256*256 slots, query/key width 512, value width 512, top-8, learning rate
    1.0, chunks of 256 tokens, input of 2 x 256 tokens;
  * the gist.science summary of "Fast-weight Product Key Memory", section 4
    (Experimental Results): models trained on 4K-token sequences, needle
    tests at 128K tokens with repeated (iterative) reading;
  * the same summary, section 2 (Core Architecture): memories of about 10^6
    slots addressed with O(sqrt(N)) scoring;
  * the PyPI page's acknowledgement of a multi-head variant.

Initial-value scales: "N(0, s)" below names a variance s, so sub-keys drawn
N(0, 1/d_h) have unit expected squared norm and V has standard deviation
sqrt(0.02).
"""

from __future__ import annotations

import dataclasses
import math


@dataclasses.dataclass(frozen=True)
class WorkloadConfig:
    index: int            # 1..5, also the seed base (seed = 1000*index + stream)
    name: str             # what the workload is, with its sizes
    batch: int            # B sequences
    heads: int            # H independent memories per sequence
    chunk: int            # C tokens per chunk call
    chunks: int           # chunk calls per pass
    passes: int           # how many times the same token stream is fed
    sqrt_slots: int       # n; N = n*n slots
    dim_qk: int           # d_qk, split into two halves of d_qk/2
    dim_v: int            # d_v
    topk: int             # k
    lr: float = 1.0       # eta
    eps: float = 1e-3     # IDW epsilon (value not given on the pages)
    query_kind: str = "normal"   # "normal" or "clustered"
    clusters: int = 0     # number of cluster centres for clustered queries
    cluster_sigma: float = 0.3   # noise norm around unit-norm centres
    value_var: float = 0.02      # variance of the initial V entries

    @property
    def num_slots(self) -> int:
        return self.sqrt_slots * self.sqrt_slots

    @property
    def half(self) -> int:
        return self.dim_qk // 2

    @property
    def units(self) -> int:
        return self.batch * self.heads

    @property
    def tokens_per_pass(self) -> int:
        return self.chunk * self.chunks

    @property
    def key_var(self) -> float:
        return 1.0 / self.half

    @property
    def key_std(self) -> float:
        return math.sqrt(self.key_var)

    @property
    def value_std(self) -> float:
        return math.sqrt(self.value_var)

    def table_bytes(self) -> dict:
        """fp32 bytes of one head's initial tables (shared by the batch)."""
        return {
            "k1": self.sqrt_slots * self.half * 4,
            "k2": self.sqrt_slots * self.half * 4,
            "v": self.num_slots * self.dim_v * 4,
        }


CONFIGS = {
    1: WorkloadConfig(
        index=1, name="tiny-1x256-n32-d64-k4",
        batch=1, heads=1, chunk=64, chunks=4, passes=1,
        sqrt_slots=32, dim_qk=64, dim_v=64, topk=4),
    2: WorkloadConfig(
        index=2, name="libdefault-2x256-n256-d512-k8",
        batch=2, heads=1, chunk=256, chunks=1, passes=1,
        sqrt_slots=256, dim_qk=512, dim_v=512, topk=8),
    3: WorkloadConfig(
        index=3, name="chained-8x4096-n256-d512-k8-clustered",
        batch=8, heads=1, chunk=256, chunks=16, passes=1,
        sqrt_slots=256, dim_qk=512, dim_v=512, topk=8,
        query_kind="clustered", clusters=64),
    4: WorkloadConfig(
        index=4, name="multihead-4x8192-h4-n512-d256-k16",
        batch=4, heads=4, chunk=512, chunks=16, passes=1,
        sqrt_slots=512, dim_qk=256, dim_v=256, topk=16),
    5: WorkloadConfig(
        index=5, name="longctx-1x131072-n1024-d512-k16-2pass",
        batch=1, heads=1, chunk=512, chunks=256, passes=2,
        sqrt_slots=1024, dim_qk=512, dim_v=512, topk=16,
        query_kind="clustered", clusters=4096),
}


def get_config(key) -> WorkloadConfig:
    """Look a workload up by index (1..5) or by name."""
    if isinstance(key, int):
        return CONFIGS[key]
    for cfg in CONFIGS.values():
        if cfg.name == key or str(cfg.index) == str(key):
            return cfg
    raise KeyError(f"unknown workload {key!r}")
