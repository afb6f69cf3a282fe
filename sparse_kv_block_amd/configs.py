"""The five workload shapes of the look-ahead sparse decode step.

Each entry fixes the tensor shapes and the distributions the seeded generator
(`gen.py`) draws from.  Sizes follow the OasisKV pages: B=16-token blocks and
K=128 resident blocks per KV head (the 2,048-token budget) and the 0.05
per-step fetch cap (pith.science paper page, "Assumptions & free parameters"),
and the Qwen3-8B 16K / concurrency-128 setting of the headline table
(agihunt.info summary, throughput table).
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class Config:
    name: str
    dtype: str                 # "f32" or "bf16": storage type of q, K, V, summaries, out
    batch: int                 # B requests
    n_q_heads: int             # Hq
    n_kv_heads: int            # Hkv
    head_dim: int              # d
    block_size: int            # S tokens per block
    ctx: Optional[int]         # fixed context length per request, or None (lognormal)
    k_resident: int            # K resident blocks per (request, KV head)
    cap: float                 # per-step fetch ratio cap (admissions: oasis_cap_to_max_admit)
    draft_sigma: float         # draft = next-step query + N(0, draft_sigma)
    rho: float                 # AR(1) coefficient of the query drift between steps
    planted: int = 0           # high-affinity blocks per (request, KV head)
    planted_shift: float = 2.0  # in units of the key standard deviation
    steps: int = 1             # consecutive decode steps with carried state
    layers: int = 1
    ctx_lognormal: Optional[Tuple[float, float, int, int]] = None  # (mean, sigma_ln, lo, hi)
    caps_sweep: Tuple[float, ...] = ()
    seed: int = 0

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def rows(self) -> int:
        """Query rows per KV head: the normal and the draft row of each query head."""
        return 2 * self.group

    @property
    def esize(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def record_elems(self) -> int:
        """Elements of one block record: keys [S][d] then transposed values [d][S]."""
        return 2 * self.block_size * self.head_dim

    def max_blocks(self, ctx_max: Optional[int] = None) -> int:
        lmax = ctx_max if ctx_max is not None else (
            self.ctx if self.ctx is not None else self.ctx_lognormal[3])
        return -(-lmax // self.block_size)

    def scaled(self, **kw) -> "Config":
        return replace(self, **kw)


# 1. Tiny single layer, fp32.
TINY = Config(
    name="tiny_f32", dtype="f32", batch=1, n_q_heads=4, n_kv_heads=2, head_dim=64,
    block_size=16, ctx=1024, k_resident=8, cap=0.25, draft_sigma=0.1, rho=1.0,
    seed=1)

# 2. Qwen3-8B-shaped layer at 16K context, batch 128 (the throughput workload).
QWEN3_8B_16K = Config(
    name="qwen3_8b_16k", dtype="bf16", batch=128, n_q_heads=32, n_kv_heads=8,
    head_dim=128, block_size=16, ctx=16384, k_resident=128, cap=0.05,
    draft_sigma=0.2, rho=0.95, planted=8, seed=2)

# 3. Long-context agentic shape: lognormal contexts, 32 carried steps.
AGENTIC = Config(
    name="agentic_long", dtype="bf16", batch=64, n_q_heads=32, n_kv_heads=8,
    head_dim=128, block_size=16, ctx=None, k_resident=128, cap=0.05,
    draft_sigma=0.2, rho=0.95, steps=32,
    ctx_lognormal=(32700.0, 0.75, 8192, 131072), seed=3)

# 4. Full 36-layer decode step with a fetch-cap sweep.
FULL_36 = Config(
    name="full_36_layer", dtype="bf16", batch=128, n_q_heads=32, n_kv_heads=8,
    head_dim=128, block_size=16, ctx=16384, k_resident=128, cap=0.05,
    draft_sigma=0.2, rho=0.95, planted=8, layers=36,
    caps_sweep=(0.01, 0.05, 0.2, 1.0), seed=4)

# 5. High-GQA (16 query heads per KV head) MoE-attention-shaped layer.
GQA16 = Config(
    name="gqa16_moe", dtype="bf16", batch=256, n_q_heads=64, n_kv_heads=4,
    head_dim=128, block_size=16, ctx=16384, k_resident=128, cap=0.05,
    draft_sigma=0.2, rho=0.95, planted=8, seed=5)

CONFIGS = {c.name: c for c in (TINY, QWEN3_8B_16K, AGENTIC, FULL_36, GQA16)}
BY_INDEX = {1: TINY, 2: QWEN3_8B_16K, 3: AGENTIC, 4: FULL_36, 5: GQA16}
