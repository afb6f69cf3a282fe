"""Full-size parity of the workloads, whole batch, every unit, every step.

Each workload runs at its full size in the launch configuration the bench
times (the fused layer step, then the gather prefetch of its admissions), from
a cold fill over several decode steps with the resident sets carried, and an
oracle twin (`parity.OracleTwin`) steps the same inputs beside it:
  - summaries of every block of every unit, by value;
  - attention of every row of every query head (1e-2 bf16, 1e-5 fp32);
  - the top-K list of every unit, within 1e-5 relative at the K-th score;
  - block maps, stamps and admissions of every unit, bit for bit, at every
    step (the oracle evicts with the GPU's validated list, so that a list
    that differs inside the tolerance does not end the comparison);
  - the prefetch, through the next step's attention (the oracle reads the
    logical records, the GPU the slots the prefetch filled), and after the
    last step by comparing every resident slot with its block.
The count of lists that differ inside the tolerance is reported and bounded
by the count of unit-steps whose oracle scores hold a near-tie."""
import sys

import numpy as np
import pytest
import torch

import oracle
from parity import OracleTwin, host
from sparse_kv_block_amd import gen
from sparse_kv_block_amd.configs import AGENTIC, GQA16, QWEN3_8B_16K, TINY

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from sparse_kv_block_amd import lib            # noqa: E402  (fails loudly if not built)
from sparse_kv_block_amd.pipeline import Layer  # noqa: E402

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_resident_copies(layer, rec_cpu: np.ndarray, what=""):
    """Every occupied slot of every unit holds its block's record, bit for bit."""
    p2l = host(layer.p2l).astype(np.int64)
    pool = host(layer.pool)
    b, h, s = np.nonzero(p2l >= 0)
    assert np.array_equal(pool[b, h, s], rec_cpu[b, h, p2l[b, h, s]]), f"{what}: resident copies"


def carry(cfg, steps: int):
    ctx = gen.context_lengths(cfg)
    nbmax = cfg.max_blocks(int(ctx.max()))
    K = cfg.k_resident
    m = lib.cap_to_max_admit(cfg.cap, K)
    say(f"{cfg.name}: B={cfg.batch} Hq={cfg.n_q_heads} Hkv={cfg.n_kv_heads} NBmax={nbmax} "
        f"K={K} m={m} steps={steps} mean context {float(ctx.mean()):.0f}")
    qseq = gen.query_sequence(cfg, steps + 1, device=DEV)
    dirs = gen.planted_directions(cfg, qseq[1]) if cfg.planted else None
    rec = gen.records(cfg, ctx, nbmax, device=DEV, planted_dir=dirs)
    layer = Layer(cfg, ctx, nbmax)
    layer.summarize(rec)
    rec_cpu = rec.cpu()
    twin = OracleTwin(cfg, rec_cpu, ctx)
    torch.cuda.synchronize()
    twin.check_summaries(layer, cfg.name)
    say(f"{cfg.name}: summaries of all {cfg.batch * cfg.n_kv_heads} units match")
    q1 = gen.step_queries(cfg, qseq, 1)
    layer.cold_fill(q1, rec)
    torch.cuda.synchronize()
    twin.cold_fill(layer, q1.cpu(), cfg.name)
    evictions = 0
    for step in range(1, steps + 1):
        q = gen.step_queries(cfg, qseq, step)
        layer.step(q, step, m)
        layer.prefetch(rec, m)
        torch.cuda.synchronize()
        admit, count = twin.step(layer, q.cpu(), step, m, cfg.name)
        evictions += int((admit[..., 2] >= 0).sum())
        say(f"{cfg.name}: step {step} matches on every unit ({int(count.sum())} admissions, "
            f"{len(twin.differ)} lists inside the tolerance so far)")
    check_resident_copies(layer, oracle.as_np(rec_cpu), cfg.name)
    say(f"{cfg.name}: {twin.report()}; {evictions} resident blocks evicted")
    assert len(twin.differ) <= twin.exposed
    return twin, evictions


def test_full_size_tiny_f32():
    carry(TINY, 6)


@pytest.mark.timeout(900)
def test_full_size_qwen3_8b_16k():
    carry(QWEN3_8B_16K, 3)


@pytest.mark.timeout(900)
def test_full_size_gqa16():
    carry(GQA16, 2)


@pytest.mark.timeout(1200)
def test_full_size_agentic_32_steps():
    twin, evictions = carry(AGENTIC, AGENTIC.steps)
    # the carried state exercises the least-recently-selected eviction
    assert evictions > 0
