"""The fused step captured once into a HIP graph and replayed: every replay
must equal the same step run eagerly.  The split path's workgroups hand their
lists over through per-unit arrival words that carry a per-launch tag; a
replay reuses the captured tag, so each launch must leave the words at a zero
count for the next replay.  Replays are interleaved with eager work and
synchronisations, and every replay is checked."""
import sys

import numpy as np
import pytest
import torch

from parity import pool_from_records
from sparse_kv_block_amd import gen
from sparse_kv_block_amd.configs import Config

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from sparse_kv_block_amd import lib            # noqa: E402  (fails loudly if not built)
from sparse_kv_block_amd.pipeline import Layer  # noqa: E402

OUTPUTS = ("out", "topk_idx", "topk_score", "l2p", "p2l", "last_sel", "admit", "admit_count")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("entry", ["workspace", "noalloc"])
@pytest.mark.parametrize("ctx", [[40000, 16 * 1024 + 1, 900, 0], [16000, 300, 5000]],
                         ids=["split", "one-part"])
def test_graph_replays_equal_eager_steps(entry, ctx):
    cfg = Config(name="graph", dtype="bf16", batch=len(ctx), n_q_heads=8, n_kv_heads=2,
                 head_dim=128, block_size=16, ctx=None, k_resident=64, cap=0.25,
                 draft_sigma=0.2, rho=0.95, planted=0, seed=41)
    ctx = np.asarray(ctx, np.int32)
    nbmax = cfg.max_blocks(int(ctx.max()))
    say(f"graph case: {entry} NBmax={nbmax} ctx={ctx.tolist()}")
    qs = gen.query_sequence(cfg, 2, seed=41, device="cuda")
    q = gen.step_queries(cfg, qs, 1, seed=41)
    rec = gen.records(cfg, ctx, nbmax, seed=41, device="cuda")
    state = gen.random_state(cfg, ctx, nbmax, 41, fill=0.8, stamp_max=3)
    a, b = Layer(cfg, ctx, nbmax), Layer(cfg, ctx, nbmax)
    for L in (a, b):
        L.summarize(rec)
        L.set_state(*state)
        L.pool.copy_(pool_from_records(rec, L.p2l))
    m = lib.cap_to_max_admit(cfg.cap, cfg.k_resident)
    step = 4

    def run_b():
        if entry == "workspace":
            b.step(q, step, m)
        else:
            lib.layer_step_noalloc(b.shape, q, b.pool, b.summ, b.ctx_len, step, m, b.out,
                                   b.topk_idx, b.topk_score, b.l2p, b.p2l, b.last_sel,
                                   b.admit, b.admit_count)

    run_b()                       # eager first call (the no-alloc scratch lookup among it)
    torch.cuda.synchronize()
    a.set_state(*state)
    b.set_state(*state)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_b()
    filler = torch.arange(1 << 20, device="cuda", dtype=torch.float32)
    for r in range(5):
        a.step(q, step, m)
        g.replay()
        filler.mul_(1.0001).add_(r)   # eager work between the replays
        torch.cuda.synchronize()
        for name in OUTPUTS:
            assert torch.equal(getattr(a, name), getattr(b, name)), (entry, r, name)
    admitted = int(a.admit_count.sum())
    say(f"graph case: {entry} 5 replays equal; admissions in the last step {admitted}")
