"""GPU parity of the dense comparator (oasis_dense_attn): attention over every
valid token of the full KV, against the oracle's attention with every block of
the context resident (which the oracle pins equal to textbook dense softmax
attention)."""
import numpy as np
import pytest
import torch

import oracle
from parity import check_attention
from sparse_kv_block_amd import gen
from sparse_kv_block_amd.configs import Config

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from sparse_kv_block_amd import lib  # noqa: E402

CASES = [
    dict(head_dim=128, n_q_heads=8, n_kv_heads=2, ctx=[5000, 1, 0, 2048]),
    dict(head_dim=64, n_q_heads=4, n_kv_heads=4, ctx=[3000, 129 * 16]),
    dict(head_dim=128, n_q_heads=32, n_kv_heads=2, ctx=[4100, 700]),          # 32 rows
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"d{c['head_dim']}-g{c['n_q_heads'] // c['n_kv_heads']}")
def test_dense_attention_matches_oracle(case):
    ctx = np.array(case["ctx"], np.int32)
    cfg = Config(name="dense", dtype="bf16", batch=len(ctx), n_q_heads=case["n_q_heads"],
                 n_kv_heads=case["n_kv_heads"], head_dim=case["head_dim"], block_size=16,
                 ctx=None, k_resident=8, cap=0.05, draft_sigma=0.2, rho=0.95, seed=41)
    nb = max(1, cfg.max_blocks(int(ctx.max())))
    qs = gen.query_sequence(cfg, 2, device="cuda")
    q = gen.step_queries(cfg, qs, 1)
    rec = gen.records(cfg, ctx, nb, device="cuda")
    shape = lib.Shape.of(cfg, nb)
    out = torch.full_like(q, 3.0)
    ws = lib.dense_attn_workspace(shape)
    lib.dense_attn(shape, q, rec, torch.from_numpy(ctx).cuda(), out, ws)
    torch.cuda.synchronize()
    # every block of the context resident, in block order
    p2l = np.tile(np.arange(nb, dtype=np.int32), (cfg.batch, cfg.n_kv_heads, 1))
    ref = oracle.attention(q.cpu(), rec.cpu(), p2l, ctx, 16)
    check_attention(out, ref, "bf16", "dense")
