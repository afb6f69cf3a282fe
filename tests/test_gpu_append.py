"""GPU parity of the decode append against the CPU oracle.

Records, resident copies and context lengths must match bit for bit (the call
only places bytes); summaries by value (the min/max of the same values).
After the appends the incrementally kept summaries must also equal a fresh
GPU summarize of the appended records.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from parity import host, i32, pool_from_records
from sparse_kv_block_amd import gen
from sparse_kv_block_amd.configs import QWEN3_8B_16K, Config

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from sparse_kv_block_amd import lib            # noqa: E402  (fails loudly if not built)

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def small(**kw) -> Config:
    base = dict(name="append", dtype="bf16", batch=5, n_q_heads=8, n_kv_heads=2, head_dim=128,
                block_size=16, ctx=1000, k_resident=16, cap=0.25, draft_sigma=0.1, rho=0.9,
                seed=303)
    base.update(kw)
    return Config(**base)


def make_tail_resident(l2p, p2l, ctx, units, S=16):
    """Put the block that receives each listed unit's next token into slot 0."""
    for (b, h) in units:
        j = int(ctx[b]) // S
        if j >= l2p.shape[2]:
            continue
        old = int(p2l[b, h, 0])
        if old >= 0:
            l2p[b, h, old] = -1
        if int(l2p[b, h, j]) >= 0:
            p2l[b, h, int(l2p[b, h, j])] = -1
        p2l[b, h, 0] = j
        l2p[b, h, j] = 0


CASES = [
    dict(dtype="bf16", head_dim=128),
    dict(dtype="bf16", head_dim=64, n_q_heads=4, n_kv_heads=4),
    dict(dtype="f32", head_dim=64, n_q_heads=4, n_kv_heads=2),
    dict(dtype="f32", head_dim=128, n_q_heads=2, n_kv_heads=1, batch=3),
]


def case_id(c):
    return "-".join(f"{k}{v}" for k, v in c.items())


@pytest.mark.parametrize("where", ["device", "pinned"])
@pytest.mark.parametrize("with_pool", [True, False])
@pytest.mark.parametrize("case", CASES, ids=case_id)
def test_append_matches_oracle(case, where, with_pool):
    cfg = small(**case)
    nbmax = 64                                   # capacity 1024 tokens
    B = cfg.batch
    # mid-block, one past a block edge, empty, three short of capacity, block edge
    ctx0 = np.array([1000, 17, 0, 1021, 32][:B], np.int32)
    steps = 20
    say(f"append {case_id(case)} {where} pool={with_pool}")
    rec = gen.records(cfg, ctx0, nbmax, seed=5)
    kn, vn = gen.new_tokens(cfg, steps, seed=9, integer=(cfg.dtype == "bf16"))
    l2p, p2l, _ = gen.random_state(cfg, ctx0, nbmax, seed=4, fill=0.7)
    picks = [(0, 0), (1, cfg.n_kv_heads - 1), (3, 0), (4, 0)]
    make_tail_resident(l2p, p2l, ctx0, [u for u in picks if u[0] < B])
    pool = pool_from_records(rec, p2l)
    shape = lib.Shape.of(cfg, nbmax)

    # oracle side
    r_o, p_o, l_o = oracle.as_np(rec).copy(), oracle.as_np(pool).copy(), l2p.numpy().copy()
    s_o = oracle.summarize(r_o, ctx0, 16)
    c_o = ctx0.copy()
    for i in range(steps):
        oracle.append(kn[i], vn[i], r_o, s_o, c_o, 16, pool=p_o if with_pool else None,
                      l2p=l_o if with_pool else None)

    # GPU side
    if where == "device":
        r_g = rec.to(DEV)
    else:
        r_g = torch.empty_like(rec).pin_memory()
        r_g.copy_(rec)
    p_g = pool.to(DEV)
    l_g = l2p.to(DEV)
    ctx_g = torch.from_numpy(ctx0).to(DEV)
    s_g = torch.zeros((B, cfg.n_kv_heads, nbmax, 2, cfg.head_dim), dtype=rec.dtype, device=DEV)
    lib.summarize(shape, r_g, ctx_g, s_g)
    kd, vd = kn.to(DEV), vn.to(DEV)
    for i in range(steps):
        lib.append_token(shape, kd[i], vd[i], r_g, s_g, ctx_g,
                         pool=p_g if with_pool else None, l2p=l_g if with_pool else None)
    torch.cuda.synchronize()

    assert i32(ctx_g).tolist() == c_o.tolist()
    assert c_o.tolist() == [1020, 37, 20, 1024, 52][:B]
    np.testing.assert_array_equal(oracle.as_np(r_g.cpu()), r_o)
    if with_pool:
        np.testing.assert_array_equal(oracle.as_np(p_g.cpu()), p_o)
    else:
        np.testing.assert_array_equal(oracle.as_np(p_g.cpu()), oracle.as_np(pool))
    np.testing.assert_array_equal(oracle.to_f64(host(s_g)), oracle.to_f64(s_o))
    # incremental summaries == a fresh summarize of the appended records
    s_fresh = torch.zeros_like(s_g)
    lib.summarize(shape, r_g, ctx_g, s_fresh)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(oracle.to_f64(host(s_g)), oracle.to_f64(host(s_fresh)))


def test_append_full_size_qwen3_8b_16k():
    """One append at the 128-request, 8-KV-head, 16K-context shape, every unit
    against the oracle: the touched block record of every unit, the whole
    resident pool (the tail block made resident in every other unit) and every
    summary, and every request's context length."""
    cfg = QWEN3_8B_16K
    ctx = gen.context_lengths(cfg)
    nbmax = cfg.max_blocks(int(ctx.max())) + 1
    say(f"append full size: B={cfg.batch} NBmax={nbmax}")
    rec = gen.records(cfg, ctx, nbmax, device=DEV)
    l2p, p2l, _ = gen.random_state(cfg, ctx, nbmax, seed=6)
    every_other = [(b, h) for b in range(cfg.batch) for h in range(cfg.n_kv_heads) if (b + h) % 2 == 0]
    make_tail_resident(l2p, p2l, ctx, every_other)
    l2p, p2l = l2p.to(DEV), p2l.to(DEV)
    pool = pool_from_records(rec, p2l)
    shape = lib.Shape.of(cfg, nbmax)
    ctx_g = torch.from_numpy(ctx).to(DEV)
    summ = torch.zeros((cfg.batch, cfg.n_kv_heads, nbmax, 2, cfg.head_dim), dtype=rec.dtype,
                       device=DEV)
    lib.summarize(shape, rec, ctx_g, summ)
    kn, vn = gen.new_tokens(cfg, 1, seed=12, device=DEV)
    torch.cuda.synchronize()
    r_o, p_o, s_o = (oracle.as_np(x.cpu()).copy() for x in (rec, pool, summ))
    c_o = ctx.copy()
    lib.append_token(shape, kn[0], vn[0], rec, summ, ctx_g, pool=pool, l2p=l2p)
    torch.cuda.synchronize()
    oracle.append(kn[0].cpu(), vn[0].cpu(), r_o, s_o, c_o, 16, pool=p_o, l2p=i32(l2p))
    np.testing.assert_array_equal(i32(ctx_g), c_o)
    assert c_o.tolist() == (ctx + 1).tolist()
    j = torch.from_numpy(ctx.astype(np.int64) // 16).to(DEV)
    touched = rec[torch.arange(cfg.batch, device=DEV), :, j]          # [B][Hkv][record]
    np.testing.assert_array_equal(host(touched), r_o[np.arange(cfg.batch), :, ctx // 16])
    np.testing.assert_array_equal(host(pool), p_o)
    np.testing.assert_array_equal(oracle.to_f64(host(summ)), oracle.to_f64(s_o))
