"""GPU parity of the top-K agreement diagnostic against the CPU oracle:
exact block scores + top-K (tolerance at the K-th score as for the summary
scan; bit-exact order on small-integer inputs, where every logit is exact in
fp32) and the agreement counts (bit-exact)."""
import sys

import numpy as np
import pytest
import torch

import oracle
from parity import check_topk, host, i32
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
    base = dict(name="diag", dtype="bf16", batch=3, n_q_heads=8, n_kv_heads=2, head_dim=128,
                block_size=16, ctx=1000, k_resident=16, cap=0.25, draft_sigma=0.2, rho=0.95,
                seed=404)
    base.update(kw)
    return Config(**base)


CASES = [
    dict(dtype="bf16", head_dim=128),
    dict(dtype="bf16", head_dim=64, n_q_heads=4, n_kv_heads=4),
    dict(dtype="bf16", head_dim=128, n_q_heads=32, n_kv_heads=2, k_resident=24),     # G = 16
    dict(dtype="bf16", head_dim=128, n_q_heads=2, n_kv_heads=2, k_resident=8),       # G = 1
    dict(dtype="f32", head_dim=64, n_q_heads=4, n_kv_heads=2, k_resident=8),
    dict(dtype="f32", head_dim=128, n_q_heads=6, n_kv_heads=2, k_resident=40),
]
RAGGED = [1000, 17, 0]


def case_id(c):
    return "-".join(f"{k}{v}" for k, v in c.items())


def inputs(cfg, ctx, seed, integer):
    ctx = np.asarray(ctx, np.int32)
    nbmax = cfg.max_blocks(int(ctx.max()))
    if integer:
        rec, q = gen.integer_inputs(cfg, ctx, nbmax, seed, device=DEV)
    else:
        qs = gen.query_sequence(cfg, 2, seed=cfg.seed + seed, device=DEV)
        q = gen.step_queries(cfg, qs, 1, seed=cfg.seed + seed)
        rec = gen.records(cfg, ctx, nbmax, seed=cfg.seed + seed, device=DEV)
    return ctx, nbmax, rec, q


def run_exact(cfg, ctx, nbmax, rec, q, q_row):
    shape = lib.Shape.of(cfg, nbmax)
    U, K = cfg.batch * cfg.n_kv_heads, cfg.k_resident
    idx = torch.full((cfg.batch, cfg.n_kv_heads, K), 7, dtype=torch.int32, device=DEV)
    sc = torch.full((cfg.batch, cfg.n_kv_heads, K), 3.0, dtype=torch.float32, device=DEV)
    lib.exact_topk(shape, q, rec, torch.from_numpy(ctx).to(DEV), idx, sc, q_row=q_row)
    torch.cuda.synchronize()
    return i32(idx), host(sc)


@pytest.mark.parametrize("q_row", [0, 1])
@pytest.mark.parametrize("case", CASES, ids=case_id)
def test_exact_topk_gaussian(case, q_row):
    cfg = small(**case)
    say(f"exact_topk gaussian {case_id(case)} row {q_row}")
    ctx, nbmax, rec, q = inputs(cfg, RAGGED, seed=1, integer=False)
    idx, sc = run_exact(cfg, ctx, nbmax, rec, q, q_row)
    ex = oracle.exact_block_scores(q.cpu(), rec.cpu(), ctx, 16, q_row=q_row)
    ref, _ = oracle.topk(ex, ctx, 16, cfg.k_resident)
    check_topk(idx, sc, ref, ex, what=f"exact {cfg.name}")


@pytest.mark.parametrize("case", CASES, ids=case_id)
def test_exact_topk_bit_exact_on_integer_inputs(case):
    cfg = small(**case)
    say(f"exact_topk integer {case_id(case)}")
    ctx, nbmax, rec, q = inputs(cfg, RAGGED, seed=2, integer=True)
    idx, sc = run_exact(cfg, ctx, nbmax, rec, q, 1)
    ex = oracle.exact_block_scores(q.cpu(), rec.cpu(), ctx, 16, q_row=1)
    ref, val = oracle.topk(ex, ctx, 16, cfg.k_resident)
    np.testing.assert_array_equal(idx, ref)
    np.testing.assert_array_equal(sc.astype(np.float64), val)


def test_exact_topk_long_context_and_more_slots_than_blocks():
    cfg = small(batch=3, k_resident=200, n_q_heads=4, n_kv_heads=1)
    say("exact_topk long context")
    ctx, nbmax, rec, q = inputs(cfg, [131072, 100, 3200], seed=3, integer=False)
    idx, sc = run_exact(cfg, ctx, nbmax, rec, q, 1)
    ex = oracle.exact_block_scores(q.cpu(), rec.cpu(), ctx, 16, q_row=1)
    ref, _ = oracle.topk(ex, ctx, 16, cfg.k_resident)
    check_topk(idx, sc, ref, ex, what="exact long")


@pytest.mark.parametrize("exact_n", [None, 1, 7])
@pytest.mark.parametrize("with_map", [True, False])
def test_agreement_counts_bit_exact(with_map, exact_n):
    cfg = small(batch=4, n_kv_heads=3, n_q_heads=6, k_resident=32)
    nbmax = 300
    rng = np.random.default_rng(7)
    B, H, K = cfg.batch, cfg.n_kv_heads, cfg.k_resident
    pred = np.full((B, H, K), -1, np.int32)
    exact = np.full((B, H, K), -1, np.int32)
    l2p = np.full((B, H, nbmax), -1, np.int32)
    for b in range(B):
        for h in range(H):
            n = [K, 20, 0, 5][b]                           # full, partial, empty, short lists
            pool = rng.choice(nbmax, size=48, replace=False)   # both lists draw from it
            pred[b, h, :n] = rng.choice(pool, size=n, replace=False)
            exact[b, h, :n] = rng.choice(pool, size=n, replace=False)
            l2p[b, h, rng.choice(nbmax, size=K, replace=False)] = np.arange(K)
    shape = lib.Shape.of(cfg, nbmax)
    counts = torch.full((B, H, 3), 99, dtype=torch.int32, device=DEV)
    lib.topk_agreement(shape, torch.from_numpy(pred).to(DEV), torch.from_numpy(exact).to(DEV),
                       counts, l2p=torch.from_numpy(l2p).to(DEV) if with_map else None,
                       exact_n=exact_n)
    torch.cuda.synchronize()
    ref = oracle.agreement(pred, exact, l2p if with_map else None, exact_n=exact_n)
    np.testing.assert_array_equal(i32(counts), ref)


def test_exact_topk_full_size_qwen3_8b_16k():
    """Batch 128, 8 KV heads, 16K context: every unit's list on the GPU against
    the oracle's exact block scores of the whole batch."""
    cfg = QWEN3_8B_16K
    ctx = gen.context_lengths(cfg)
    nbmax = cfg.max_blocks(int(ctx.max()))
    say(f"exact_topk full size B={cfg.batch} NBmax={nbmax}")
    qs = gen.query_sequence(cfg, 2, device=DEV)
    q = gen.step_queries(cfg, qs, 1)
    dirs = gen.planted_directions(cfg, qs[1]) if cfg.planted else None
    rec = gen.records(cfg, ctx, nbmax, device=DEV, planted_dir=dirs)
    idx, sc = run_exact(cfg, ctx, nbmax, rec, q, 1)
    ex = oracle.exact_block_scores(q.cpu(), rec.cpu(), ctx, 16, q_row=1)
    ref, _ = oracle.topk(ex, ctx, 16, cfg.k_resident)
    differ = check_topk(idx, sc, ref, ex, what="exact top-K full size")
    say(f"exact top-K full size: {differ} of {cfg.batch * cfg.n_kv_heads} lists differ inside "
        f"the tolerance")


def test_agreement_study_matches_oracle_composition():
    """Eight look-ahead steps on small-integer inputs (every score exact in
    fp32, so every list must agree bit for bit): the study's per-unit counts
    against the same study composed from oracle calls."""
    from sparse_kv_block_amd.diagnostics import AgreementStudy
    from sparse_kv_block_amd.pipeline import Layer
    cfg = small(batch=3, k_resident=12, cap=0.25, n_q_heads=8, n_kv_heads=2)
    ctx = np.array([1000, 300, 17], np.int32)
    nbmax = cfg.max_blocks(1000)
    say("agreement study vs oracle")
    rec, _ = gen.integer_inputs(cfg, ctx, nbmax, seed=11, device=DEV)
    qs = gen.integer_queries(cfg, 10, seed=12, device=DEV)
    m = lib.cap_to_max_admit(cfg.cap, cfg.k_resident)
    layer = Layer(cfg, ctx, nbmax)
    layer.summarize(rec)
    layer.cold_fill(qs[0], rec)
    study = AgreementStudy(layer, top=5)

    rec_c = oracle.as_np(rec.cpu())
    summ_c = oracle.summarize(rec_c, ctx, 16)
    l2p, p2l, last = (x.cpu().numpy().copy() for x in layer.state())
    for s in range(1, 9):
        got = study.step(rec, qs[s], qs[s + 1], s, keep_units=True)
        q, qn = qs[s].cpu(), qs[s + 1].cpu()
        _, T, _, _, _ = oracle.layer_step(q, rec_c, summ_c, ctx, 16, cfg.k_resident, s, m,
                                          l2p, p2l, last)
        E, _ = oracle.topk(oracle.exact_block_scores(qn, rec_c, ctx, 16, 0), ctx, 16,
                           cfg.k_resident)
        lists = {
            "pred": (T, l2p),
            "bound": (oracle.topk(oracle.block_scores(qn, summ_c, ctx, 16, 0), ctx, 16,
                                  cfg.k_resident)[0], None),
            "drift": (oracle.topk(oracle.exact_block_scores(q, rec_c, ctx, 16, 1), ctx, 16,
                                  cfg.k_resident)[0], None),
            "previous": (oracle.topk(oracle.block_scores(q, summ_c, ctx, 16, 0), ctx, 16,
                                     cfg.k_resident)[0], None),
        }
        for name, (P, lp) in lists.items():
            np.testing.assert_array_equal(got[name], oracle.agreement(P, E, lp),
                                          err_msg=f"step {s} {name}")
            np.testing.assert_array_equal(got[name + "@top"], oracle.agreement(P, E, lp, 5),
                                          err_msg=f"step {s} {name} top 5")
        assert got["resident"] is got["pred"]
        np.testing.assert_array_equal(i32(layer.l2p), l2p)
