"""GPU parity: every C-ABI call against the CPU oracle on seeded inputs.

Small shapes, element by element.  The five workloads at their full sizes,
carried over decode steps and compared unit by unit in full, are in
test_gpu_full_size.py and test_gpu_full36.py.

Tolerances: maps, admissions and summaries bit-exact (summaries by value);
top-K exact except swaps within 1e-5 relative of the K-th score (and exact on
small-integer inputs, where every score is exact in fp32); attention within
1e-2 (bf16) or 1e-5 (fp32) absolute + relative of the fp64 oracle.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from parity import check_attention, check_topk, host, i32, pool_from_records
from sparse_kv_block_amd import gen
from sparse_kv_block_amd.configs import Config

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from sparse_kv_block_amd import lib            # noqa: E402  (fails loudly if not built)
from sparse_kv_block_amd.pipeline import Layer  # noqa: E402

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def small(**kw) -> Config:
    base = dict(name="small", dtype="bf16", batch=3, n_q_heads=8, n_kv_heads=2, head_dim=128,
                block_size=16, ctx=1000, k_resident=16, cap=0.25, draft_sigma=0.2, rho=0.95,
                planted=4, seed=101)
    base.update(kw)
    return Config(**base)


def setup(cfg: Config, ctx=None, seed=0, integer=False, device=DEV, nbmax=None):
    ctx = gen.context_lengths(cfg) if ctx is None else np.asarray(ctx, np.int32)
    nbmax = nbmax or max(1, cfg.max_blocks(int(max(ctx.max(), 1))))
    if integer:
        rec, q = gen.integer_inputs(cfg, ctx, nbmax, seed, device=device)
    else:
        qs = gen.query_sequence(cfg, 2, seed=cfg.seed + seed, device=device)
        q = gen.step_queries(cfg, qs, 1, seed=cfg.seed + seed)
        dirs = gen.planted_directions(cfg, qs[1]) if cfg.planted else None
        rec = gen.records(cfg, ctx, nbmax, seed=cfg.seed + seed, device=device, planted_dir=dirs)
    return ctx, nbmax, rec, q


SMALL_CASES = [
    dict(dtype="f32", head_dim=64, n_q_heads=4, n_kv_heads=2, k_resident=8, batch=1, ctx=1024),
    dict(dtype="bf16", head_dim=128),
    dict(dtype="bf16", head_dim=64, n_q_heads=4, n_kv_heads=4),
    dict(dtype="bf16", head_dim=128, n_q_heads=32, n_kv_heads=2, k_resident=24),     # G = 16
    dict(dtype="f32", head_dim=128, n_q_heads=6, n_kv_heads=2, k_resident=40),
    # 24 stacked rows: the second 16-row tile is partly empty
    dict(dtype="bf16", head_dim=64, n_q_heads=24, n_kv_heads=2, k_resident=16),
    dict(dtype="bf16", head_dim=128, n_q_heads=12, n_kv_heads=1, k_resident=32, batch=2),
]
RAGGED = [1000, 17, 0]      # partial last block, one full block + 1 token, empty request


def case_id(c):
    return "-".join(f"{k}{v}" for k, v in c.items())


# --------------------------------------------------------------------------- summaries
@pytest.mark.parametrize("case", SMALL_CASES, ids=case_id)
def test_summarize(case):
    cfg = small(**case)
    ctx = RAGGED[:cfg.batch] if cfg.batch > 1 else [cfg.ctx]
    ctx, nbmax, rec, q = setup(cfg, ctx, seed=1)
    layer = Layer(cfg, ctx, nbmax)
    layer.summ.fill_(7)                       # sentinel for entries that must stay untouched
    init = host(layer.summ).copy()
    layer.summarize(rec)
    got = oracle.to_f64(host(layer.summ))
    ref = oracle.to_f64(oracle.summarize(rec.cpu(), ctx, 16, summ=init))
    np.testing.assert_array_equal(got, ref)


def test_summarize_from_pinned_host_records():
    cfg = small(batch=2)
    ctx, nbmax, rec, q = setup(cfg, [1000, 333], seed=2, device="cpu")
    pinned = rec.pin_memory()
    layer = Layer(cfg, ctx, nbmax)
    layer.summarize(pinned)
    torch.cuda.synchronize()
    ref = oracle.summarize(rec, ctx, 16)
    np.testing.assert_array_equal(oracle.to_f64(host(layer.summ)), oracle.to_f64(ref))


# --------------------------------------------------------------------------- scores + top-K
@pytest.mark.parametrize("case", SMALL_CASES, ids=case_id)
@pytest.mark.parametrize("q_row", [0, 1])
def test_score_topk_gaussian(case, q_row):
    cfg = small(**case)
    ctx = RAGGED[:cfg.batch] if cfg.batch > 1 else [cfg.ctx]
    ctx, nbmax, rec, q = setup(cfg, ctx, seed=3)
    layer = Layer(cfg, ctx, nbmax)
    layer.summarize(rec)
    lib.score_topk(layer.shape, q, layer.summ, layer.ctx_len, layer.topk_idx, layer.topk_score,
                   q_row=q_row, workspace=layer.workspace)
    summ = oracle.summarize(rec.cpu(), ctx, 16)
    sc = oracle.block_scores(q.cpu(), summ, ctx, 16, q_row=q_row)
    idx, _ = oracle.topk(sc, ctx, 16, cfg.k_resident)
    check_topk(i32(layer.topk_idx), host(layer.topk_score), idx, sc, what=cfg.name)


@pytest.mark.parametrize("case", SMALL_CASES, ids=case_id)
def test_score_topk_exact_on_integer_inputs(case):
    # scores of small integers are exact in fp32: ties abound and the order
    # (score desc, block asc) must agree bit for bit
    cfg = small(**case)
    ctx = RAGGED[:cfg.batch] if cfg.batch > 1 else [cfg.ctx]
    ctx, nbmax, rec, q = setup(cfg, ctx, seed=4, integer=True)
    layer = Layer(cfg, ctx, nbmax)
    layer.summarize(rec)
    lib.score_topk(layer.shape, q, layer.summ, layer.ctx_len, layer.topk_idx, layer.topk_score,
                   workspace=layer.workspace)
    summ = oracle.summarize(rec.cpu(), ctx, 16)
    sc = oracle.block_scores(q.cpu(), summ, ctx, 16)
    idx, val = oracle.topk(sc, ctx, 16, cfg.k_resident)
    np.testing.assert_array_equal(i32(layer.topk_idx), idx)
    np.testing.assert_array_equal(host(layer.topk_score).astype(np.float64), val)


def test_topk_with_more_slots_than_blocks_and_large_context():
    # K > NB_b for short requests; NBmax 8192 (a 128K context) for the long one
    cfg = small(batch=3, k_resident=200, n_q_heads=4, n_kv_heads=1)
    ctx, nbmax, rec, q = setup(cfg, [131072, 100, 3200], seed=5)
    layer = Layer(cfg, ctx, nbmax)
    layer.summarize(rec)
    lib.score_topk(layer.shape, q, layer.summ, layer.ctx_len, layer.topk_idx, layer.topk_score,
                   workspace=layer.workspace)
    summ = oracle.summarize(rec.cpu(), ctx, 16)
    sc = oracle.block_scores(q.cpu(), summ, ctx, 16)
    idx, _ = oracle.topk(sc, ctx, 16, cfg.k_resident)
    check_topk(i32(layer.topk_idx), host(layer.topk_score), idx, sc, what="large")


@pytest.mark.parametrize("dtype,K,d", [("bf16", 1, 128), ("bf16", 37, 64), ("bf16", 128, 128),
                                       ("bf16", 256, 128), ("f32", 128, 64)])
def test_score_topk_split_over_scan_parts_exact_on_integer_inputs(dtype, K, d):
    # contexts past 1024 blocks: one workgroup per 1024-block part; every
    # part but the last publishes its list, the last part hands over its keys
    # unselected (1-block last parts finish first and take that path; a
    # 1024-block last part, dispatched late, usually merges at once), and the
    # last to arrive merges (K = 256 over 8 parts: 2,816 entries); contexts on
    # and around the part boundaries, one that fits a single part (finished by
    # its part workgroup) and an empty request
    cfg = small(dtype=dtype, batch=7, k_resident=K, head_dim=d, n_q_heads=8, n_kv_heads=2,
                planted=0)
    ctx = [16 * 1024, 16 * 1024 + 1, 16 * 2048 + 15, 16 * 5000 - 3, 700, 0, 131072]
    ctx, nbmax, rec, q = setup(cfg, ctx, seed=21, integer=True)
    layer = Layer(cfg, ctx, nbmax)
    assert layer.workspace is not None
    layer.summarize(rec)
    for q_row in (0, 1):
        layer.topk_idx.fill_(-7)
        lib.score_topk(layer.shape, q, layer.summ, layer.ctx_len, layer.topk_idx, layer.topk_score,
                       q_row=q_row, workspace=layer.workspace)
        summ = oracle.summarize(rec.cpu(), ctx, 16)
        sc = oracle.block_scores(q.cpu(), summ, ctx, 16, q_row=q_row)
        idx, val = oracle.topk(sc, ctx, 16, K)
        np.testing.assert_array_equal(i32(layer.topk_idx), idx)
        np.testing.assert_array_equal(host(layer.topk_score).astype(np.float64), val)


def designed_scores(nb: int, pattern: int) -> np.ndarray:
    """Per-block values v_j (all exact in bf16) whose scores G * v_j exercise
    the top-K's distinct paths: all keys equal (no radix round), one outlier
    above a cluster, powers of two over ~120 binades (the highest differing
    bit is the sign/exponent), ties at the threshold, a negative cluster, and
    distinct integers (the search ends early on an exact digit)."""
    j = np.arange(nb)
    if pattern == 0:
        return np.full(nb, 3.0)
    if pattern == 1:
        v = np.ones(nb)
        v[min(7, nb - 1)] = 200.0
        return v
    if pattern == 2:
        e = (j * 37) % 120 - 60
        return np.where(j % 3 == 0, -1.0, 1.0) * np.exp2(e.astype(np.float64))
    if pattern == 3:
        return (j % 5).astype(np.float64)
    if pattern == 4:
        return -(1.0 + (j % 3) / 4.0)
    return ((j * 101) % 256).astype(np.float64)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("K", [16, 128])
def test_topk_designed_key_distributions(dtype, K):
    # one-hot draft and normal queries on channel 0 make block j's score
    # G * (its largest channel-0 key), so each unit's scores follow one
    # designed pattern exactly; the standalone scan + top-K and the fused
    # step must both reproduce the oracle's order bit for bit
    cfg = small(dtype=dtype, batch=3, n_q_heads=8, n_kv_heads=2, head_dim=128, k_resident=K,
                ctx=16000)
    ctx = np.array([16000, 16000 - 40, 2100], np.int32)
    nbmax = cfg.max_blocks(int(ctx.max()))
    B, H, S, d = cfg.batch, cfg.n_kv_heads, cfg.block_size, cfg.head_dim
    rec = torch.zeros((B, H, nbmax, 2, S, d), dtype=torch.float32)    # V = 0: only the order matters
    for b in range(B):
        nb = cfg.max_blocks(int(ctx[b]))
        for h in range(H):
            v = torch.from_numpy(designed_scores(nb, (b * H + h) % 6)).to(torch.float32)
            rec[b, h, :nb, 0, :, 0] = v[:, None]
        tok = torch.arange(nbmax * S).reshape(nbmax, S)
        rec[b, :, :, 0] *= (tok < int(ctx[b])).to(torch.float32)[None, :, :, None]
    dt = gen.TORCH_DTYPE[dtype]
    rec = rec.reshape(B, H, nbmax, 2 * S * d).to(dt).to(DEV)
    q = torch.zeros((B, 2, cfg.n_q_heads, d), dtype=torch.float32)
    q[..., 0] = 1.0
    q = q.to(dt).to(DEV)
    say("designed top-K:", dtype, "K", K, "nbmax", nbmax)
    summ = oracle.summarize(rec.cpu(), ctx, 16)
    sc = oracle.block_scores(q.cpu(), summ, ctx, 16)
    idx, val = oracle.topk(sc, ctx, 16, K)
    layer = Layer(cfg, ctx, nbmax)
    layer.summarize(rec)
    lib.score_topk(layer.shape, q, layer.summ, layer.ctx_len, layer.topk_idx, layer.topk_score,
                   workspace=layer.workspace)
    np.testing.assert_array_equal(i32(layer.topk_idx), idx)
    np.testing.assert_array_equal(host(layer.topk_score).astype(np.float64), val)
    layer.cold_fill(q, rec)
    layer.topk_idx.fill_(-7)
    layer.step(q, 1)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(i32(layer.topk_idx), idx)
    np.testing.assert_array_equal(host(layer.topk_score).astype(np.float64), val)


# --------------------------------------------------------------------------- eviction
@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("K", [8, 128, 256])
def test_capped_evict_bit_exact(seed, K):
    cfg = small(batch=4, k_resident=K, ctx=K * 16 * 3, n_q_heads=8, n_kv_heads=2)
    rng = np.random.default_rng(seed)
    ctx = np.array([cfg.ctx, K * 8, 40, cfg.ctx], np.int32)   # the 3rd has fewer blocks than K
    nbmax = cfg.max_blocks()
    fill = [1.0, 0.6, 0.0, 0.3][seed % 4]
    l2p, p2l, ls = [x.numpy() for x in gen.random_state(cfg, ctx, nbmax, seed, fill=fill,
                                                            stamp_max=6)]
    scores = rng.integers(-4, 5, size=(cfg.batch, cfg.n_kv_heads, nbmax)).astype(np.float64)
    T, _ = oracle.topk(scores, ctx, 16, K)
    layer = Layer(cfg, ctx, nbmax)
    layer.set_state(l2p, p2l, ls)
    m = [0, 1, 6, K][seed]
    lib.capped_evict(layer.shape, torch.from_numpy(T).to(DEV), 7, m, layer.l2p, layer.p2l,
                     layer.last_sel, layer.admit, layer.admit_count)
    l2p_o, p2l_o, ls_o = l2p.copy(), p2l.copy(), ls.copy()
    admit, count = oracle.capped_evict(T, 7, m, l2p_o, p2l_o, ls_o)
    np.testing.assert_array_equal(i32(layer.l2p), l2p_o)
    np.testing.assert_array_equal(i32(layer.p2l), p2l_o)
    np.testing.assert_array_equal(i32(layer.last_sel), ls_o)
    np.testing.assert_array_equal(i32(layer.admit), admit)
    np.testing.assert_array_equal(i32(layer.admit_count), count)


# --------------------------------------------------------------------------- attention
@pytest.mark.parametrize("case", SMALL_CASES, ids=case_id)
@pytest.mark.parametrize("fill", [1.0, 0.5])
def test_lookahead_attention(case, fill):
    cfg = small(**case)
    ctx = RAGGED[:cfg.batch] if cfg.batch > 1 else [cfg.ctx]
    ctx, nbmax, rec, q = setup(cfg, ctx, seed=6)
    l2p, p2l, ls = gen.random_state(cfg, ctx, nbmax, 6, fill=fill)
    layer = Layer(cfg, ctx, nbmax)
    layer.set_state(l2p, p2l, ls)
    layer.pool.copy_(pool_from_records(rec, layer.p2l))
    lib.lookahead_attn(layer.shape, q, layer.pool, layer.p2l, layer.ctx_len, layer.out)
    ref = oracle.attention(q.cpu(), rec.cpu(), p2l, ctx, 16)
    check_attention(layer.out, ref, cfg.dtype, cfg.name)


def test_attention_scale_argument():
    cfg = small(batch=2)
    ctx, nbmax, rec, q = setup(cfg, [1000, 200], seed=7)
    l2p, p2l, ls = gen.random_state(cfg, ctx, nbmax, 7)
    layer = Layer(cfg, ctx, nbmax)
    layer.set_state(l2p, p2l, ls)
    layer.pool.copy_(pool_from_records(rec, layer.p2l))
    lib.lookahead_attn(layer.shape, q, layer.pool, layer.p2l, layer.ctx_len, layer.out, scale=0.3)
    ref = oracle.attention(q.cpu(), rec.cpu(), p2l, ctx, 16, scale=0.3)
    check_attention(layer.out, ref, "bf16")


# --------------------------------------------------------------------------- prefetch
# (batch, admissions per unit): the gather grid follows the item count (one
# workgroup per 32 items between 32 and 128, at least two items per group),
# so these cover 3 workgroups, 15 and 64.
@pytest.mark.parametrize("batch,m", [(3, 5), (3, 1), (64, 16)])
@pytest.mark.parametrize("mode", ["gather", "memcpy"])
@pytest.mark.parametrize("src", ["pinned", "device"])
def test_prefetch(mode, src, batch, m):
    cfg = small(batch=batch, k_resident=16)
    ctxs = [1000, 500, 40] if batch == 3 else [1000 - 13 * i for i in range(batch)]
    ctx, nbmax, rec, q = setup(cfg, ctxs, seed=8, device="cpu")
    l2p, p2l, ls = [x.numpy() for x in gen.random_state(cfg, ctx, nbmax, 8, fill=0.7)]
    scores = np.random.default_rng(8).normal(size=(cfg.batch, cfg.n_kv_heads, nbmax))
    T, _ = oracle.topk(scores, ctx, 16, cfg.k_resident)
    admit, count = oracle.capped_evict(T, 3, m, l2p, p2l, ls)
    layer = Layer(cfg, ctx, nbmax)
    layer.pool.fill_(3)
    layer.admit.copy_(torch.from_numpy(admit))
    layer.admit_count.copy_(torch.from_numpy(count))
    records = rec.pin_memory() if src == "pinned" else rec.to(DEV)
    side = torch.cuda.Stream()
    before = torch.cuda.Event()
    done = torch.cuda.Event()
    before.record()
    staging = torch.empty(cfg.batch * cfg.n_kv_heads * (3 * cfg.k_resident + 1), dtype=torch.int32,
                          pin_memory=True)
    layer.prefetch(records, m, mode=lib.GATHER if mode == "gather" else lib.MEMCPY,
                   host_staging=staging, side_stream=side, wait_before=before, done=done)
    torch.cuda.current_stream().wait_event(done)
    torch.cuda.synchronize()
    ref = np.full(tuple(layer.pool.shape), 0, dtype=np.uint16)
    ref[...] = host(torch.full_like(layer.pool, 3, device="cpu"))
    oracle.prefetch(rec, ref, admit, count, 16)
    np.testing.assert_array_equal(host(layer.pool), ref)


# --------------------------------------------------------------------------- fused step
@pytest.mark.parametrize("case", SMALL_CASES, ids=case_id)
def test_fused_step_equals_separate_calls(case):
    cfg = small(**case)
    ctx = RAGGED[:cfg.batch] if cfg.batch > 1 else [cfg.ctx]
    ctx, nbmax, rec, q = setup(cfg, ctx, seed=9)
    state = gen.random_state(cfg, ctx, nbmax, 9, fill=0.8, stamp_max=3)
    a, b = Layer(cfg, ctx, nbmax), Layer(cfg, ctx, nbmax)
    for L in (a, b):
        L.summarize(rec)
        L.set_state(*state)
        L.pool.copy_(pool_from_records(rec, L.p2l))
    a.step(q, 4)
    b.step_unfused(q, 4)
    torch.cuda.synchronize()
    for name in ("out", "topk_idx", "topk_score", "l2p", "p2l", "last_sel", "admit", "admit_count"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name


@pytest.mark.parametrize("dtype,K,hq,hkv,d", [("bf16", 128, 8, 2, 128), ("f32", 128, 8, 2, 128),
                                              ("bf16", 256, 8, 2, 128), ("bf16", 128, 32, 2, 128),
                                              ("bf16", 64, 8, 2, 64)])
def test_fused_step_split_scan_equals_separate_calls(dtype, K, hq, hkv, d):
    # contexts past 1024 blocks split the scan over several workgroups whose
    # lists the unit's last workgroup to finish merges; the result must equal
    # one workgroup's (separate calls)
    # K = 256 at 8192 blocks: the merge sees its largest input, 8 lists of 256;
    # 32 query heads per 2 KV heads: two row tiles; d = 64
    cfg = small(dtype=dtype, batch=4, k_resident=K, n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                planted=0)
    ctx = [131072, 40000, 16 * 1024 + 1, 900]
    ctx, nbmax, rec, q = setup(cfg, ctx, seed=12)
    assert lib.layer_step_workspace_bytes(lib.Shape.of(cfg, nbmax)) > 0
    state = gen.random_state(cfg, ctx, nbmax, 12, fill=0.9, stamp_max=3)
    a, b = Layer(cfg, ctx, nbmax), Layer(cfg, ctx, nbmax)
    for L in (a, b):
        L.summarize(rec)
        L.set_state(*state)
        L.pool.copy_(pool_from_records(rec, L.p2l))
    for step in (4, 5, 6):          # repeated launches reuse the workspace
        a.step(q, step)
        b.step_unfused(q, step)
        torch.cuda.synchronize()
        for name in ("out", "topk_idx", "topk_score", "l2p", "p2l", "last_sel", "admit",
                     "admit_count"):
            assert torch.equal(getattr(a, name), getattr(b, name)), (step, name)


def fill_garbage(ws: torch.Tensor, kind: int) -> None:
    """Workspace contents a caller might hand over: all ones, random bytes,
    or arrival words holding large counts."""
    if kind == 0:
        ws.fill_(0xFF)
    elif kind == 1:
        g = torch.Generator(device="cpu").manual_seed(77)
        ws.copy_(torch.randint(0, 256, ws.shape, generator=g, dtype=torch.uint8))
    else:
        ws.view(torch.int64)[:].fill_(0x0123456789AB0007)


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_split_step_needs_no_workspace_initialisation(kind):
    # a split unit's workgroups count their arrivals in the workspace; stale or
    # random contents there (another shape's lists, never-written memory)
    # must not change the result
    cfg = small(dtype="bf16", batch=4, k_resident=128, n_q_heads=8, n_kv_heads=2, planted=0)
    ctx = [131072, 40000, 16 * 1024 + 1, 900]
    ctx, nbmax, rec, q = setup(cfg, ctx, seed=31)
    state = gen.random_state(cfg, ctx, nbmax, 31, fill=0.9, stamp_max=3)
    a, b = Layer(cfg, ctx, nbmax), Layer(cfg, ctx, nbmax)
    for L in (a, b):
        L.summarize(rec)
        L.set_state(*state)
        L.pool.copy_(pool_from_records(rec, L.p2l))
    for step in (4, 5):
        fill_garbage(a.workspace, kind)
        a.step(q, step)
        b.step_unfused(q, step)
        torch.cuda.synchronize()
        for name in ("out", "topk_idx", "topk_score", "l2p", "p2l", "last_sel", "admit",
                     "admit_count"):
            assert torch.equal(getattr(a, name), getattr(b, name)), (kind, step, name)
    fill_garbage(a.workspace, kind)
    a.topk_idx.fill_(-7)
    lib.score_topk(a.shape, q, a.summ, a.ctx_len, a.topk_idx, a.topk_score, workspace=a.workspace)
    b.topk_idx.fill_(-9)
    lib.score_topk(b.shape, q, b.summ, b.ctx_len, b.topk_idx, b.topk_score, workspace=b.workspace)
    torch.cuda.synchronize()
    assert torch.equal(a.topk_idx, b.topk_idx) and torch.equal(a.topk_score, b.topk_score)


def test_split_shapes_share_one_workspace():
    # launches of different shapes on one workspace buffer: the arrival words
    # and list slots of one shape overlap other data of the next
    big = small(dtype="bf16", batch=6, k_resident=64, n_q_heads=8, n_kv_heads=2, planted=0)
    ctx_big = [16 * 8192, 16 * 3000 + 5, 16 * 1024 + 1, 16 * 2048, 5, 16 * 6000]
    ctx_big, nb_big, rec_big, q_big = setup(big, ctx_big, seed=32, integer=True)
    sml = small(dtype="bf16", batch=3, k_resident=128, n_q_heads=4, n_kv_heads=4, planted=0)
    ctx_sml = [16 * 1500, 16 * 2100 + 3, 16 * 700]
    ctx_sml, nb_sml, rec_sml, q_sml = setup(sml, ctx_sml, seed=33, integer=True)
    Lb, Ls = Layer(big, ctx_big, nb_big), Layer(sml, ctx_sml, nb_sml)
    shared = Lb.workspace
    assert Ls.workspace is not None and Ls.workspace.numel() <= shared.numel()
    Ls.workspace = shared
    for L, rec, ctx, seed in ((Lb, rec_big, ctx_big, 32), (Ls, rec_sml, ctx_sml, 33)):
        L.summarize(rec)
        L.state0 = gen.random_state(L.cfg, ctx, L.nbmax, seed, fill=0.9, stamp_max=3)
        L.set_state(*L.state0)
        L.pool.copy_(pool_from_records(rec, L.p2l))
    m_b = lib.cap_to_max_admit(big.cap, big.k_resident)
    m_s = lib.cap_to_max_admit(sml.cap, sml.k_resident)
    refs = {}
    for L, cfg, rec, q, ctx, m in ((Lb, big, rec_big, q_big, ctx_big, m_b),
                                   (Ls, sml, rec_sml, q_sml, ctx_sml, m_s)):
        refs[id(L)] = oracle_step(cfg, rec.cpu(), q.cpu(), ctx, L.state0, 5, m)
    # big, small, big again (the small shape's words now sit in the big one's lists)
    for L, q, m in ((Lb, q_big, m_b), (Ls, q_sml, m_s), (Lb, q_big, m_b)):
        L.set_state(*L.state0)
        L.step(q, 5, m)
        torch.cuda.synchronize()
        ref = refs[id(L)]
        check_attention(L.out, ref["out"], L.cfg.dtype)
        np.testing.assert_array_equal(i32(L.topk_idx), ref["idx"])
        for k in ("l2p", "p2l"):
            np.testing.assert_array_equal(i32(getattr(L, k)), ref[k])
        np.testing.assert_array_equal(i32(L.admit), ref["admit"])
        np.testing.assert_array_equal(i32(L.admit_count), ref["count"])


@pytest.mark.parametrize("batch,longest", [(130, 2100), (260, 1100)])
def test_split_step_workgroup_orders(batch, longest):
    # long contexts among many requests: up to 256 requests the scan
    # workgroups follow the length-ordered mapping (here over three 64-request
    # groups), above it the fixed one; both must give the oracle's result
    cfg = small(dtype="bf16", batch=batch, k_resident=16, n_q_heads=4, n_kv_heads=1, head_dim=64,
                planted=0)
    rng = np.random.default_rng(batch)
    ctx = rng.integers(0, 16 * 300, batch)
    longs = rng.choice(batch, 24, replace=False)
    ctx[longs] = rng.integers(16 * 1000, 16 * longest, 24)
    ctx[longs[:2]] = [16 * 1024, 16 * 1024 + 1]                  # on a part boundary
    ctx[longs[2]] = 16 * longest
    ctx, nbmax, rec, q = setup(cfg, ctx, seed=34, integer=True)
    say(f"batch {batch}: NBmax {nbmax}, {int(np.sum(ctx > 16 * 1024))} split requests")
    state = gen.random_state(cfg, ctx, nbmax, 34, fill=0.8, stamp_max=3)
    layer = Layer(cfg, ctx, nbmax)
    layer.summarize(rec)
    layer.set_state(*state)
    layer.pool.copy_(pool_from_records(rec, layer.p2l))
    m = lib.cap_to_max_admit(cfg.cap, cfg.k_resident)
    layer.step(q, 5, m)
    torch.cuda.synchronize()
    ref = oracle_step(cfg, rec.cpu(), q.cpu(), ctx, state, 5, m)
    check_attention(layer.out, ref["out"], cfg.dtype)
    np.testing.assert_array_equal(i32(layer.topk_idx), ref["idx"])
    for k in ("l2p", "p2l"):
        np.testing.assert_array_equal(i32(getattr(layer, k)), ref[k])
    np.testing.assert_array_equal(i32(layer.last_sel), ref["ls"])
    np.testing.assert_array_equal(i32(layer.admit), ref["admit"])
    np.testing.assert_array_equal(i32(layer.admit_count), ref["count"])
    layer.topk_idx.fill_(-7)
    lib.score_topk(layer.shape, q, layer.summ, layer.ctx_len, layer.topk_idx, layer.topk_score,
                   workspace=layer.workspace)
    torch.cuda.synchronize()
    idx, val = oracle.topk(ref["scores"], ctx, 16, cfg.k_resident)
    np.testing.assert_array_equal(i32(layer.topk_idx), idx)
    np.testing.assert_array_equal(host(layer.topk_score).astype(np.float64), val)


def oracle_step(cfg, rec, q, ctx, state, step, m):
    l2p, p2l, ls = [np.ascontiguousarray(x.numpy() if isinstance(x, torch.Tensor) else x,
                                         dtype=np.int32).copy() for x in state]
    summ = oracle.summarize(rec, ctx, 16)
    out, idx, val, admit, count = oracle.layer_step(q, rec, summ, ctx, 16, cfg.k_resident, step, m,
                                                    l2p, p2l, ls)
    sc = oracle.block_scores(q, summ, ctx, 16)
    return dict(out=out, idx=idx, scores=sc, l2p=l2p, p2l=p2l, ls=ls, admit=admit, count=count)


@pytest.mark.parametrize("case", SMALL_CASES, ids=case_id)
def test_fused_step_exact_on_integer_inputs(case):
    cfg = small(**case)
    ctx = RAGGED[:cfg.batch] if cfg.batch > 1 else [cfg.ctx]
    ctx, nbmax, rec, q = setup(cfg, ctx, seed=10, integer=True)
    state = gen.random_state(cfg, ctx, nbmax, 10, fill=0.9, stamp_max=3)
    layer = Layer(cfg, ctx, nbmax)
    layer.summarize(rec)
    layer.set_state(*state)
    layer.pool.copy_(pool_from_records(rec, layer.p2l))
    m = lib.cap_to_max_admit(cfg.cap, cfg.k_resident)
    layer.step(q, 5, m)
    ref = oracle_step(cfg, rec.cpu(), q.cpu(), ctx, state, 5, m)
    check_attention(layer.out, ref["out"], cfg.dtype)
    np.testing.assert_array_equal(i32(layer.topk_idx), ref["idx"])
    for k in ("l2p", "p2l"):
        np.testing.assert_array_equal(i32(getattr(layer, k)), ref[k])
    np.testing.assert_array_equal(i32(layer.last_sel), ref["ls"])
    np.testing.assert_array_equal(i32(layer.admit), ref["admit"])
    np.testing.assert_array_equal(i32(layer.admit_count), ref["count"])


def random_case(seed: int):
    """A seeded random shape: dtype, head dim, heads per KV head (1..16), KV
    heads, K (1..256), slot-pool fill, cap, and per-request contexts within a
    maximum block count that sometimes exceeds one scan part (the split path
    then runs, also for the requests that fit one part)."""
    rng = np.random.default_rng(1000 + seed)
    dtype = "f32" if rng.random() < 0.2 else "bf16"
    d = int(rng.choice([64, 128]))
    hkv = int(rng.integers(1, 5))
    G = int(rng.integers(1, 17))
    batch = int(rng.integers(1, 9 // hkv + 1))
    nbmax = int(rng.choice([64, 500, 1024, 1500] + ([] if dtype == "f32" else [4096])))
    K = int(min(rng.choice([1, 3, 8, 16, 37, 64, 128, 256]), 256))
    ctx = [int(rng.integers(0, nbmax * 16 + 1)) for _ in range(batch)]
    ctx[int(rng.integers(batch))] = int(rng.integers(max(1, nbmax * 16 - 40), nbmax * 16 + 1))
    cap = float(rng.choice([0.0, 0.05, 0.25, 0.5, 1.0, 1.0]))
    fill = float(rng.choice([0.0, 0.5, 0.9, 1.0]))
    cfg = small(dtype=dtype, head_dim=d, n_q_heads=G * hkv, n_kv_heads=hkv, batch=batch,
                k_resident=K, cap=cap, planted=0)
    return cfg, ctx, nbmax, fill


@pytest.mark.parametrize("seed", range(16))
def test_fused_step_random_shapes_exact_on_integer_inputs(seed):
    cfg, ctx, nbmax, fill = random_case(seed)
    say(f"random case {seed}: {cfg.dtype} d={cfg.head_dim} Hq={cfg.n_q_heads} Hkv={cfg.n_kv_heads} "
        f"K={cfg.k_resident} NBmax={nbmax} ctx={ctx} cap={cfg.cap} fill={fill}")
    ctx, nbmax, rec, q = setup(cfg, ctx, seed=40 + seed, integer=True, nbmax=nbmax)
    state = gen.random_state(cfg, ctx, nbmax, 40 + seed, fill=fill, stamp_max=3)
    layer = Layer(cfg, ctx, nbmax)
    layer.summarize(rec)
    layer.set_state(*state)
    layer.pool.copy_(pool_from_records(rec, layer.p2l))
    m = lib.cap_to_max_admit(cfg.cap, cfg.k_resident)
    layer.step(q, 5, m)
    ref = oracle_step(cfg, rec.cpu(), q.cpu(), ctx, state, 5, m)
    check_attention(layer.out, ref["out"], cfg.dtype, f"random case {seed}")
    np.testing.assert_array_equal(i32(layer.topk_idx), ref["idx"])
    for k in ("l2p", "p2l"):
        np.testing.assert_array_equal(i32(getattr(layer, k)), ref[k])
    np.testing.assert_array_equal(i32(layer.last_sel), ref["ls"])
    np.testing.assert_array_equal(i32(layer.admit), ref["admit"])
    np.testing.assert_array_equal(i32(layer.admit_count), ref["count"])


# --------------------------------------------------------------------------- edge cases
EDGE_CASES = [
    dict(k_resident=1, ctx=1000, batch=2),                       # one slot per unit
    dict(n_q_heads=2, n_kv_heads=2, k_resident=8),                # G = 1 (2 stacked rows)
    dict(k_resident=256, ctx=16 * 256 * 2, batch=2),              # largest K
    dict(k_resident=64, ctx=500, batch=3),                        # fewer blocks than slots
    dict(dtype="f32", k_resident=5, ctx=333, n_q_heads=3, n_kv_heads=1),
]


@pytest.mark.parametrize("case", EDGE_CASES, ids=case_id)
def test_fused_step_edge_cases(case):
    cfg = small(**case)
    ctx = np.array([cfg.ctx, 1, 0][:cfg.batch] if cfg.batch >= 2 else [cfg.ctx], np.int32)
    if cfg.batch > 3:
        ctx = np.full(cfg.batch, cfg.ctx, np.int32)
    ctx, nbmax, rec, q = setup(cfg, ctx, seed=13, integer=True)
    state = gen.random_state(cfg, ctx, nbmax, 13, fill=0.7, stamp_max=2)
    layer = Layer(cfg, ctx, nbmax)
    layer.summarize(rec)
    layer.set_state(*state)
    layer.pool.copy_(pool_from_records(rec, layer.p2l))
    m = max(1, lib.cap_to_max_admit(cfg.cap, cfg.k_resident))
    layer.step(q, 3, m)
    ref = oracle_step(cfg, rec.cpu(), q.cpu(), ctx, state, 3, m)
    check_attention(layer.out, ref["out"], cfg.dtype, str(case))
    np.testing.assert_array_equal(i32(layer.topk_idx), ref["idx"])
    np.testing.assert_array_equal(i32(layer.p2l), ref["p2l"])
    np.testing.assert_array_equal(i32(layer.l2p), ref["l2p"])
    np.testing.assert_array_equal(i32(layer.admit), ref["admit"])


def test_empty_resident_set_gives_zero_output():
    cfg = small(batch=2)
    ctx, nbmax, rec, q = setup(cfg, [1000, 40], seed=14)
    layer = Layer(cfg, ctx, nbmax)          # every slot empty
    layer.summarize(rec)
    layer.out.fill_(5)
    lib.lookahead_attn(layer.shape, q, layer.pool, layer.p2l, layer.ctx_len, layer.out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(layer.out).item() == 0
    # and the fused step fills the empty slots from the top-K, stamping them
    layer.step(q, 1, cfg.k_resident)
    torch.cuda.synchronize()
    assert int(layer.admit_count.sum()) == int(sum(min(cfg.k_resident, -(-c // 16)) for c in ctx)) * cfg.n_kv_heads


def test_zero_batch_launches_nothing():
    cfg = small(batch=1)
    ctx, nbmax, rec, q = setup(cfg, [300], seed=15)
    layer = Layer(cfg, ctx, nbmax)
    empty = lib.Shape.of(cfg, nbmax, batch=0)
    p = torch.empty(0, device="cuda")
    raw = lib.raw()
    import ctypes
    assert raw.oasis_layer_step(ctypes.byref(empty), *([None] * 4), 0.0, 1, 6, *([None] * 8), None,
                                0, None) == lib.OK
