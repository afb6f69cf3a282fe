"""Pins of the CPU oracle to facts other than itself: hand-worked examples,
closed forms, library routines, brute force and the invariants the OasisKV
pages state.  None of these tests needs a GPU."""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from sparse_kv_block_amd import gen
from sparse_kv_block_amd.configs import TINY, QWEN3_8B_16K, FULL_36, Config

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tiny(**kw) -> Config:
    base = dict(name="t", dtype="f32", batch=2, n_q_heads=4, n_kv_heads=2, head_dim=8,
                block_size=4, ctx=37, k_resident=4, cap=0.5, draft_sigma=0.1, rho=0.9,
                seed=17)
    base.update(kw)
    return Config(**base)


def make(cfg, ctx=None, nbmax=None, seed=0):
    ctx = gen.context_lengths(cfg) if ctx is None else np.asarray(ctx, np.int32)
    nbmax = nbmax or cfg.max_blocks(int(ctx.max()))
    rec = gen.records(cfg, ctx, nbmax, seed=seed + 5)
    qs = gen.query_sequence(cfg, 2, seed=seed + 9)
    q = gen.step_queries(cfg, qs, 1, seed=seed + 9)
    return ctx, nbmax, rec, q


def f64(x):
    import oracle
    return oracle.to_f64(oracle.as_np(x))


def keys_values(cfg, rec):
    """Token-major keys and values [B][H][NB*S][d] from the record layout."""
    import oracle
    r = oracle.to_f64(oracle.as_np(rec))
    B, H, NB, _ = r.shape
    S, d = cfg.block_size, cfg.head_dim
    k = r[..., : S * d].reshape(B, H, NB, S, d).reshape(B, H, NB * S, d)
    v = r[..., S * d:].reshape(B, H, NB, d, S).transpose(0, 1, 2, 4, 3).reshape(B, H, NB * S, d)
    return k, v


# --------------------------------------------------------------------------
# Summaries
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_summaries_are_numpy_min_max_of_valid_keys(ora, dtype):
    cfg = tiny(dtype=dtype, batch=3)
    ctx = np.array([37, 16, 1], np.int32)         # ragged tail, exact block, one token
    ctx_, nbmax, rec, _ = make(cfg, ctx, nbmax=12)
    summ = ora.summarize(rec, ctx, cfg.block_size)
    k, _ = keys_values(cfg, rec)
    s = ora.to_f64(summ)
    S = cfg.block_size
    for b in range(cfg.batch):
        nb = -(-int(ctx[b]) // S)
        for j in range(nb):
            valid = k[b, :, j * S: min((j + 1) * S, int(ctx[b]))]
            np.testing.assert_array_equal(s[b, :, j, 0], valid.min(axis=1))
            np.testing.assert_array_equal(s[b, :, j, 1], valid.max(axis=1))
        assert not np.any(s[b, :, nb:]), "blocks past the context must stay untouched"


def test_summary_is_one_sixteenth_of_kv():
    # pith.science paper page, free parameters: summaries about 1/16 of the KV
    # size.  One block holds 2*S*d KV elements and 2*d summary elements.
    S, d = 16, 128
    assert (2 * d) / (2 * S * d) == 1 / 16


# --------------------------------------------------------------------------
# Scores
def test_score_worked_example(ora):
    g = json.load(open(os.path.join(GOLDEN, "score_worked_example.json")))
    S, d = g["block_size"], g["head_dim"]
    keys = np.array(g["keys_by_token"], np.float32)            # [L][d]
    L = keys.shape[0]
    NB = L // S
    rec = np.zeros((1, 1, NB, 2 * S * d), np.float32)
    for j in range(NB):
        rec[0, 0, j, : S * d] = keys[j * S:(j + 1) * S].reshape(-1)
    ctx = np.array([g["ctx_len"]], np.int32)
    summ = ora.summarize(rec, ctx, S)
    np.testing.assert_array_equal(summ[0, 0, :, 0], np.array(g["summary_min"], np.float32))
    np.testing.assert_array_equal(summ[0, 0, :, 1], np.array(g["summary_max"], np.float32))
    q = np.zeros((1, 2, g["n_q_heads"], d), np.float32)
    q[0, 1] = np.array(g["draft_q_by_head"], np.float32)
    q[0, 0] = 100.0                                           # the normal row must not matter
    sc = ora.block_scores(q, summ, ctx, S, q_row=1)
    np.testing.assert_array_equal(sc[0, 0], np.array(g["scores"], np.float64))
    idx, _ = ora.topk(sc, ctx, S, 1)
    assert idx[0, 0].tolist() == g["top1"]


@pytest.mark.parametrize("G", [1, 4])
def test_score_upper_bounds_every_token_logit(ora, G):
    # Quest bound: for every block, sum_c max(q_c min_c, q_c max_c) >= q.k_t for
    # each valid token t; for a group, the sum of the per-head bounds is >= the
    # group's summed logit sum_i q_i.k_t.
    cfg = tiny(n_q_heads=2 * G, n_kv_heads=2, head_dim=16, ctx=203, batch=2)
    ctx, nbmax, rec, q = make(cfg, seed=3)
    summ = ora.summarize(rec, ctx, cfg.block_size)
    sc = ora.block_scores(q, summ, ctx, cfg.block_size, q_row=1)
    k, _ = keys_values(cfg, rec)
    qd = f64(q)[:, 1]                                          # [B][Hq][d]
    S = cfg.block_size
    for b in range(cfg.batch):
        for h in range(cfg.n_kv_heads):
            qg = qd[b, h * G:(h + 1) * G].sum(axis=0)
            logit = k[b, h, : int(ctx[b])] @ qg
            nb = -(-int(ctx[b]) // S)
            for j in range(nb):
                exact = logit[j * S:(j + 1) * S].max()
                assert sc[b, h, j] >= exact - 1e-9 * (1 + abs(exact))
            assert np.all(np.isneginf(sc[b, h, nb:]))


def test_sign_split_factoring_of_the_group_bound_equals_the_definition(ora):
    # The HIP scan factors the group bound per channel as
    # min_c * sum_i min(q_ic, 0) + max_c * sum_i max(q_ic, 0) (valid for
    # min_c <= max_c); in fp64 that must reproduce the oracle's definition
    # sum_i sum_c max(q_ic min_c, q_ic max_c) on real summaries, including
    # zero query rows and a partial last block.
    cfg = tiny(n_q_heads=8, n_kv_heads=2, head_dim=16, ctx=203, batch=2)
    ctx, nbmax, rec, q = make(cfg, seed=21)
    q = q.clone()
    q[0, 1, :3] = 0.0                                          # some zero query rows
    qd = f64(q)
    summ = ora.summarize(rec, ctx, cfg.block_size)
    sc = ora.block_scores(q, summ, ctx, cfg.block_size, q_row=1)
    sm = f64(summ)                                             # [B][H][NB][2][d]
    G = cfg.group
    for b in range(cfg.batch):
        nb = -(-int(ctx[b]) // cfg.block_size)
        for h in range(cfg.n_kv_heads):
            qg = qd[b, 1, h * G:(h + 1) * G]                  # [G][d]
            neg, pos = np.minimum(qg, 0).sum(axis=0), np.maximum(qg, 0).sum(axis=0)
            mn, mx = sm[b, h, :nb, 0], sm[b, h, :nb, 1]
            assert np.all(mn <= mx)
            fact = mn @ neg + mx @ pos
            np.testing.assert_allclose(fact, sc[b, h, :nb], rtol=1e-12, atol=1e-12)


def test_score_with_one_token_blocks_is_the_dot_product(ora):
    # With S = 1 the summary min and max both equal the key, so the bound is
    # exact: score(j) = sum_i q_i . k_j (grouped query heads of the KV head).
    cfg = tiny(block_size=1, ctx=29, n_q_heads=6, n_kv_heads=2, head_dim=8)
    ctx, nbmax, rec, q = make(cfg, seed=4)
    summ = ora.summarize(rec, ctx, 1)
    sc = ora.block_scores(q, summ, ctx, 1, q_row=1)
    k, _ = keys_values(cfg, rec)
    qd = f64(q)[:, 1].reshape(cfg.batch, cfg.n_kv_heads, cfg.group, cfg.head_dim).sum(axis=2)
    expect = np.einsum("bhtd,bhd->bht", k, qd)
    np.testing.assert_allclose(sc, expect, rtol=1e-13, atol=1e-13)
    # and the top-K is the exact dot-product top-K (lexsort on -score, index)
    idx, _ = ora.topk(sc, ctx, 1, 5)
    for b in range(cfg.batch):
        for h in range(cfg.n_kv_heads):
            order = np.lexsort((np.arange(29), -expect[b, h]))
            assert idx[b, h].tolist() == order[:5].tolist()


def test_zero_query_scores_zero_and_picks_lowest_blocks(ora):
    cfg = tiny(ctx=64)
    ctx, nbmax, rec, q = make(cfg, seed=5)
    q = torch.zeros_like(q)
    summ = ora.summarize(rec, ctx, cfg.block_size)
    sc = ora.block_scores(q, summ, ctx, cfg.block_size)
    assert np.all(sc == 0.0)
    idx, val = ora.topk(sc, ctx, cfg.block_size, cfg.k_resident)
    assert np.all(idx == np.arange(cfg.k_resident))


# --------------------------------------------------------------------------
# Top-K
def brute_topk(s, n, K):
    rank = [sum(1 for jj in range(n) if s[jj] > s[j] or (s[jj] == s[j] and jj < j))
            for j in range(n)]
    out = [-1] * K
    for j in range(n):
        if rank[j] < K:
            out[rank[j]] = j
    return out


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_brute_force_ranks_with_ties(ora, seed):
    rng = np.random.default_rng(seed)
    B, H, NB, S, K = 3, 2, 40, 16, 7
    scores = rng.integers(-3, 4, size=(B, H, NB)).astype(np.float64)   # many ties
    scores[0, 0, 3] = -0.0                                             # -0 equals +0
    ctx = np.array([NB * S, 5 * S - 3, 0], np.int32)                   # full, 5 blocks, empty
    idx, val = ora.topk(scores, ctx, S, K)
    for b in range(B):
        n = min(NB, -(-int(ctx[b]) // S))
        for h in range(H):
            assert idx[b, h].tolist() == brute_topk(scores[b, h], n, K)
            kk = min(K, n)
            np.testing.assert_array_equal(val[b, h, :kk], scores[b, h, idx[b, h, :kk]])
            assert np.all(np.isneginf(val[b, h, kk:]))


# --------------------------------------------------------------------------
# Capped eviction
@pytest.mark.parametrize("name", ["evict_worked_example.json", "evict_lrs_order_example.json"])
def test_evict_worked_example(ora, name):
    g = json.load(open(os.path.join(GOLDEN, name)))
    K, NB = g["K"], g["n_blocks"]
    p2l = np.array([[g["p2l_before"]]], np.int32)
    last = np.array([[g["last_sel_before"]]], np.int32)
    l2p = np.full((1, 1, NB), -1, np.int32)
    for s, j in enumerate(g["p2l_before"]):
        if j >= 0:
            l2p[0, 0, j] = s
    T = np.array([[g["topk"]]], np.int32)
    admit, count = ora.capped_evict(T, g["step"], g["max_admit"], l2p, p2l, last)
    assert p2l[0, 0].tolist() == g["p2l_after"]
    assert last[0, 0].tolist() == g["last_sel_after"]
    assert l2p[0, 0].tolist() == g["l2p_after"]
    assert admit[0, 0].tolist() == g["admit"]
    assert int(count[0, 0]) == g["admit_count"]


def check_evict_invariants(T, step, m, before, after, admit, count):
    l2p0, p2l0, ls0 = before
    l2p1, p2l1, ls1 = after
    B, H, K = p2l0.shape
    for b in range(B):
        for h in range(H):
            t = [j for j in T[b, h] if j >= 0]
            R0 = {j for j in p2l0[b, h] if j >= 0}
            R1 = {j for j in p2l1[b, h] if j >= 0}
            a = int(count[b, h])
            miss = [j for j in t if j not in R0]
            empty0 = int((p2l0[b, h] < 0).sum())
            assert a <= m and a <= len(miss)
            assert a == min(m, len(miss)), "enough victims always exist for a consistent state"
            adm = admit[b, h, :a, 0].tolist()
            assert adm == miss[:a], "admissions follow the top-K order"
            evicted = {int(e) for e in admit[b, h, :a, 2] if e >= 0}
            assert not (evicted & set(t)), "a block of the top-K is never evicted"
            assert R1 == (R0 - evicted) | set(adm)
            filled = sum(1 for e in admit[b, h, :a, 2] if e < 0)
            assert len(R1) == len(R0) + filled and filled <= empty0
            assert len(R1 & set(t)) == len(R0 & set(t)) + a
            # l2p and p2l are mutual inverses without duplicates
            for s in range(K):
                j = p2l1[b, h, s]
                if j >= 0:
                    assert l2p1[b, h, j] == s
            assert int((l2p1[b, h] >= 0).sum()) == len(R1)
            for s in range(K):
                if p2l1[b, h, s] in set(t):
                    assert ls1[b, h, s] == step
            assert np.all(admit[b, h, a:] == -1)
            # victim order: empty slots first, in slot order; then the least
            # recently selected resident blocks outside the top-K, by (stamp,
            # block).  Stamps are the ones before this step (a top-K member is
            # never a candidate, so its refresh to `step` does not matter).
            slots = admit[b, h, :a, 1].tolist()
            empties = [s for s in range(K) if p2l0[b, h, s] < 0]
            assert slots[:filled] == empties[:filled], "empty slots are filled first, in slot order"
            if filled < a:
                assert filled == empty0, "a resident block is evicted only once no slot is empty"
            cand = [(int(ls0[b, h, s]), int(p2l0[b, h, s]), s) for s in range(K)
                    if p2l0[b, h, s] >= 0 and p2l0[b, h, s] not in set(t) and ls0[b, h, s] < step]
            chosen = [(int(ls0[b, h, s]), int(p2l0[b, h, s]), s) for s in slots[filled:]]
            assert chosen == sorted(chosen), "victims are taken least recently selected first"
            kept = [c for c in cand if c[2] not in set(slots)]
            if chosen and kept:
                assert max(chosen) < min(kept), (
                    "every evicted block was selected no more recently than every kept stale block "
                    "(ties: lower block first)")


@pytest.mark.parametrize("seed", range(8))
def test_evict_invariants_random(ora, seed):
    rng = np.random.default_rng(seed)
    cfg = tiny(batch=3, k_resident=int(rng.integers(1, 12)), ctx=int(rng.integers(1, 300)))
    K = cfg.k_resident
    ctx = np.array([cfg.ctx, max(1, cfg.ctx // 2), cfg.ctx], np.int32)
    nbmax = cfg.max_blocks()
    l2p, p2l, ls = [x.numpy().copy() for x in
                    gen.random_state(cfg, ctx, nbmax, seed, fill=float(rng.uniform(0, 1)), stamp_max=5)]
    scores = rng.normal(size=(cfg.batch, cfg.n_kv_heads, nbmax))
    T, _ = ora.topk(scores, ctx, cfg.block_size, K)
    m = int(rng.integers(0, K + 1))
    before = (l2p.copy(), p2l.copy(), ls.copy())
    admit, count = ora.capped_evict(T, 5, m, l2p, p2l, ls)
    check_evict_invariants(T, 5, m, before, (l2p, p2l, ls), admit, count)


def random_evict_case(rng):
    """A consistent random state of a few units: K slots, NB blocks, a fill,
    stamps below the step (some at or above it: never victims), a top-K list
    of distinct blocks (fewer than K when the request is short) and a cap."""
    B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    K = int(rng.integers(1, 17))
    NB = int(rng.integers(1, 40))
    step = int(rng.integers(1, 9))
    l2p = np.full((B, H, NB), -1, np.int32)
    p2l = np.full((B, H, K), -1, np.int32)
    ls = rng.integers(0, step + 2, size=(B, H, K)).astype(np.int32)
    T = np.full((B, H, K), -1, np.int32)
    for b in range(B):
        for h in range(H):
            n = int(rng.integers(0, min(K, NB) + 1))
            blocks = rng.choice(NB, size=n, replace=False)
            slots = rng.choice(K, size=n, replace=False)
            p2l[b, h, slots] = blocks
            l2p[b, h, blocks] = slots
            nt = int(rng.integers(0, min(K, NB) + 1))
            T[b, h, :nt] = rng.choice(NB, size=nt, replace=False)
    m = int(rng.integers(0, K + 2))
    return T, step, m, l2p, p2l, ls


def assert_evict_matches_numpy(ora, T, step, m, l2p, p2l, ls):
    import evict_np
    want = evict_np.capped_evict(T, step, m, l2p, p2l, ls)
    before = (l2p.copy(), p2l.copy(), ls.copy())
    admit, count = ora.capped_evict(T, step, m, l2p, p2l, ls)
    for name, got, exp in zip(("l2p", "p2l", "last_sel", "admit", "admit_count"),
                              (l2p, p2l, ls, admit, count), want):
        np.testing.assert_array_equal(got, exp, err_msg=f"{name} differs from the numpy eviction")
    return before, admit, count


@pytest.mark.parametrize("seed", range(40))
def test_evict_matches_independent_numpy_eviction(ora, seed):
    rng = np.random.default_rng(700 + seed)
    T, step, m, l2p, p2l, ls = random_evict_case(rng)
    before, admit, count = assert_evict_matches_numpy(ora, T, step, m, l2p, p2l, ls)
    if np.all(before[2] < step):
        check_evict_invariants(T, step, m, before, (l2p, p2l, ls), admit, count)


def test_evict_matches_numpy_at_full_unit_size(ora):
    # one batch of the Qwen3-8B shape's per-unit sizes: K = 128 slots over 1024
    # blocks, cap 0.05 (6 admissions), stamps spread over the previous steps
    cfg = QWEN3_8B_16K.scaled(batch=4)
    ctx = gen.context_lengths(cfg)
    nbmax = cfg.max_blocks()
    l2p, p2l, ls = [x.numpy().copy() for x in gen.random_state(cfg, ctx, nbmax, 3, fill=0.97,
                                                               stamp_max=9)]
    scores = np.random.default_rng(3).normal(size=(cfg.batch, cfg.n_kv_heads, nbmax))
    T, _ = ora.topk(scores, ctx, cfg.block_size, cfg.k_resident)
    m = ora.max_admit(cfg.cap, cfg.k_resident)
    before, admit, count = assert_evict_matches_numpy(ora, T, 9, m, l2p, p2l, ls)
    check_evict_invariants(T, 9, m, before, (l2p, p2l, ls), admit, count)
    assert int(count.min()) == m


def test_evict_zero_cap_only_stamps(ora):
    cfg = tiny(k_resident=6, ctx=300)
    ctx = gen.context_lengths(cfg)
    nbmax = cfg.max_blocks()
    l2p, p2l, ls = [x.numpy().copy() for x in gen.random_state(cfg, ctx, nbmax, 1, stamp_max=3)]
    scores = np.random.default_rng(1).normal(size=(cfg.batch, cfg.n_kv_heads, nbmax))
    T, _ = ora.topk(scores, ctx, cfg.block_size, 6)
    l0, p0 = l2p.copy(), p2l.copy()
    admit, count = ora.capped_evict(T, 9, 0, l2p, p2l, ls)
    assert np.all(count == 0) and np.all(admit == -1)
    np.testing.assert_array_equal(l2p, l0)
    np.testing.assert_array_equal(p2l, p0)


def test_evict_uncapped_makes_topk_resident(ora):
    cfg = tiny(k_resident=6, ctx=300)
    ctx = gen.context_lengths(cfg)
    nbmax = cfg.max_blocks()
    l2p, p2l, ls = [x.numpy().copy() for x in gen.random_state(cfg, ctx, nbmax, 2, stamp_max=3)]
    scores = np.random.default_rng(2).normal(size=(cfg.batch, cfg.n_kv_heads, nbmax))
    T, _ = ora.topk(scores, ctx, cfg.block_size, 6)
    ora.capped_evict(T, 9, 6, l2p, p2l, ls)
    for b in range(cfg.batch):
        for h in range(cfg.n_kv_heads):
            assert set(T[b, h].tolist()) <= set(p2l[b, h].tolist())


# --------------------------------------------------------------------------
# Attention
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_attention_with_every_block_resident_is_dense_attention(ora, dtype):
    cfg = tiny(dtype=dtype, ctx=45, k_resident=16)      # NB = 12 <= K
    ctx = np.array([45, 13], np.int32)
    ctx, nbmax, rec, q = make(cfg, ctx, seed=6)
    K = cfg.k_resident
    p2l = np.full((cfg.batch, cfg.n_kv_heads, K), -1, np.int32)
    rng = np.random.default_rng(0)
    for b in range(cfg.batch):
        nb = -(-int(ctx[b]) // cfg.block_size)
        for h in range(cfg.n_kv_heads):
            p2l[b, h, rng.permutation(K)[:nb]] = np.arange(nb)   # any slot order
    out = ora.attention(q, rec, p2l, ctx, cfg.block_size)
    k, v = keys_values(cfg, rec)
    qd = f64(q)
    scale = 1 / math.sqrt(cfg.head_dim)
    for b in range(cfg.batch):
        L = int(ctx[b])
        for r in range(2):
            for i in range(cfg.n_q_heads):
                h = i // cfg.group
                w = scipy.special.softmax(scale * (k[b, h, :L] @ qd[b, r, i]))
                np.testing.assert_allclose(out[b, r, i], w @ v[b, h, :L], rtol=1e-12, atol=1e-12)


def test_attention_special_cases(ora):
    cfg = tiny(ctx=40)
    ctx = np.array([40, 33], np.int32)
    ctx, nbmax, rec, q = make(cfg, ctx, seed=7)
    K = cfg.k_resident
    k, v = keys_values(cfg, rec)
    # exactly one valid token (block 8 of request 1 holds token 32 only) -> o = v
    p2l = np.full((2, cfg.n_kv_heads, K), -1, np.int32)
    p2l[1, :, 2] = 8
    out = ora.attention(q, rec, p2l, ctx, cfg.block_size)
    for i in range(cfg.n_q_heads):
        h = i // cfg.group
        np.testing.assert_allclose(out[1, :, i], np.broadcast_to(v[1, h, 32], (2, cfg.head_dim)),
                                   rtol=1e-14, atol=0)
    # empty resident set -> 0
    np.testing.assert_array_equal(out[0], 0.0)
    # zero query -> equal logits -> mean of the resident values
    p2l[0, :, 0] = 1
    p2l[0, :, 3] = 4
    out = ora.attention(torch.zeros_like(q), rec, p2l, ctx, cfg.block_size)
    for i in range(cfg.n_q_heads):
        h = i // cfg.group
        toks = list(range(4, 8)) + list(range(16, 20))
        np.testing.assert_allclose(out[0, 0, i], v[0, h, toks].mean(axis=0), rtol=1e-13, atol=1e-15)


# --------------------------------------------------------------------------
# Prefetch
def test_prefetch_copies_whole_records(ora):
    cfg = tiny(dtype="bf16", ctx=100)
    ctx, nbmax, rec, _ = make(cfg, seed=8)
    recn = ora.as_np(rec)
    K = cfg.k_resident
    pool = np.zeros((cfg.batch, cfg.n_kv_heads, K, recn.shape[-1]), np.uint16)
    admit = np.full((cfg.batch, cfg.n_kv_heads, K, 3), -1, np.int32)
    count = np.zeros((cfg.batch, cfg.n_kv_heads), np.int32)
    admit[0, 1, 0] = (5, 2, -1)
    admit[1, 0, :2] = [(0, 3, 7), (6, 0, -1)]
    count[0, 1], count[1, 0] = 1, 2
    ora.prefetch(rec, pool, admit, count, cfg.block_size)
    np.testing.assert_array_equal(pool[0, 1, 2], recn[0, 1, 5])
    np.testing.assert_array_equal(pool[1, 0, 3], recn[1, 0, 0])
    np.testing.assert_array_equal(pool[1, 0, 0], recn[1, 0, 6])
    assert int((pool != 0).any(axis=-1).sum()) == 3


# --------------------------------------------------------------------------
# Cap rounding and the byte model against the pages' numbers
def test_cap_rounding(ora):
    assert [ora.max_admit(c, 128) for c in (0.0, 0.01, 0.05, 0.2, 1.0)] == [0, 1, 6, 25, 128]
    assert ora.max_admit(0.25, 8) == 2 == ora.max_admit(TINY.cap, TINY.k_resident)
    assert ora.max_admit(QWEN3_8B_16K.cap, QWEN3_8B_16K.k_resident) == 6


def test_bytes_per_step_at_cap_001_is_the_pages_030_gb(ora):
    # agihunt.info summary, fetch-cap ablation: cap 0.01 moves 0.30 GB per step.
    # Batch 128, 8 KV heads, 36 layers, one 16-token bf16 K+V block of d=128
    # (8 KiB) per KV head and layer when the cap saturates.
    c = FULL_36
    rec_bytes = 2 * c.block_size * c.head_dim * 2
    per_step = c.batch * c.n_kv_heads * c.layers * ora.max_admit(0.01, c.k_resident) * rec_bytes
    assert abs(per_step / 1e9 - 0.30) < 0.005
    # rounding up instead of down would double it
    assert abs(2 * per_step / 1e9 - 0.30) > 0.25


def test_kv_bytes_per_request_is_the_pages_86_gb():
    # agihunt.info summary, opening paragraph: a 32B GQA model at 32.7K
    # context needs 8.6 GB of KV per request (64 layers, 8 KV heads, d = 128,
    # bf16 K and V).
    per_token = 64 * 8 * 128 * 2 * 2
    assert abs(per_token * 32.7e3 / 1e9 - 8.6) < 0.05


# --------------------------------------------------------------------------
# Decode append
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_append_places_tokens_and_keeps_summaries_exact(ora, dtype):
    # Appending tokens one at a time must give the same records as placing
    # them directly (key row t%S, value column t%S of block t/S) and summaries
    # equal to a fresh summarize of the result (itself pinned to numpy).
    cfg = tiny(dtype=dtype, batch=3, head_dim=8, block_size=4, k_resident=3)
    ctx0 = np.array([5, 0, 12], np.int32)          # mid-block, empty, block boundary
    nb = 6                                         # capacity 24 tokens
    ctx, _, rec, _ = make(cfg, ctx0, nbmax=nb, seed=21)
    rec = ora.as_np(rec).copy()
    summ = ora.summarize(rec, ctx0, 4)
    ctx = ctx0.copy()
    rng = np.random.default_rng(3)
    H, d, S = cfg.n_kv_heads, cfg.head_dim, cfg.block_size
    expect = rec.copy()
    pool = np.zeros((3, H, 3, rec.shape[-1]), rec.dtype)
    l2p = np.full((3, H, nb), -1, np.int32)
    l2p[2, 1, 3] = 2                               # block 3 of request 2, head 1 resident
    pool[2, 1, 2] = rec[2, 1, 3]
    for step in range(14):
        kf = rng.integers(-4, 5, size=(3, H, d)).astype(np.float32)
        vf = rng.integers(-4, 5, size=(3, H, d)).astype(np.float32)
        if dtype == "bf16":
            kn = (kf.view(np.uint32) >> 16).astype(np.uint16)
            vn = (vf.view(np.uint32) >> 16).astype(np.uint16)
        else:
            kn, vn = kf, vf
        for b in range(3):
            t = ctx[b]
            if t >= nb * S:
                continue
            j, u = divmod(int(t), S)
            for h in range(H):
                expect[b, h, j, u * d:(u + 1) * d] = kn[b, h]
                expect[b, h, j, S * d + u::S][:d] = vn[b, h]
        before = ctx.copy()
        ora.append(kn, vn, rec, summ, ctx, S, pool=pool, l2p=l2p)
        np.testing.assert_array_equal(ctx, np.where(before >= nb * S, before, before + 1))
    np.testing.assert_array_equal(rec, expect)
    np.testing.assert_array_equal(ora.to_f64(summ), ora.to_f64(ora.summarize(rec, ctx, S)))
    np.testing.assert_array_equal(pool[2, 1, 2], rec[2, 1, 3])
    assert ctx.tolist() == [19, 14, 24]            # request 2 stopped at capacity


# --------------------------------------------------------------------------
# Exact block scores and top-K agreement (the diagnostic's ground truth)
def test_exact_score_worked_example(ora):
    g = json.load(open(os.path.join(GOLDEN, "exact_score_worked_example.json")))
    S, d = g["block_size"], g["head_dim"]
    keys = np.array(g["keys_by_token"], np.float32)
    NB = keys.shape[0] // S
    rec = np.zeros((1, 1, NB, 2 * S * d), np.float32)
    for j in range(NB):
        rec[0, 0, j, : S * d] = keys[j * S:(j + 1) * S].reshape(-1)
    ctx = np.array([g["ctx_len"]], np.int32)
    q = np.full((1, 2, g["n_q_heads"], d), 50.0, np.float32)      # row 1 must not matter
    q[0, 0] = np.array(g["q_by_head"], np.float32)
    ex = ora.exact_block_scores(q, rec, ctx, S, q_row=0)
    np.testing.assert_array_equal(ex[0, 0], np.array(g["exact_scores"], np.float64))
    summ = ora.summarize(rec, ctx, S)
    qs = ora.block_scores(q, summ, ctx, S, q_row=0)
    np.testing.assert_array_equal(qs[0, 0], np.array(g["quest_scores"], np.float64))
    idx, _ = ora.topk(ex, ctx, S, 1)
    assert idx[0, 0].tolist() == g["top1"]
    # the other query row is read when asked for
    q2 = q[:, ::-1].copy()
    np.testing.assert_array_equal(ora.exact_block_scores(q2, rec, ctx, S, q_row=1), ex)


def test_exact_scores_equal_the_bound_for_one_token_blocks(ora):
    # With S = 1 a block's min and max are its key, so the Quest bound is exact
    # and the two independently computed scores must coincide.
    cfg = tiny(block_size=1, ctx=41, n_q_heads=6, n_kv_heads=2, head_dim=8, batch=3)
    ctx, nbmax, rec, q = make(cfg, ctx=[41, 7, 0], seed=8)
    summ = ora.summarize(rec, ctx, 1)
    for row in (0, 1):
        ex = ora.exact_block_scores(q, rec, ctx, 1, q_row=row)
        qs = ora.block_scores(q, summ, ctx, 1, q_row=row)
        np.testing.assert_allclose(ex, qs, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_exact_scores_never_exceed_the_bound(ora, dtype):
    cfg = tiny(dtype=dtype, n_q_heads=8, n_kv_heads=2, head_dim=16, ctx=333, batch=2)
    ctx, nbmax, rec, q = make(cfg, ctx=[333, 100], seed=9)
    summ = ora.summarize(rec, ctx, cfg.block_size)
    ex = ora.exact_block_scores(q, rec, ctx, cfg.block_size, q_row=1)
    qs = ora.block_scores(q, summ, ctx, cfg.block_size, q_row=1)
    fin = np.isfinite(qs)
    assert np.array_equal(fin, np.isfinite(ex))
    assert np.all(ex[fin] <= qs[fin] + 1e-9 * (1 + np.abs(qs[fin])))
    # and the bound is not trivially loose: some block comes within 30 %
    assert np.any(ex[fin] > 0.7 * qs[fin])


def test_exact_scores_ignore_token_order_and_duplicates(ora):
    # The max over a block's tokens does not depend on their order, and
    # replacing a token by a copy of another token of the block cannot raise it.
    cfg = tiny(head_dim=8, ctx=64, n_q_heads=4, n_kv_heads=1, batch=1)
    ctx, nbmax, rec, q = make(cfg, seed=10)
    S, d = cfg.block_size, cfg.head_dim
    ex = ora.exact_block_scores(q, rec, ctx, S, q_row=0)
    r = ora.as_np(rec).copy()
    k = r[..., : S * d].reshape(1, 1, nbmax, S, d)
    k[:] = k[:, :, :, ::-1].copy()
    np.testing.assert_allclose(ora.exact_block_scores(q, r, ctx, S, q_row=0), ex, rtol=1e-12)
    k[:, :, :, 0] = k[:, :, :, 1]
    assert np.all(ora.exact_block_scores(q, r, ctx, S, q_row=0) <= ex + 1e-12)


def test_agreement_counts(ora):
    pred = np.array([[[0, 2, 5, -1]]], np.int32)
    exact = np.array([[[2, 3, 5, -1]]], np.int32)
    l2p = np.full((1, 1, 8), -1, np.int32)
    l2p[0, 0, [3, 5, 7]] = [0, 1, 2]
    assert ora.agreement(pred, exact, l2p)[0, 0].tolist() == [3, 2, 2]
    assert ora.agreement(exact, exact)[0, 0].tolist() == [3, 3, -1]
    # recall of the exact list's two best blocks: 2 and 3; only 2 is predicted
    assert ora.agreement(pred, exact, l2p, exact_n=2)[0, 0].tolist() == [2, 1, 1]
