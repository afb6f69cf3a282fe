"""oasis_layer_step_noalloc (the fused step with the library's own device
scratch) against oasis_layer_step with a caller workspace: bit-identical
outputs and maps on two calls in a row, the second with a smaller input (the
scratch then still holds the first call's lists), plus the refusal of a shape
whose lists exceed the scratch."""
import ctypes
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


def cfg_of(batch, dtype="bf16", hq=8, hkv=2, K=128):
    return Config(name="noalloc", dtype=dtype, batch=batch, n_q_heads=hq, n_kv_heads=hkv,
                  head_dim=128, block_size=16, ctx=None, k_resident=K, cap=0.05,
                  draft_sigma=0.2, rho=0.95, planted=0, seed=23)


def one_call(cfg, ctx, seed, step):
    ctx = np.asarray(ctx, np.int32)
    nbmax = cfg.max_blocks(int(ctx.max()))
    shape = lib.Shape.of(cfg, nbmax)
    say(f"no-alloc case: B={cfg.batch} NBmax={nbmax} K={cfg.k_resident} dtype={cfg.dtype} "
        f"lists {lib.layer_step_workspace_bytes(shape)} B")
    qs = gen.query_sequence(cfg, 2, seed=seed, device="cuda")
    q = gen.step_queries(cfg, qs, 1, seed=seed)
    rec = gen.records(cfg, ctx, nbmax, seed=seed, device="cuda")
    state = gen.random_state(cfg, ctx, nbmax, seed, fill=0.8, stamp_max=step)
    a, b = Layer(cfg, ctx, nbmax), Layer(cfg, ctx, nbmax)
    for L in (a, b):
        L.summarize(rec)
        L.set_state(*state)
        L.pool.copy_(pool_from_records(rec, L.p2l))
    m = lib.cap_to_max_admit(cfg.cap, cfg.k_resident)
    a.step(q, step, m)
    lib.layer_step_noalloc(b.shape, q, b.pool, b.summ, b.ctx_len, step, m, b.out, b.topk_idx,
                           b.topk_score, b.l2p, b.p2l, b.last_sel, b.admit, b.admit_count)
    torch.cuda.synchronize()
    for name in OUTPUTS:
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    return lib.layer_step_workspace_bytes(shape)


def test_noalloc_step_equals_workspace_step_twice_then_smaller():
    # long contexts: the scan is split and its lists live in the scratch
    first = one_call(cfg_of(6), [40000, 131072, 17000, 900, 65000, 16385], seed=3, step=4)
    second = one_call(cfg_of(2), [20000, 3000], seed=4, step=5)
    assert first > second > 0
    # one scan part: no scratch used
    assert one_call(cfg_of(3, dtype="f32", K=16), [5000, 100, 0], seed=5, step=2) == 0


def test_noalloc_refuses_lists_above_its_scratch():
    cfg = cfg_of(240, hq=8, hkv=8, K=256)
    shape = lib.Shape.of(cfg, 8192)
    assert lib.layer_step_workspace_bytes(shape) > 32 << 20
    raw = lib.raw()
    st = raw.oasis_layer_step_noalloc(ctypes.byref(shape), *([None] * 4), 0.0, 1, 6,
                                      *([None] * 8), None)
    assert st == lib.ERR_UNSUPPORTED
    assert "scratch" in lib.last_error()
