"""Full-size parity of the 36-layer decode step with the fetch-cap sweep:
batch 128 at 16K context, 32 query / 8 KV heads, d = 128, K = 128, every cap
of the sweep (0.01, 0.05, 0.2, 1.0), in the launch configuration the bench
times: per layer the fused step on the main stream, the gather prefetch of its
admissions from one pinned host pool on a side stream, layer-local events.

Layers 0, 17 and 35 are checked in full: every unit of each is carried by an
oracle twin (`parity.OracleTwin`) through the cold fill and two decode steps
per cap.  Attention reads the slots the previous step's prefetch filled (from
the host pool over the host link), the oracle reads the logical blocks, so
attention parity also checks the prefetch; after the last step of each cap
every resident slot of those layers is compared with its block.  Top-K lists
must agree within the tolerance at the K-th score; maps, stamps and
admissions bit for bit on every unit at every step.  Every unit of every
layer is checked for the map invariants after each step."""
import sys

import numpy as np
import pytest
import torch

import oracle
from parity import OracleTwin, host, i32
from sparse_kv_block_amd import gen
from sparse_kv_block_amd.configs import FULL_36

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from sparse_kv_block_amd import lib                    # noqa: E402  (fails loudly if not built)
from sparse_kv_block_amd.pipeline import Decoder, Layer  # noqa: E402

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def layer_seed(cfg, l):
    return 1000 * 4 + l


@pytest.mark.timeout(1200)
def test_full_size_36_layer_pipeline_cap_sweep():
    cfg = FULL_36
    L, K = cfg.layers, cfg.k_resident
    ctx = gen.context_lengths(cfg)
    nbmax = cfg.max_blocks()
    steps = 2
    check_layers = (0, L // 2 - 1, L - 1)
    say(f"full 36-layer: every unit of layers {check_layers}")

    # queries per layer: q[1..steps+1] with AR(1) drift, own seed per layer
    qs = []
    for l in range(L):
        seq = gen.query_sequence(cfg, steps + 2, seed=layer_seed(cfg, l), device=DEV)
        qs.append([None] + [gen.step_queries(cfg, seq, t, seed=layer_seed(cfg, l))
                            for t in range(1, steps + 2)])
        if l == 0:
            dirs = gen.planted_directions(cfg, seq[1])
    rec_dev = gen.records(cfg, ctx, nbmax, device=DEV, planted_dir=dirs)
    src = Layer(cfg, ctx, nbmax)
    src.summarize(rec_dev)
    rec_host = torch.empty(rec_dev.shape, dtype=rec_dev.dtype, pin_memory=True)
    rec_host.copy_(rec_dev)
    del rec_dev
    torch.cuda.synchronize()
    rec_np = oracle.as_np(rec_host)
    summ = oracle.summarize(rec_np, ctx, 16)
    OracleTwin(cfg, rec_np, ctx, summ=summ).check_summaries(src, "36-layer summaries")
    say("summaries of every unit match")

    dec = Decoder(cfg, ctx, nbmax, L, device=DEV)
    differ, exposed, unit_steps = 0, 0, 0
    for cap in cfg.caps_sweep:
        m = lib.cap_to_max_admit(cap, K)
        say(f"cap {cap} (m={m}): setup")
        dec.setup(rec_host, [qs[l][1] for l in range(L)], summ_from=src)
        torch.cuda.synchronize()
        twins = {}
        for l in check_layers:
            twins[l] = OracleTwin(cfg, rec_np, ctx, summ=summ)
            twins[l].cold_fill(dec.layers[l], qs[l][1].cpu(), f"cap {cap} layer {l}")
        for t in range(1, steps + 1):
            say(f"cap {cap} (m={m}): step {t}")
            dec.step(rec_host, [qs[l][t] for l in range(L)], t, m)
            dec.drain()
            torch.cuda.synchronize()
            for l in range(L):
                check_map_invariants(dec.layers[l], m, t, f"cap {cap} step {t} layer {l}")
            for l in check_layers:
                _, count = twins[l].step(dec.layers[l], qs[l][t].cpu(), t, m, f"cap {cap} layer {l}")
                assert int(count.max()) <= m
            say(f"cap {cap} (m={m}): step {t}: every unit of layers {check_layers} matches")
        for l in check_layers:
            layer = dec.layers[l]
            p2l = host(layer.p2l).astype(np.int64)
            pool = host(layer.pool)
            b, h, s = np.nonzero(p2l >= 0)
            assert np.array_equal(pool[b, h, s], rec_np[b, h, p2l[b, h, s]]), \
                f"cap {cap} layer {l}: resident copies"
            differ += len(twins[l].differ)
            exposed += twins[l].exposed
            unit_steps += twins[l].unit_steps
        torch.cuda.synchronize()
    say(f"{unit_steps} unit-steps compared in full, {differ} top-K lists differed, each only "
        f"between blocks within the fp32 rounding scale of each other (bound: {exposed} "
        f"unit-steps with such a near-tie)")
    assert differ <= exposed


def check_map_invariants(layer, m, t, what):
    """Every unit of a layer: the slot map and the block map are inverse to each
    other with no block held twice, at most m admissions, every admission's
    slot holds its block and is stamped with the step, and every resident
    member of the top-K list is stamped with the step."""
    p2l = i32(layer.p2l)                                       # [B][H][K]
    l2p = i32(layer.l2p)                                       # [B][H][NB]
    ls = i32(layer.last_sel)
    B, H, K = p2l.shape
    bb, hh, ss = np.nonzero(p2l >= 0)
    jj = p2l[bb, hh, ss]
    assert np.array_equal(l2p[bb, hh, jj], ss), what
    assert int((l2p >= 0).sum()) == len(jj), what             # no block mapped twice
    cnt = i32(layer.admit_count)
    assert cnt.min() >= 0 and cnt.max() <= m, what
    adm = i32(layer.admit)                                     # [B][H][K][3]
    for b, h in zip(*np.nonzero(cnt)):
        a = adm[b, h, :cnt[b, h]]
        assert np.array_equal(p2l[b, h, a[:, 1]], a[:, 0]), what
        assert np.all(ls[b, h, a[:, 1]] == t), what
    top = i32(layer.topk_idx)                                  # [B][H][K]
    tb, th, tk = np.nonzero(top >= 0)
    slot = l2p[tb, th, top[tb, th, tk]]
    res = slot >= 0
    assert np.all(ls[tb[res], th[res], slot[res]] == t), what
