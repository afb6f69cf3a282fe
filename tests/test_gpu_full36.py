"""Full-size parity of the 36-layer decode step with the fetch-cap sweep:
batch 128 at 16K context, 32 query / 8 KV heads, d = 128, K = 128, every cap
of the sweep (0.01, 0.05, 0.2, 1.0), in the launch configuration the bench
times: per layer the fused step on the main stream, the gather prefetch of its
admissions from one pinned host pool on a side stream, layer-local events.

Sampled (request, KV head) units of three layers are carried by the oracle,
each as its own one-unit problem, through the cold fill and two decode steps
per cap.  Attention reads the slots the previous step's prefetch filled (from
the host pool over the host link), the oracle reads the logical blocks, so
attention parity also checks the prefetch.  Top-K lists must agree within the
tolerance at the K-th score; maps, stamps and admissions bit for bit on every
unit whose list agrees (a unit whose list differs inside the tolerance is set
back to the oracle's state before the next step).  Every unit of every layer
is checked for the map invariants after each step."""
import sys

import numpy as np
import pytest
import torch

import oracle
from parity import check_attention, check_topk, host, i32, pool_from_records, sample_units, unit_slice
from sparse_kv_block_amd import gen
from sparse_kv_block_amd.configs import FULL_36

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from sparse_kv_block_amd import lib                    # noqa: E402,F401  (fails loudly if not built)
from sparse_kv_block_amd.pipeline import Decoder, Layer  # noqa: E402

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def layer_seed(cfg, l):
    return 1000 * 4 + l


def test_full_size_36_layer_pipeline_cap_sweep():
    cfg = FULL_36
    L, G, K = cfg.layers, cfg.group, cfg.k_resident
    ctx = gen.context_lengths(cfg)
    nbmax = cfg.max_blocks()
    steps = 2
    check_layers = (0, L // 2 - 1, L - 1)
    units = sample_units(cfg.batch, cfg.n_kv_heads, 3, cfg.seed)
    say(f"full 36-layer: layers {check_layers}, units {units}")

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
    # the sampled units' records stay on the device (for resyncs) and on the host (oracle)
    u_dev = {u: unit_slice(rec_dev, u[0], u[1], G, "unit").clone() for u in units}
    u_cpu = {u: x.cpu() for u, x in u_dev.items()}
    u_ctx = {u: unit_slice(ctx, u[0], u[1], G, "ctx") for u in units}
    u_summ = {u: oracle.summarize(u_cpu[u], u_ctx[u], 16) for u in units}
    del rec_dev
    torch.cuda.synchronize()

    dec = Decoder(cfg, ctx, nbmax, L, device=DEV)
    resyncs = 0
    for cap in cfg.caps_sweep:
        m = cfg.max_admit(cap)
        say(f"cap {cap} (m={m}): setup")
        dec.setup(rec_host, [qs[l][1] for l in range(L)], summ_from=src)
        torch.cuda.synchronize()
        ora = {}
        for l in check_layers:
            layer = dec.layers[l]
            for (b, h) in units:
                u = (b, h)
                sl = (slice(b, b + 1), slice(h, h + 1))
                qq = unit_slice(qs[l][1], b, h, G, "q").cpu()
                sc = oracle.block_scores(qq, u_summ[u], u_ctx[u], 16, q_row=0)
                idx, _ = oracle.topk(sc, u_ctx[u], 16, K)
                o = dict(l2p=np.full((1, 1, nbmax), -1, np.int32),
                         p2l=np.full((1, 1, K), -1, np.int32), ls=np.zeros((1, 1, K), np.int32))
                oracle.capped_evict(idx, 0, K, o["l2p"], o["p2l"], o["ls"])
                ora[(l, u)] = o
                if not (np.array_equal(i32(layer.p2l[sl]), o["p2l"]) and
                        np.array_equal(i32(layer.l2p[sl]), o["l2p"])):
                    resyncs += 1
                    set_unit(layer, sl, o, u_dev[u])
        torch.cuda.synchronize()
        for t in range(1, steps + 1):
            say(f"cap {cap} (m={m}): step {t}")
            dec.step(rec_host, [qs[l][t] for l in range(L)], t, m)
            dec.drain()
            torch.cuda.synchronize()
            for l in range(L):
                check_map_invariants(dec.layers[l], m, t, f"cap {cap} step {t} layer {l}")
            for l in check_layers:
                layer = dec.layers[l]
                for (b, h) in units:
                    u = (b, h)
                    o = ora[(l, u)]
                    sl = (slice(b, b + 1), slice(h, h + 1))
                    qq = unit_slice(qs[l][t], b, h, G, "q").cpu()
                    out, idx, _, admit, count = oracle.layer_step(
                        qq, u_cpu[u], u_summ[u], u_ctx[u], 16, K, t, m, o["l2p"], o["p2l"], o["ls"])
                    what = f"cap {cap} step {t} layer {l} unit {u}"
                    check_attention(layer.out[b:b + 1, :, h * G:(h + 1) * G], out, cfg.dtype, what)
                    sc = oracle.block_scores(qq, u_summ[u], u_ctx[u], 16)
                    differ = check_topk(i32(layer.topk_idx[sl]), host(layer.topk_score[sl]), idx, sc,
                                        what=what)
                    if differ == 0:
                        np.testing.assert_array_equal(i32(layer.l2p[sl]), o["l2p"], err_msg=what)
                        np.testing.assert_array_equal(i32(layer.p2l[sl]), o["p2l"], err_msg=what)
                        np.testing.assert_array_equal(i32(layer.last_sel[sl]), o["ls"], err_msg=what)
                        np.testing.assert_array_equal(i32(layer.admit[sl]), admit, err_msg=what)
                        np.testing.assert_array_equal(i32(layer.admit_count[sl]), count, err_msg=what)
                        assert int(count.max()) <= m
                        # the slots the side stream filled hold the admitted blocks
                        for k in range(int(count[0, 0])):
                            j, s = int(admit[0, 0, k, 0]), int(admit[0, 0, k, 1])
                            assert torch.equal(layer.pool[b, h, s], u_dev[u][0, 0, j]), what
                    else:
                        resyncs += 1
                        set_unit(layer, sl, o, u_dev[u])
            torch.cuda.synchronize()
    say(f"resyncs {resyncs}")


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


def set_unit(layer, sl, o, rec_unit):
    """Puts the oracle's state of one unit (maps, stamps, resident copies) on the GPU."""
    layer.l2p[sl] = torch.from_numpy(o["l2p"]).to(DEV)
    layer.p2l[sl] = torch.from_numpy(o["p2l"]).to(DEV)
    layer.last_sel[sl] = torch.from_numpy(o["ls"]).to(DEV)
    layer.pool[sl] = pool_from_records(rec_unit, layer.p2l[sl])
