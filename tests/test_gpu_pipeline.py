"""GPU tests of the multi-layer pipeline: the fused step on the main stream,
the prefetch on a side stream, and the layer-local events between them.

Small-integer inputs make every score exact, so the GPU and the oracle must
agree on every top-K list, map and admission at every step, and attention
(which reads the slots the prefetch filled) must match the oracle's, which
reads the logical blocks directly."""
import numpy as np
import pytest
import torch

import oracle
from parity import check_attention, host, i32
from sparse_kv_block_amd import gen
from sparse_kv_block_amd.configs import Config

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from sparse_kv_block_amd import lib                    # noqa: E402
from sparse_kv_block_amd.pipeline import Decoder, Layer  # noqa: E402


def cfg_small(**kw):
    base = dict(name="pipe", dtype="bf16", batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128,
                block_size=16, ctx=1000, k_resident=16, cap=0.25, draft_sigma=0.2, rho=0.95,
                seed=31)
    base.update(kw)
    return Config(**base)


class OracleLayer:
    """The oracle's own copy of one layer's state."""

    def __init__(self, cfg, rec, ctx, q_cold):
        self.cfg, self.rec, self.ctx = cfg, rec, ctx
        self.summ = oracle.summarize(rec, ctx, 16)
        sc = oracle.block_scores(q_cold, self.summ, ctx, 16, q_row=0)
        idx, _ = oracle.topk(sc, ctx, 16, cfg.k_resident)
        B, H, NB = rec.shape[0], rec.shape[1], rec.shape[2]
        self.l2p = np.full((B, H, NB), -1, np.int32)
        self.p2l = np.full((B, H, cfg.k_resident), -1, np.int32)
        self.ls = np.zeros((B, H, cfg.k_resident), np.int32)
        oracle.capped_evict(idx, 0, cfg.k_resident, self.l2p, self.p2l, self.ls)

    def step(self, q, t, m):
        return oracle.layer_step(q, self.rec, self.summ, self.ctx, 16, self.cfg.k_resident, t, m,
                                 self.l2p, self.p2l, self.ls)


@pytest.mark.parametrize("records_on", ["pinned", "device"])
@pytest.mark.parametrize("delay", [False, True])
def test_decoder_layers_match_oracle(records_on, delay):
    cfg = cfg_small()
    n_layers, n_steps = 3, 4
    ctx = np.array([1000, 700], np.int32)
    nb = cfg.max_blocks()
    rec_cpu, _ = gen.integer_inputs(cfg, ctx, nb, seed=3)
    records = rec_cpu.pin_memory() if records_on == "pinned" else rec_cpu.cuda()
    qs = [gen.integer_queries(cfg, n_steps + 1, seed=100 + i, device="cuda") for i in range(n_layers)]
    dec = Decoder(cfg, ctx, nb, n_layers)
    dec.setup(records, [qs[i][0] for i in range(n_layers)])
    m = lib.cap_to_max_admit(cfg.cap, cfg.k_resident)
    # a long spin on the side stream before every prefetch: if the next step's
    # attention did not wait for the layer's prefetch it would read stale slots
    slow = (lambda i: torch.cuda._sleep(20_000_000)) if delay else None
    got = []
    for t in range(1, n_steps + 1):
        dec.step(records, [qs[i][t] for i in range(n_layers)], t, m, before_prefetch=slow)
        got.append([(L.out.clone(), L.topk_idx.clone(), L.p2l.clone(), L.l2p.clone(),
                     L.last_sel.clone(), L.admit.clone(), L.admit_count.clone()) for L in dec.layers])
    dec.drain()
    torch.cuda.synchronize()
    ora = [OracleLayer(cfg, rec_cpu, ctx, qs[i][0].cpu()) for i in range(n_layers)]
    for t in range(1, n_steps + 1):
        for i in range(n_layers):
            out, idx, _, admit, count = ora[i].step(qs[i][t].cpu(), t, m)
            g = got[t - 1][i]
            what = f"step {t} layer {i}"
            check_attention(g[0], out, "bf16", what)
            np.testing.assert_array_equal(i32(g[1]), idx, err_msg=what)
            np.testing.assert_array_equal(i32(g[2]), ora[i].p2l, err_msg=what)
            np.testing.assert_array_equal(i32(g[3]), ora[i].l2p, err_msg=what)
            np.testing.assert_array_equal(i32(g[4]), ora[i].ls, err_msg=what)
            np.testing.assert_array_equal(i32(g[5]), admit, err_msg=what)
            np.testing.assert_array_equal(i32(g[6]), count, err_msg=what)
            assert int(count.sum()) > 0, "the inputs should force admissions"


@pytest.mark.parametrize("records_on", ["pinned", "device"])
def test_decoder_append_between_pipelined_steps(records_on):
    # a token per request is appended to the layer after every step, while the
    # step's prefetch (delayed on the side stream) may still be filling slots
    cfg = cfg_small(batch=3)
    n_steps = 5
    ctx = np.array([1000, 31, 700], np.int32)        # the second crosses into a new block
    nb = cfg.max_blocks() + 1
    rec_cpu, _ = gen.integer_inputs(cfg, ctx, nb, seed=5)
    records = rec_cpu.pin_memory() if records_on == "pinned" else rec_cpu.cuda()
    qs = gen.integer_queries(cfg, n_steps + 1, seed=77, device="cuda")
    kn, vn = gen.new_tokens(cfg, n_steps, seed=78, device="cuda", integer=True)
    dec = Decoder(cfg, ctx, nb, 1)
    dec.setup(records, [qs[0]])
    m = lib.cap_to_max_admit(cfg.cap, cfg.k_resident)
    slow = lambda i: torch.cuda._sleep(20_000_000)      # noqa: E731
    got = []
    for t in range(1, n_steps + 1):
        dec.step(records, [qs[t]], t, m, before_prefetch=slow)
        L = dec.layers[0]
        got.append((L.out.clone(), L.topk_idx.clone(), L.p2l.clone(), L.admit.clone()))
        dec.append(0, records, kn[t - 1], vn[t - 1])
    dec.drain()
    torch.cuda.synchronize()
    ora = OracleLayer(cfg, rec_cpu.clone(), ctx.copy(), qs[0].cpu())
    rec_np = oracle.as_np(ora.rec)
    for t in range(1, n_steps + 1):
        out, idx, _, admit, count = ora.step(qs[t].cpu(), t, m)
        what = f"step {t}"
        check_attention(got[t - 1][0], out, "bf16", what)
        np.testing.assert_array_equal(i32(got[t - 1][1]), idx, err_msg=what)
        np.testing.assert_array_equal(i32(got[t - 1][2]), ora.p2l, err_msg=what)
        np.testing.assert_array_equal(i32(got[t - 1][3]), admit, err_msg=what)
        oracle.append(kn[t - 1].cpu(), vn[t - 1].cpu(), rec_np, ora.summ, ora.ctx, 16)
    L = dec.layers[0]
    np.testing.assert_array_equal(i32(L.ctx_len), ora.ctx)
    assert np.array_equal(host(records), rec_np)
    np.testing.assert_array_equal(oracle.to_f64(host(L.summ)), oracle.to_f64(ora.summ))
    p2l = i32(L.p2l).astype(np.int64)
    pool = host(L.pool)
    b, h, s = np.nonzero(p2l >= 0)
    assert np.array_equal(pool[b, h, s], rec_np[b, h, p2l[b, h, s]]), "resident copies"


def test_memcpy_mode_pipeline():
    cfg = cfg_small()
    ctx = np.array([1000, 333], np.int32)
    nb = cfg.max_blocks()
    rec_cpu, _ = gen.integer_inputs(cfg, ctx, nb, seed=4)
    records = rec_cpu.pin_memory()
    qs = gen.integer_queries(cfg, 4, seed=7, device="cuda")
    dec = Decoder(cfg, ctx, nb, 2)
    dec.setup(records, [qs[0], qs[0]])
    ora = [OracleLayer(cfg, rec_cpu, ctx, qs[0].cpu()) for _ in range(2)]
    m = lib.cap_to_max_admit(cfg.cap, cfg.k_resident)
    for t in range(1, 4):
        dec.step(records, [qs[t], qs[t]], t, m, mode=lib.MEMCPY)
        outs = [L.out.clone() for L in dec.layers]
        torch.cuda.synchronize()
        for i in range(2):
            out, idx, _, admit, count = ora[i].step(qs[t].cpu(), t, m)
            check_attention(outs[i], out, "bf16", f"step {t} layer {i}")
            np.testing.assert_array_equal(i32(dec.layers[i].p2l), ora[i].p2l)


def test_snapshot_replay_is_bit_identical():
    cfg = cfg_small(batch=3)
    ctx = np.array([1000, 600, 160], np.int32)
    nb = cfg.max_blocks()
    qseq = gen.query_sequence(cfg, 8, device="cuda")
    rec = gen.records(cfg, ctx, nb, device="cuda")
    layer = Layer(cfg, ctx, nb)
    layer.summarize(rec)
    layer.cold_fill(gen.step_queries(cfg, qseq, 1), rec)
    for t in (1, 2):
        layer.step(gen.step_queries(cfg, qseq, t), t)
        layer.prefetch(rec)
    snap = [x.clone() for x in layer.state()] + [layer.pool.clone()]

    def run():
        res = []
        for t in (3, 4, 5):
            layer.step(gen.step_queries(cfg, qseq, t), t)
            layer.prefetch(rec)
            res.append([x.clone() for x in (layer.out, layer.topk_idx, layer.topk_score,
                                            layer.p2l, layer.l2p, layer.last_sel, layer.admit)])
        return res

    first = run()
    layer.set_state(*snap[:3])
    layer.pool.copy_(snap[3])
    second = run()
    torch.cuda.synchronize()
    for a, b in zip(first, second):
        for x, y in zip(a, b):
            assert torch.equal(x, y)


@pytest.mark.parametrize("m", [0, 16])
def test_cap_extremes(m):
    # m = 0: only stamps change; m = K: the whole top-K becomes resident
    cfg = cfg_small()
    ctx = np.array([1000, 700], np.int32)
    nb = cfg.max_blocks()
    rec, q = gen.integer_inputs(cfg, ctx, nb, seed=9, device="cuda")
    layer = Layer(cfg, ctx, nb)
    layer.summarize(rec)
    state = gen.random_state(cfg, ctx, nb, 9, fill=1.0, stamp_max=3)
    layer.set_state(*state)
    layer.step(q, 5, m)
    torch.cuda.synchronize()
    if m == 0:
        assert torch.equal(layer.p2l.cpu(), state[1]) and torch.equal(layer.l2p.cpu(), state[0])
        assert int(layer.admit_count.sum()) == 0
    else:
        for b in range(cfg.batch):
            for h in range(cfg.n_kv_heads):
                T = set(layer.topk_idx[b, h].tolist()) - {-1}
                assert T <= set(layer.p2l[b, h].tolist())
