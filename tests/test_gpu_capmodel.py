"""The host-link / fetch-cap budget on the GPU at a reduced size: a 4-layer
pipelined decode step (fused step on the main stream, gather prefetch from a
pinned host pool on a side stream, layer-local events) swept over fetch caps,
as the 36-layer bench leg runs it (agihunt.info summary, fetch-cap ablation;
pith.science paper page, "Assumptions & free parameters": the overlap window).

Checks: the bytes moved per step are the admission counts times the record
size; where the cap saturates (every unit finds at least max_admit misses,
forced here by independent queries at every step) they equal
layers * units * max_admit * record_bytes, never more; the cap rule is the
library's; the model's predicted step is never below its window; the measured
overlap fraction lies in [0, 1]; the pipelined step's resident sets are valid."""
import numpy as np
import pytest
import torch

from sparse_kv_block_amd import capmodel as cm
from sparse_kv_block_amd import gen
from sparse_kv_block_amd.configs import Config

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from sparse_kv_block_amd import lib                                  # noqa: E402
from sparse_kv_block_amd.pipeline import Decoder, time_cap_sweep      # noqa: E402


def test_cap_sweep_bytes_and_model_at_reduced_size():
    cfg = Config(name="capmodel_small", dtype="bf16", batch=8, n_q_heads=8, n_kv_heads=2,
                 head_dim=128, block_size=16, ctx=4000, k_resident=16, cap=0.125,
                 draft_sigma=0.2, rho=0.0, seed=41)
    L, steps, warmup = 4, 3, 1
    caps = (0.0625, 0.125, 0.25, 1.0)
    ctx = gen.context_lengths(cfg)
    nbmax = cfg.max_blocks()
    rec_host = gen.records(cfg, ctx, nbmax).pin_memory()
    qs = []
    for l in range(L):
        # independent queries at every step (rho 0): the top-K moves, so small
        # caps saturate
        seq = gen.query_sequence(cfg, warmup + steps + 3, seed=500 + l, device="cuda")
        qs.append([None] + [gen.step_queries(cfg, seq, t, seed=500 + l)
                            for t in range(1, warmup + steps + 2)])
    dec = Decoder(cfg, ctx, nbmax, L)
    dec.layers[0].summarize(rec_host)
    torch.cuda.synchronize()
    rows = time_cap_sweep(dec, rec_host, qs, caps, steps, warmup, summ_from=dec.layers[0])
    units = cfg.batch * cfg.n_kv_heads
    rec_bytes = lib.record_bytes(dec.layers[0].shape)
    assert rec_bytes == 2 * 16 * 128 * 2
    for row in rows:
        m = row["max_admit"]
        assert m == lib.cap_to_max_admit(row["cap"], cfg.k_resident)
        assert row["bytes_bound"] == cm.bytes_per_step(L, units, m, rec_bytes)
        assert 0 <= row["bytes_per_step"] <= row["bytes_bound"]
        if m <= 2:
            assert row["bytes_per_step"] == row["bytes_bound"], row     # saturated
        assert row["step_ms"] > 0 and row["compute_only_ms"] > 0
        window = row["compute_only_ms"] / 1e3                      # the layers' fused steps
        bw = max(row["host_link_GBps"], 1e-3) * 1e9
        assert cm.predicted_step_s(window, row["bytes_per_step"], bw) >= window
        f = cm.overlap_fraction(row["step_ms"] / 1e3, row["compute_only_ms"] / 1e3,
                                row["bytes_per_step"] / bw)
        assert 0.0 <= f <= 1.0
        print(row, "overlap", round(f, 3), flush=True)
    # the last sweep's state: every layer's maps are mutual inverses
    for layer in dec.layers:
        p2l = layer.p2l.cpu().numpy()
        l2p = layer.l2p.cpu().numpy()
        b, h, s = np.nonzero(p2l >= 0)
        assert np.array_equal(l2p[b, h, p2l[b, h, s]], s)
        assert int((l2p >= 0).sum()) == len(s)
