"""Benchmark of the fused look-ahead layer step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config qwen3_8b_16k]

Workload: the Qwen3-8B-shaped layer (batch 128, 32 query / 8 KV heads,
head_dim 128, 16K context, K = 128 resident 16-token blocks, cap 0.05, bf16),
synthetic seeded inputs.  One step = one look-ahead layer step for the whole
batch: attention of the normal and draft rows over the resident sets, the
draft summary scan, top-K and capped eviction (one fused kernel), with the
queries drifting AR(1) from step to step and the resident sets carried.  The
prefetch of the admitted blocks crosses the host link and is timed in its own
leg (`pcie`), never in `value`.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
COUNTERS_WORKLOAD = "qwen3_8b_16k"
COUNTERS_FILE = os.path.join(ROOT, "profiles", f"layer_step_{COUNTERS_WORKLOAD}_counters.json")


def kernel_name(cfg) -> str:
    tiles = 1 if 2 * cfg.group <= 16 else 2
    return (f"layer_step_kernel<{cfg.dtype}, d={cfg.head_dim}, {tiles} row tile"
            f"{'s' if tiles > 1 else ''}>")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(cfg, ctx: np.ndarray) -> dict:
    """Bytes the fused step must move per launch (one layer, whole batch)."""
    from sparse_kv_block_amd import lib
    B, H, K, d, Hq = cfg.batch, cfg.n_kv_heads, cfg.k_resident, cfg.head_dim, cfg.n_q_heads
    es = cfg.esize
    S = cfg.block_size
    nb = np.minimum(-(-ctx.astype(np.int64) // S), cfg.max_blocks(int(ctx.max())))
    m = lib.cap_to_max_admit(cfg.cap, cfg.k_resident)
    kv = B * H * K * 2 * S * d * es                       # resident records (keys + values)
    summ = int(H * nb.sum()) * 2 * d * es                  # min/max rows of every block
    q_out = 2 * (B * 2 * Hq * d * es)                      # queries read, outputs written
    maps = B * H * (K * 4 * 2          # p2l read + write
                    + K * 4 * 2        # last_sel read + write
                    + 2 * m * 4        # l2p updates (residency comes from p2l)
                    + K * 8            # top-K index + score written
                    + K * 12 + 4)      # admission list + count written
    return dict(kv=kv, summaries=summ, q_out=q_out, maps=maps,
                total=kv + summ + q_out + maps + B * 4)


def traffic_from_profile(cfg):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they
    were taken on this workload and the current kernel sources."""
    if cfg.name != COUNTERS_WORKLOAD:
        return None
    try:
        rec = json.load(open(COUNTERS_FILE))
    except (OSError, ValueError):
        return None
    from sparse_kv_block_amd.profiling import kernel_source_hash
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, ctx, records_host, qs_host, min_cpu_seconds: float):
    """The fp64 oracle (as it stands) on the same step: whole layer steps over
    all units, repeated until about `min_cpu_seconds` of CPU time is spent."""
    import oracle
    from sparse_kv_block_amd import gen
    B, H = cfg.batch, cfg.n_kv_heads
    nb = cfg.max_blocks(int(ctx.max()))
    rec = oracle.as_np(records_host)
    nth = oracle.default_threads()
    summ = oracle.summarize(rec, ctx, cfg.block_size, nthreads=nth)
    state = [x.numpy().copy() for x in gen.random_state(cfg, ctx, nb, 77, stamp_max=1)]
    q = oracle.as_np(qs_host)
    reps, spent = 0, 0.0
    while spent * nth < min_cpu_seconds or reps == 0:
        l2p, p2l, ls = [x.copy() for x in state]
        t0 = time.perf_counter()
        oracle.layer_step(q, rec, summ, ctx, cfg.block_size, cfg.k_resident, 1,
                          oracle.max_admit(cfg.cap, cfg.k_resident),
                          l2p, p2l, ls, nthreads=nth)
        spent += time.perf_counter() - t0
        reps += 1
    # one thread on a slice of the units (the same work per unit), scaled to a
    # whole layer step
    n1 = min(B * H, 64)
    units = np.arange(n1, dtype=np.int32)
    l2p, p2l, ls = [x.copy() for x in state]
    t0 = time.perf_counter()
    oracle.layer_step(q, rec, summ, ctx, cfg.block_size, cfg.k_resident, 1,
                      oracle.max_admit(cfg.cap, cfg.k_resident),
                      l2p, p2l, ls, units=units, nthreads=1)
    t1 = (time.perf_counter() - t0) * (B * H) / n1
    return {"value": reps / spent, "unit": "layer-steps/s", "cores": min(nth, B * H),
            "kind": "oracle",
            "sample": f"{reps} whole layer steps ({B * H} units each: attention, scan, top-K, "
                      f"eviction) in {spent:.2f} s wall on {nth} threads",
            "single_thread": {"value": round(1.0 / t1, 4), "unit": "layer-steps/s",
                              "sample": f"{n1} of {B * H} units on one thread, scaled"},
            "cpu_model": cpu_model()}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def dense_leg(cfg, layer, rec, q, reps: int = 10):
    """The dense comparator on the same layer: attention of both rows over the
    full KV held in HBM (`rec`, the device copy of the records; the capacity
    the method avoids needing)."""
    import torch
    from sparse_kv_block_amd import lib
    ws = lib.dense_attn_workspace(layer.shape)
    out = torch.empty_like(layer.out)
    for _ in range(2):
        lib.dense_attn(layer.shape, q, rec, layer.ctx_len, out, ws)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        lib.dense_attn(layer.shape, q, rec, layer.ctx_len, out, ws)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps
    kv = rec.numel() * rec.element_size()
    log(f"[bench] dense attention over {kv / 2**30:.1f} GiB of KV: {us:.1f} us, {kv / us / 1e3:.0f} GB/s")
    return {"us": round(us, 2), "kv_bytes": kv, "GBps": round(kv / us / 1e3, 1),
            "hbm_kv_per_layer_GiB": round(kv / 2**30, 2)}


def achievable_leg(mib: int, reps: int = 10) -> dict:
    """What a plain streaming kernel reaches on this GPU, beside the step: a
    device-to-device copy of `mib` MiB (the runtime's copy kernel; it reads and
    writes the bytes once each), timed with HIP events, median of `reps`."""
    import torch
    n = mib * 2**20 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    dst.copy_(src)
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dst.copy_(src)
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) / 1e3)
    s = float(np.median(ts))
    moved = 2 * n * 4
    del src, dst
    log(f"[bench] achievable: {mib} MiB device copy {moved / s / 1e9:.0f} GB/s (read + write)")
    return {"copy_GBps": round(moved / s / 1e9, 1), "copy_bytes": moved,
            "kind": f"device-to-device copy of {mib} MiB (bytes read + written per second)"}


def kernels_leg(cfg, layer, ctx, nbmax, qs, rec, reps: int = 10):
    """Each standalone kernel of the step on the timed layer's state, timed
    with HIP events on the current stream (median of `reps`), against its
    algorithmic bytes: summarize (reads every key of the full KV, here the
    device-resident copy `rec`), look-ahead attention (the resident pool),
    summary scan + top-K (the summaries), capped eviction (maps only)."""
    import torch
    from sparse_kv_block_amd import gen, lib
    stream = torch.cuda.current_stream()
    sh = layer.shape
    es = 2 if cfg.dtype == "bf16" else 4
    units = cfg.batch * cfg.n_kv_heads
    nb = np.minimum((ctx.astype(np.int64) + 15) // 16, nbmax)
    sum_blocks = int(nb.sum()) * cfg.n_kv_heads

    def timed(fn, restore=None):
        fn()
        ts = []
        for _ in range(reps):
            if restore:
                restore()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e3)
        return float(np.median(ts))

    torch.cuda.synchronize()
    time.sleep(1.0)                 # earlier legs may have freed large buffers
    out = {}
    summ = torch.empty_like(layer.summ)
    us = timed(lambda: lib.summarize(sh, rec, layer.ctx_len, summ))
    byt = sum_blocks * (16 * cfg.head_dim * es + 2 * cfg.head_dim * es)
    out["summarize"] = {"us": round(us, 1), "bytes": byt, "GBps": round(byt / us / 1e3, 1)}
    del summ
    q = qs[0]
    us = timed(lambda: lib.lookahead_attn(sh, q, layer.pool, layer.p2l, layer.ctx_len, layer.out))
    byt = units * cfg.k_resident * 2 * 16 * cfg.head_dim * es + 2 * q.numel() * es
    out["lookahead_attn"] = {"us": round(us, 1), "bytes": byt, "GBps": round(byt / us / 1e3, 1)}
    us = timed(lambda: lib.score_topk(sh, q, layer.summ, layer.ctx_len, layer.topk_idx,
                                      layer.topk_score, q_row=1, workspace=layer.workspace))
    byt = sum_blocks * 2 * cfg.head_dim * es + q.numel() * es // 2 + units * cfg.k_resident * 8
    out["score_topk"] = {"us": round(us, 1), "bytes": byt, "GBps": round(byt / us / 1e3, 1)}
    saved = layer.state()
    m = lib.cap_to_max_admit(cfg.cap, cfg.k_resident)

    def restore():
        layer.set_state(*saved)

    us = timed(lambda: lib.capped_evict(sh, layer.topk_idx, 10**6, m, layer.l2p, layer.p2l,
                                        layer.last_sel, layer.admit, layer.admit_count),
               restore=restore)
    restore()
    out["capped_evict"] = {"us": round(us, 1)}
    log(f"[bench] kernels: " + ", ".join(f"{k} {v['us']} us" + (f" ({v['GBps']} GB/s)" if 'GBps' in v else "")
                                         for k, v in out.items()))
    return out


def append_leg(layer, rec_host, reps: int = 8):
    """Decode append of one token per request into the pinned host records
    (written over the host link), the resident copies and the summaries."""
    import torch
    from sparse_kv_block_amd import gen
    cfg = layer.cfg
    kn, vn = gen.new_tokens(cfg, reps + 1, seed=77, device=layer.device)
    stream = torch.cuda.current_stream()
    layer.append(rec_host, kn[0], vn[0])                       # warm-up
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for i in range(reps):
        ev[i][0].record(stream)
        layer.append(rec_host, kn[i + 1], vn[i + 1])
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    us = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3
    es = 2 if cfg.dtype == "bf16" else 4
    units = cfg.batch * cfg.n_kv_heads
    res = {"us": round(us, 2), "records": "pinned host (host-mapped)",
           "host_link_bytes": units * 2 * cfg.head_dim * es,
           "hbm_bytes_summaries": units * 2 * 2 * cfg.head_dim * es}
    log(f"[bench] append: {us:.1f} us per token step ({units} units)")
    return res


def agreement_leg(cfg, ctx, nbmax, steps: int, caps, sigmas):
    """Top-K agreement study on device-resident records (see
    sparse_kv_block_amd.diagnostics): by fetch cap at the workload's draft
    noise, and by draft noise at the workload's cap.  Also times one exact
    top-K launch (the scan of every key of the batch)."""
    import torch
    from sparse_kv_block_amd import gen, lib
    from sparse_kv_block_amd.diagnostics import run_study
    from sparse_kv_block_amd.pipeline import Layer
    dev = "cuda"
    qseq = gen.query_sequence(cfg, steps + 3, device=dev)
    dirs = gen.planted_directions(cfg, qseq[1]) if cfg.planted else None
    rec = gen.records(cfg, ctx, nbmax, device=dev, planted_dir=dirs)
    out = {"steps": steps, "draft_sigma": cfg.draft_sigma, "cap": cfg.cap, "by_cap": {},
           "by_sigma": {}}

    def one(c, cap):
        qs = [None] + [gen.step_queries(c, qseq, s) for s in range(1, steps + 2)]
        layer = Layer(c, ctx, nbmax, device=dev)
        layer.summarize(rec)
        layer.cold_fill(qs[1], rec)
        res = run_study(layer, rec, qs, steps, max_admit=lib.cap_to_max_admit(cap, c.k_resident))
        del layer
        return res, qs

    for cap in caps:
        out["by_cap"][str(cap)], qs = one(cfg, cap)
        log(f"[bench] agreement cap {cap}: {out['by_cap'][str(cap)]}")
    for sg in sigmas:
        out["by_sigma"][str(sg)], _ = one(cfg.scaled(draft_sigma=sg), cfg.cap)
        log(f"[bench] agreement sigma {sg}: {out['by_sigma'][str(sg)]}")
    # exact top-K timing
    shape = lib.Shape.of(cfg, nbmax)
    ctx_d = torch.from_numpy(ctx).to(dev)
    K = cfg.k_resident
    idx = torch.empty((cfg.batch, cfg.n_kv_heads, K), dtype=torch.int32, device=dev)
    sc = torch.empty((cfg.batch, cfg.n_kv_heads, K), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    lib.exact_topk(shape, qs[1], rec, ctx_d, idx, sc, q_row=1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(5)]
    for a, b in ev:
        a.record(stream)
        lib.exact_topk(shape, qs[1], rec, ctx_d, idx, sc, q_row=1)
        b.record(stream)
    torch.cuda.synchronize()
    us = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3
    es = 2 if cfg.dtype == "bf16" else 4
    nb = np.minimum((ctx.astype(np.int64) + 15) // 16, nbmax)
    key_bytes = int(nb.sum()) * cfg.n_kv_heads * 16 * cfg.head_dim * es
    out["exact_topk"] = {"us": round(us, 1), "key_bytes": key_bytes,
                         "GBps": round(key_bytes / (us * 1e-6) / 1e9, 1)}
    log(f"[bench] exact top-K: {us:.1f} us over {key_bytes / 2**30:.2f} GiB of keys")
    del rec
    torch.cuda.empty_cache()
    return out


def capmodel_leg(cfg, layer, rec_host, ctx, nbmax, qs, t_layer_s: float, gather: dict,
                 pipeline: dict = None, layers: int = 36, caps=(0.01, 0.05, 0.2, 1.0)):
    """Host-link budget (sparse_kv_block_amd.capmodel): measured link rates
    (the gather kernel's, and one large SDMA copy from the pinned pool),
    measured fused-step times at K and at the smaller K/2, the largest cap
    whose bytes hide in a `layers`-layer decode step, and the predicted step
    times beside the measured 36-layer pipeline when it ran."""
    import torch
    from sparse_kv_block_amd import capmodel as cm
    from sparse_kv_block_amd import lib
    from sparse_kv_block_amd.pipeline import Layer
    dev = layer.device
    stream = torch.cuda.current_stream()
    # SDMA: one contiguous 1 GiB host-to-device copy from the pinned pool
    flat = rec_host.view(-1)
    n = min(flat.numel(), (1 << 30) // flat.element_size())
    dst = torch.empty(n, dtype=flat.dtype, device=dev)
    dst.copy_(flat[:n], non_blocking=True)
    ts = []
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dst.copy_(flat[:n], non_blocking=True)
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) / 1e3)
    sdma_Bps = n * flat.element_size() / float(np.median(ts))
    del dst
    # the smaller-K variant: the fused step at K/2
    K2 = cfg.k_resident // 2
    c2 = cfg.scaled(k_resident=K2)
    l2 = Layer(c2, ctx, nbmax, device=dev)
    l2.summ.copy_(layer.summ)
    l2.cold_fill(qs[0], rec_host)
    for i in range(5):
        l2.step(qs[i % len(qs)], i + 1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(20)]
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        l2.step(qs[i % len(qs)], i + 6)
        b.record(stream)
    torch.cuda.synchronize()
    t_half_s = float(np.mean([a.elapsed_time(b) for a, b in ev])) / 1e3
    del l2
    torch.cuda.empty_cache()

    units = cfg.batch * cfg.n_kv_heads
    rec_bytes = lib.record_bytes(layer.shape)
    gather_Bps = gather["bytes"] / gather["device_s"]
    out = {"layers": layers, "units": units, "record_bytes": rec_bytes,
           "link_GBps": {"gather_kernel": round(gather_Bps / 1e9, 2),
                         "sdma_1GiB_copy": round(sdma_Bps / 1e9, 2)},
           "fused_step_us": {str(cfg.k_resident): round(t_layer_s * 1e6, 1),
                             str(K2): round(t_half_s * 1e6, 1)},
           "largest_hidden": [], "predicted_step_ms": []}
    for K, t in ((cfg.k_resident, t_layer_s), (K2, t_half_s)):
        window = layers * t
        for name, bw in (("gather_kernel", gather_Bps), ("sdma_1GiB_copy", sdma_Bps)):
            m = cm.largest_hidden_admit(bw, window, layers, units, rec_bytes, K)
            out["largest_hidden"].append({"K": K, "link": name, "window_ms": round(window * 1e3, 3),
                                          "max_admit": m, "cap": round(m / K, 5),
                                          "bytes": cm.bytes_per_step(layers, units, m, rec_bytes)})
    window = layers * t_layer_s
    measured, moved = {}, {}
    if pipeline:
        measured = {row["cap"]: row["step_ms"] for row in pipeline["caps"]}
        moved = {row["cap"]: row["bytes_per_step"] for row in pipeline["caps"]}
    for cap in caps:
        m = lib.cap_to_max_admit(cap, cfg.k_resident)
        nbytes = cm.bytes_per_step(layers, units, m, rec_bytes)
        out["predicted_step_ms"].append({
            "cap": cap, "max_admit": m, "bytes": nbytes,
            "overlapped_ms": round(cm.predicted_step_s(window, nbytes, gather_Bps) * 1e3, 2),
            "serial_ms": round(cm.predicted_step_s(window, nbytes, gather_Bps, False) * 1e3, 2),
            "measured_ms": measured.get(cap),
            # the bound assumes every unit finds m misses; with the bytes the
            # pipeline actually moved:
            "overlapped_ms_moved_bytes": (round(cm.predicted_step_s(window, moved[cap], gather_Bps)
                                                * 1e3, 2) if cap in moved else None)})
    log(f"[bench] cap model: link gather {gather_Bps / 1e9:.1f} GB/s, SDMA {sdma_Bps / 1e9:.1f} GB/s; "
        f"fused step K={cfg.k_resident} {t_layer_s * 1e6:.0f} us, K={K2} {t_half_s * 1e6:.0f} us; "
        f"hidden: {[(h['K'], h['link'], h['max_admit']) for h in out['largest_hidden']]}")
    return out


def pipeline_leg(src_layer, rec_host, steps: int, warmup: int, gather_GBps=None):
    """The 36-layer decode step with the fetch-cap sweep: per layer the fused
    step on the main stream and the gather prefetch of its admissions on a side
    stream, layer-local events between them.  One host pool serves all layers
    (36 per-layer 8 GiB pools would exceed the host memory of one box); each
    layer has its own queries, resident pool and summaries in HBM."""
    import torch
    from sparse_kv_block_amd import capmodel as cm
    from sparse_kv_block_amd import gen
    from sparse_kv_block_amd.configs import FULL_36
    from sparse_kv_block_amd.pipeline import Decoder, time_cap_sweep
    cfg = FULL_36
    ctx = gen.context_lengths(cfg)
    nbmax = cfg.max_blocks()
    L = cfg.layers
    dev = "cuda"
    dec = Decoder(cfg, ctx, nbmax, L, device=dev)
    n_q = warmup + steps + 1
    qs = []
    for l in range(L):
        seq = gen.query_sequence(cfg, n_q + 1, seed=1000 * 4 + l, device=dev)
        qs.append([None] + [gen.step_queries(cfg, seq, t, seed=1000 * 4 + l) for t in range(1, n_q + 1)])
    out = {"layers": L, "batch": cfg.batch, "ctx": int(ctx.max()), "k_resident": cfg.k_resident,
           "host_pool": "one pinned pool shared by all layers", "caps": []}
    rows = time_cap_sweep(dec, rec_host, qs, cfg.caps_sweep, steps, warmup, summ_from=src_layer)
    for row in rows:
        row["attention_path_tokens_per_s"] = round(cfg.batch / (row["step_ms"] / 1e3), 1)
        if gather_GBps:
            xfer_s = row["bytes_per_step"] / (gather_GBps * 1e9)
            row["transfer_alone_ms"] = round(xfer_s * 1e3, 3)
            row["overlap_fraction"] = round(cm.overlap_fraction(
                row["step_ms"] / 1e3, row["compute_only_ms"] / 1e3, xfer_s), 3)
        out["caps"].append(row)
        log(f"[bench] 36 layers cap {row['cap']} (m={row['max_admit']}): "
            f"{row['bytes_per_step'] / 1e9:.3f} GB/step, step {row['step_ms']:.2f} ms, "
            f"fused kernels alone {row['compute_only_ms']:.2f} ms")
    del dec
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--settle-seconds", type=float, default=5.0,
                    help="idle pause before the warm-up steps (see below)")
    ap.add_argument("--config", default="qwen3_8b_16k")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU time (wall x threads) the oracle baseline runs for")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-pcie", action="store_true")
    ap.add_argument("--query-sets", type=int, default=8)
    ap.add_argument("--pipeline", action="store_true",
                    help="also run the 36-layer decode step with the fetch-cap sweep")
    ap.add_argument("--pipeline-steps", type=int, default=3)
    ap.add_argument("--dense", action="store_true",
                    help="also time the dense comparator (attention over the full HBM-resident KV)")
    ap.add_argument("--append", action="store_true",
                    help="also time the decode append (after every other GPU leg)")
    ap.add_argument("--kernels", action="store_true",
                    help="also time each standalone kernel of the step (per-kernel GB/s)")
    ap.add_argument("--capmodel", action="store_true",
                    help="also measure the host-link budget (SDMA copy, K/2 step) and the "
                         "largest cap that hides in a 36-layer step")
    ap.add_argument("--agreement", action="store_true",
                    help="also run the top-K agreement study (after every other GPU leg; "
                         "releases the timed layer's buffers)")
    ap.add_argument("--agreement-steps", type=int, default=16)
    ap.add_argument("--copy-probe-mib", type=int, default=1024,
                    help="size of the device copy reported as 'achievable'")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="after the run, launch a plain elementwise copy of this many MiB "
                         "(calibrates rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the look-ahead step has "
              "no cross-GPU exchange: every (request, KV head) unit is independent, so requests or "
              "KV heads shard across GPUs with no communication", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    from sparse_kv_block_amd import gen, lib
    from sparse_kv_block_amd.configs import CONFIGS
    from sparse_kv_block_amd.pipeline import Layer

    cfg = CONFIGS[args.config]
    dev = "cuda"
    ctx = gen.context_lengths(cfg)
    nbmax = cfg.max_blocks(int(ctx.max()))
    nq = args.query_sets
    log(f"[bench] {cfg.name}: B={cfg.batch} Hq={cfg.n_q_heads} Hkv={cfg.n_kv_heads} d={cfg.head_dim} "
        f"NBmax={nbmax} K={cfg.k_resident} m={lib.cap_to_max_admit(cfg.cap, cfg.k_resident)}")
    qseq = gen.query_sequence(cfg, nq + 1, device=dev)
    dirs = gen.planted_directions(cfg, qseq[1]) if cfg.planted else None
    qs = [gen.step_queries(cfg, qseq, s) for s in range(1, nq + 1)]
    t0 = time.perf_counter()
    rec_dev = gen.records(cfg, ctx, nbmax, device=dev, planted_dir=dirs)
    torch.cuda.synchronize()
    log(f"[bench] generated {rec_dev.numel() * rec_dev.element_size() / 2**30:.1f} GiB of records "
        f"in {time.perf_counter() - t0:.1f} s")
    layer = Layer(cfg, ctx, nbmax, device=dev)
    layer.summarize(rec_dev)
    # The host pool (pinned) feeds the cold fill and the prefetch; the device
    # copy stays allocated for the dense and per-kernel legs.  Freeing it
    # before the timed steps left the driver clearing the freed memory in the
    # background, which took HBM bandwidth from the first second of timed
    # work (measured 258 instead of 250 us per step).
    rec_host = torch.empty(rec_dev.shape, dtype=rec_dev.dtype, pin_memory=True)
    rec_host.copy_(rec_dev)
    torch.cuda.synchronize()
    layer.cold_fill(qs[0], rec_host)
    torch.cuda.synchronize()
    log("[bench] cold fill done")
    dense = None
    if args.dense:
        dense = dense_leg(cfg, layer, rec_dev, qs[0])

    # Settle: started right after another process that used (and freed) tens
    # of GiB of device memory, the step runs ~3 % slower for a few seconds
    # (measured 255.6, 249.6, 247.6 us in three back-to-back runs after the GPU
    # test suite, 247.0 us after a 5 s pause), so the bench idles first.
    # Warm-up: after idle the first ~5 ms of steps run a few per cent slower
    # (clock ramp), hence the 200-step default.
    torch.cuda.synchronize()
    time.sleep(max(0.0, args.settle_seconds))
    stream = torch.cuda.current_stream()
    step = 0
    for _ in range(args.warmup):
        step += 1
        layer.step(qs[(step - 1) % nq], step)
    torch.cuda.synchronize()

    # Timed region: two events on the kernel's stream bracket the K launches
    # (an event pair around every launch would put a marker between every two
    # launches, a ~10 us gap each); their span over K is the average launch
    # duration.  The per-launch spread comes from a separate pass afterwards.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step += 1
        layer.step(qs[(step - 1) % nq], step)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_kernel_s = e0.elapsed_time(e1) / 1e3 / args.steps
    spread = []
    for _ in range(20):
        step += 1
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        layer.step(qs[(step - 1) % nq], step)
        b.record(stream)
        spread.append((a, b))
    torch.cuda.synchronize()
    kern_ms = [a.elapsed_time(b) for a, b in spread]
    median_kernel_us = float(np.median(kern_ms)) * 1e3
    ms_per_step = wall / args.steps * 1e3
    value = args.steps / wall
    algo = algorithmic_bytes(cfg, ctx)
    achieved = algo["total"] / avg_kernel_s / 1e9
    admits = int(layer.admit_count.sum().item())
    log(f"[bench] {args.steps} steps in {wall * 1e3:.2f} ms: {value:.1f} layer-steps/s; kernel avg "
        f"{avg_kernel_s * 1e6:.1f} us, {achieved:.0f} GB/s (per launch: min {min(kern_ms) * 1e3:.1f}, "
        f"median {median_kernel_us:.1f} us); "
        f"last step admitted {admits} blocks")

    result = {
        "metric": "look-ahead layer-steps/s (batch 128, 16K ctx) + achieved HBM GB/s % of peak",
        "value": round(value, 2),
        "unit": "layer-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: one look-ahead layer step (attention + draft scan + "
                               f"top-K + capped eviction)",
                   "batch": cfg.batch, "ctx": int(ctx.max()), "n_q_heads": cfg.n_q_heads,
                   "n_kv_heads": cfg.n_kv_heads, "head_dim": cfg.head_dim,
                   "block_size": cfg.block_size, "k_resident": cfg.k_resident, "cap": cfg.cap},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile(cfg),
                     "kernel": kernel_name(cfg), "algorithmic_bytes_per_launch": algo["total"],
                     "avg_kernel_us": round(avg_kernel_s * 1e6, 2),
                     "median_kernel_us": round(median_kernel_us, 2)},
    }
    # one layer step's latency (the tiny workload's figure of merit)
    result["latency_us"] = {"avg": round(avg_kernel_s * 1e6, 2), "median": round(median_kernel_us, 2),
                            "min": round(min(kern_ms) * 1e3, 2),
                            "kind": "fused layer step on the GPU, HIP events (avg over the timed "
                                    "steps; median and min of 20 single launches)"}
    result["achievable"] = achievable_leg(args.copy_probe_mib)

    if not args.no_pcie:
        # prefetch leg: the blocks the last step admitted, gather kernel reading
        # pinned host memory on a side stream, then DMA copies
        side = torch.cuda.Stream()
        res = {}
        nbytes = admits * lib.record_bytes(layer.shape)
        staging = torch.empty(cfg.batch * cfg.n_kv_heads * (3 * cfg.k_resident + 1),
                              dtype=torch.int32, pin_memory=True)
        for name, mode in (("gather", lib.GATHER), ("memcpy", lib.MEMCPY)):
            ts = []
            for rep in range(4):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                h0 = time.perf_counter()
                a.record(side)
                layer.prefetch(rec_host, mode=mode, host_staging=staging, side_stream=side)
                b.record(side)
                torch.cuda.synchronize()
                ts.append((a.elapsed_time(b) / 1e3, time.perf_counter() - h0))
            dev_s = float(np.median([t[0] for t in ts[1:]]))
            host_s = float(np.median([t[1] for t in ts[1:]]))
            res[name] = {"bytes": nbytes, "device_s": dev_s, "host_s": host_s,
                         "GBps": round(nbytes / max(host_s, 1e-9) / 1e9, 2)}
        best = min(r["host_s"] for r in res.values())
        result["pcie"] = {"admitted_blocks_per_step": admits, "bytes_per_step": nbytes,
                          "gather": res["gather"], "memcpy": res["memcpy"],
                          "pcie_inclusive_layer_steps_per_s": round(1.0 / (ms_per_step / 1e3 + best), 2)}
        log(f"[bench] prefetch {nbytes / 1e6:.1f} MB: gather {res['gather']['GBps']} GB/s, "
            f"memcpy {res['memcpy']['GBps']} GB/s")

    if dense is not None:
        dense["sparse_step_speedup"] = round(dense["us"] / (avg_kernel_s * 1e6), 2)
        result["dense_comparator"] = dense
    if args.pipeline:
        result["pipeline_36_layer"] = pipeline_leg(
            layer, rec_host, args.pipeline_steps, 2,
            gather_GBps=(result["pcie"]["gather"]["bytes"] / result["pcie"]["gather"]["device_s"] / 1e9
                         if "pcie" in result else None))

    if args.kernels:
        result["per_kernel"] = kernels_leg(cfg, layer, ctx, nbmax, qs, rec_dev)
    if args.capmodel:
        if "pcie" not in result:
            log("[bench] --capmodel needs the prefetch leg (drop --no-pcie)")
        else:
            result["cap_model"] = capmodel_leg(cfg, layer, rec_host, ctx, nbmax, qs, avg_kernel_s,
                                               result["pcie"]["gather"],
                                               result.get("pipeline_36_layer"))
    if args.append:
        result["append"] = append_leg(layer, rec_host)
    if args.agreement:
        del layer
        torch.cuda.empty_cache()
        result["agreement"] = agreement_leg(cfg, ctx, nbmax, args.agreement_steps,
                                            (0.01, 0.05, 0.2, 1.0), (0.0, 0.1, 0.2, 0.4))

    if not args.no_cpu_baseline:
        log(f"[bench] oracle baseline ...")
        result["cpu_baseline"] = cpu_baseline(cfg, ctx, rec_host, qs[0].cpu(), args.cpu_seconds)
        log(f"[bench] oracle: {result['cpu_baseline']['value']:.3f} layer-steps/s on "
            f"{result['cpu_baseline']['cores']} threads")
    if args.copy_calib_mib:
        n = args.copy_calib_mib * 2**20 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)       # a kernel name nothing else in the run uses
        torch.cuda.synchronize()
        result["copy_calib_bytes"] = n * 4
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
