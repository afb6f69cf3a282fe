"""Device state of one attention layer and the calls that drive it.

`Layer` owns the HBM side of the look-ahead decode step for one layer: the
resident slot pool, the block summaries, the per-KV-head block maps and the
per-step outputs.  The full KV (records) lives elsewhere (pinned host memory
or device memory) and is read through `summarize`, `cold_fill` and `prefetch`
and written by `append`.  Every method enqueues C-ABI calls on the current stream.
"""
from __future__ import annotations

import time
from typing import Optional, Sequence

import numpy as np
import torch

from . import lib
from .configs import Config
from .gen import TORCH_DTYPE


class Layer:
    def __init__(self, cfg: Config, ctx: np.ndarray, nbmax: int, device="cuda"):
        self.cfg = cfg
        self.shape = lib.Shape.of(cfg, nbmax)
        B, H, K, d, Hq = cfg.batch, cfg.n_kv_heads, cfg.k_resident, cfg.head_dim, cfg.n_q_heads
        dt = TORCH_DTYPE[cfg.dtype]
        self.device = device
        self.nbmax = nbmax
        self.ctx_len = torch.as_tensor(np.asarray(ctx, np.int32), device=device)
        self.pool = torch.zeros((B, H, K, cfg.record_elems), dtype=dt, device=device)
        self.summ = torch.zeros((B, H, nbmax, 2, d), dtype=dt, device=device)
        self.l2p = torch.full((B, H, nbmax), -1, dtype=torch.int32, device=device)
        self.p2l = torch.full((B, H, K), -1, dtype=torch.int32, device=device)
        self.last_sel = torch.zeros((B, H, K), dtype=torch.int32, device=device)
        self.out = torch.zeros((B, 2, Hq, d), dtype=dt, device=device)
        self.topk_idx = torch.full((B, H, K), -1, dtype=torch.int32, device=device)
        self.topk_score = torch.zeros((B, H, K), dtype=torch.float32, device=device)
        self.admit = torch.full((B, H, K, 3), -1, dtype=torch.int32, device=device)
        self.admit_count = torch.zeros((B, H), dtype=torch.int32, device=device)
        self.workspace = lib.layer_step_workspace(self.shape, device)
        # admissions per unit and step at the workload's cap (the library's rule)
        self.max_admit = lib.cap_to_max_admit(cfg.cap, K)

    # ------------------------------------------------------------------ setup
    def summarize(self, records):
        lib.summarize(self.shape, records, self.ctx_len, self.summ)

    def cold_fill(self, q: torch.Tensor, records, mode: int = lib.GATHER, host_staging=None):
        """Initial resident set: the top-K blocks of the normal query's scores,
        stamped 0, copied in from `records`."""
        K = self.shape.k_resident
        self.l2p.fill_(-1)
        self.p2l.fill_(-1)
        self.last_sel.zero_()
        lib.score_topk(self.shape, q, self.summ, self.ctx_len, self.topk_idx, self.topk_score, q_row=0,
                       workspace=self.workspace)
        lib.capped_evict(self.shape, self.topk_idx, 0, K, self.l2p, self.p2l, self.last_sel,
                         self.admit, self.admit_count)
        self.prefetch(records, K, mode=mode, host_staging=host_staging)

    def append(self, records, k_new: torch.Tensor, v_new: torch.Tensor):
        """Decode append of one token per request ([B][Hkv][d] keys and values):
        into `records`, the resident copy of its block when resident, and the
        block's summary; this layer's context lengths grow by one.  Enqueued on
        the current stream: the caller orders it after any prefetch still
        filling this layer's slots (`Decoder.append` does), or a gather that
        read the record before the append could overwrite the slot after it."""
        lib.append_token(self.shape, k_new, v_new, records, self.summ, self.ctx_len,
                         pool=self.pool, l2p=self.l2p)

    def set_state(self, l2p, p2l, last_sel):
        self.l2p.copy_(torch.as_tensor(l2p))
        self.p2l.copy_(torch.as_tensor(p2l))
        self.last_sel.copy_(torch.as_tensor(last_sel))

    def state(self):
        return (self.l2p.clone(), self.p2l.clone(), self.last_sel.clone())

    # ------------------------------------------------------------------ per step
    def step(self, q: torch.Tensor, step: int, max_admit: Optional[int] = None, scale: float = 0.0):
        """Fused look-ahead layer step (attention, scan, top-K, eviction)."""
        m = self.max_admit if max_admit is None else max_admit
        lib.layer_step(self.shape, q, self.pool, self.summ, self.ctx_len, step, m, self.out,
                       self.topk_idx, self.topk_score, self.l2p, self.p2l, self.last_sel,
                       self.admit, self.admit_count, scale=scale, workspace=self.workspace)

    def step_unfused(self, q: torch.Tensor, step: int, max_admit: Optional[int] = None,
                     scale: float = 0.0):
        """The same step as four separate C-ABI calls."""
        m = self.max_admit if max_admit is None else max_admit
        lib.lookahead_attn(self.shape, q, self.pool, self.p2l, self.ctx_len, self.out, scale=scale)
        lib.score_topk(self.shape, q, self.summ, self.ctx_len, self.topk_idx, self.topk_score, q_row=1,
                       workspace=self.workspace)
        lib.capped_evict(self.shape, self.topk_idx, step, m, self.l2p, self.p2l, self.last_sel,
                         self.admit, self.admit_count)

    def prefetch(self, records, max_admit: Optional[int] = None, mode: int = lib.GATHER,
                 host_staging=None, side_stream=None, wait_before=None, done=None):
        m = self.max_admit if max_admit is None else max_admit
        lib.prefetch(self.shape, records, self.pool, self.admit, self.admit_count, m, mode=mode,
                     host_staging=host_staging, side_stream=side_stream,
                     wait_before=wait_before, done=done)


class Decoder:
    """Several layers stepped in order, the way a decode step runs them.

    Per layer and step, on the caller's (main) stream: wait for this layer's
    previous prefetch, run the fused look-ahead step, record `ev_sel`.  On the
    side stream: wait for `ev_sel`, prefetch the admitted blocks, record
    `ev_pf`.  The event after the fused step covers both the admission list
    and the write-after-read hazard on the victim slots (attention of this
    step read them); the event after the prefetch is the layer-local
    synchronisation the next step waits on.  Prefetches of different layers
    queue on the one side stream (the host link is one resource) and overlap
    the main stream's later layers.

    All layers may share one `records` array (the host pool) when host memory
    cannot hold one per layer; their queries differ.
    """

    def __init__(self, cfg: Config, ctx: np.ndarray, nbmax: int, n_layers: int, device="cuda"):
        self.cfg = cfg
        self.layers = [Layer(cfg, ctx, nbmax, device) for _ in range(n_layers)]
        self.side = torch.cuda.Stream(device=device)
        self.ev_sel = [torch.cuda.Event() for _ in range(n_layers)]
        self.ev_pf = [torch.cuda.Event() for _ in range(n_layers)]
        self.pending = [False] * n_layers
        self.staging = None

    def setup(self, records, qs_first, summ_from: Optional[Layer] = None):
        """Summaries (computed once from `records`, or copied from `summ_from`)
        and the cold fill of every layer."""
        for i, layer in enumerate(self.layers):
            if summ_from is not None:
                layer.summ.copy_(summ_from.summ)
            elif i == 0:
                layer.summarize(records)
            else:
                layer.summ.copy_(self.layers[0].summ)
            layer.cold_fill(qs_first[i], records)
        self.pending = [False] * len(self.layers)

    def step(self, records, qs, step: int, max_admit: Optional[int] = None, mode: int = lib.GATHER,
             before_prefetch=None):
        """One decode step over all layers; qs[i] is layer i's query tensor.
        `before_prefetch(i)` (optional) is enqueued on the side stream before
        layer i's prefetch (tests use it to delay the side stream)."""
        m = self.layers[0].max_admit if max_admit is None else max_admit
        main = torch.cuda.current_stream()
        if mode == lib.MEMCPY and self.staging is None:
            n = self.layers[0].shape.units() * (3 * self.cfg.k_resident + 1)
            self.staging = torch.empty(n, dtype=torch.int32, pin_memory=True)
        for i, layer in enumerate(self.layers):
            if self.pending[i]:
                main.wait_event(self.ev_pf[i])
            layer.step(qs[i], step, m)
            self.ev_sel[i].record(main)
            if before_prefetch is not None:
                self.side.wait_event(self.ev_sel[i])
                with torch.cuda.stream(self.side):
                    before_prefetch(i)
            layer.prefetch(records, m, mode=mode, host_staging=self.staging,
                           side_stream=self.side, wait_before=self.ev_sel[i], done=self.ev_pf[i])
            self.pending[i] = True

    def append(self, i: int, records, k_new: torch.Tensor, v_new: torch.Tensor):
        """Decode append into layer i (see `Layer.append`), ordered after that
        layer's pending prefetch on the side stream."""
        if self.pending[i]:
            torch.cuda.current_stream().wait_event(self.ev_pf[i])
        self.layers[i].append(records, k_new, v_new)

    def drain(self):
        main = torch.cuda.current_stream()
        for i in range(len(self.layers)):
            if self.pending[i]:
                main.wait_event(self.ev_pf[i])


def time_cap_sweep(dec: Decoder, records, qs, caps: Sequence[float], steps: int, warmup: int,
                   summ_from: Optional[Layer] = None):
    """The pipelined decode step of every layer of `dec` at each fetch cap.

    Per cap: cold fill (`Decoder.setup`), `warmup` untimed steps, then `steps`
    timed steps (the fused step of each layer on the current stream, its
    gather prefetch on the side stream, layer-local events), bracketed by two
    events on the current stream after a drain; then the same number of steps
    with no admissions (the fused kernels alone).  qs[l][t] is layer l's query
    tensor at step t (t >= 1; qs[l][0] unused).  Returns one row per cap:
    admissions allowed per unit (max_admit, from the library's cap rule),
    bytes moved per step (from the admission counts) and their bound
    (layers * units * max_admit * record bytes), step and compute-only times,
    and the host-link rate the step sustained."""
    L = len(dec.layers)
    shape = dec.layers[0].shape
    K = shape.k_resident
    units = shape.units()
    rec_bytes = lib.record_bytes(shape)
    main = torch.cuda.current_stream()
    rows = []
    for cap in caps:
        m = lib.cap_to_max_admit(cap, K)
        dec.setup(records, [qs[l][1] for l in range(L)], summ_from=summ_from)
        torch.cuda.synchronize()
        t = 0
        for _ in range(warmup):
            t += 1
            dec.step(records, [qs[l][t] for l in range(L)], t, m)
        dec.drain()
        torch.cuda.synchronize()
        admitted = torch.zeros((), dtype=torch.int64, device=dec.layers[0].device)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        h0 = time.perf_counter()
        a.record(main)
        for _ in range(steps):
            t += 1
            dec.step(records, [qs[l][t] for l in range(L)], t, m)
            for layer in dec.layers:
                admitted += layer.admit_count.sum()
        dec.drain()
        b.record(main)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - h0) / steps
        step_s = a.elapsed_time(b) / 1e3 / steps
        c, d = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c.record(main)
        for _ in range(steps):
            for l, layer in enumerate(dec.layers):
                layer.step(qs[l][t], t + 1, 0)
        d.record(main)
        torch.cuda.synchronize()
        compute_s = c.elapsed_time(d) / 1e3 / steps
        moved = int(admitted.item()) * rec_bytes / steps
        rows.append({"cap": cap, "max_admit": m, "bytes_per_step": moved,
                     "bytes_bound": units * L * m * rec_bytes,
                     "step_ms": round(step_s * 1e3, 3), "wall_ms": round(wall * 1e3, 3),
                     "compute_only_ms": round(compute_s * 1e3, 3),
                     "host_link_GBps": round(moved / step_s / 1e9, 2)})
    return rows
