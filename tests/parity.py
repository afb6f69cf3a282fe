"""Comparison helpers for the GPU-vs-oracle parity tests (imported by tests only)."""
from __future__ import annotations

import numpy as np
import torch

import oracle

TOPK_REL = 1e-5      # swaps allowed within 1e-5 relative of the K-th score
RANK_MARGIN = 8.0    # swaps explained by rounding: within 8x the largest score error seen
ATTN_TOL = {"bf16": 1e-2, "f32": 1e-5}


def host(t: torch.Tensor) -> np.ndarray:
    """numpy copy of a tensor (bf16 as uint16 bit patterns)."""
    return oracle.as_np(t.detach().cpu())


def i32(t) -> np.ndarray:
    return np.ascontiguousarray(host(t) if isinstance(t, torch.Tensor) else t, dtype=np.int32)


def check_attention(out_gpu: torch.Tensor, out_ora: np.ndarray, dtype: str, what=""):
    g = oracle.to_f64(host(out_gpu))
    tol = ATTN_TOL[dtype]
    err = np.abs(g - out_ora) - (tol + tol * np.abs(out_ora))
    bad = np.argwhere(err > 0)
    assert bad.size == 0, (f"{what}: {len(bad)} attention outputs out of tolerance, first at "
                           f"{bad[0].tolist()}: gpu {g[tuple(bad[0])]} oracle {out_ora[tuple(bad[0])]}")
    return float(np.max(np.abs(g - out_ora)))


def check_topk(idx_gpu: np.ndarray, sc_gpu: np.ndarray, idx_ora: np.ndarray, scores_ora: np.ndarray,
               what="", exact=False, differ_units=None):
    """Top-K parity per unit.  The lists must have the same length; every block
    in their symmetric difference must score within TOPK_REL (relative) of the
    oracle's K-th score; position r of the GPU list must hold a block whose
    oracle score equals the oracle's r-th score within the same tolerance; the
    fp32 scores the GPU reports must match the oracle's.  Returns the number of
    units whose lists differ."""
    B, H, K = idx_ora.shape
    differ = 0
    for b in range(B):
        for h in range(H):
            ig, io = idx_gpu[b, h], idx_ora[b, h]
            n = int((io >= 0).sum())
            assert int((ig >= 0).sum()) == n, f"{what} unit ({b},{h}): list lengths differ"
            assert np.all(ig[n:] == -1) and np.all(io[n:] == -1)
            if np.array_equal(ig, io):
                s = scores_ora[b, h, io[:n]]
                np.testing.assert_allclose(sc_gpu[b, h, :n], s, rtol=TOPK_REL,
                                           atol=TOPK_REL * (abs(s[-1]) if n else 0) + 1e-30,
                                           err_msg=f"{what} unit ({b},{h}) reported scores")
                continue
            assert not exact, f"{what} unit ({b},{h}): top-K lists differ on exact inputs"
            differ += 1
            if differ_units is not None:
                differ_units.append((b, h))
            s_row = scores_ora[b, h]
            kth = s_row[io[n - 1]]
            tol = TOPK_REL * abs(kth)
            for j in set(ig[:n].tolist()) ^ set(io[:n].tolist()):
                assert abs(s_row[j] - kth) <= tol, (
                    f"{what} unit ({b},{h}): block {j} (score {s_row[j]}) swapped at the K-th "
                    f"score {kth}")
            for r in range(n):
                assert abs(s_row[ig[r]] - s_row[io[r]]) <= tol, (
                    f"{what} unit ({b},{h}) position {r}: gpu block {ig[r]} ({s_row[ig[r]]}) "
                    f"vs oracle {io[r]} ({s_row[io[r]]})")
    return differ


def unit_slice(x, b: int, h: int, G: int, kind: str):
    """The slice of an array that belongs to unit (b, h), as a batch of one
    request with one KV head.  kind: 'unit' ([B][H]...), 'q' ([B][2][Hq][d]),
    'ctx' ([B])."""
    if kind == "unit":
        return x[b:b + 1, h:h + 1]
    if kind == "q":
        return x[b:b + 1, :, h * G:(h + 1) * G]
    if kind == "ctx":
        return x[b:b + 1]
    raise ValueError(kind)


def sample_units(B: int, H: int, n: int, seed: int):
    rng = np.random.default_rng(seed)
    picks = {(0, 0), (B - 1, H - 1)}
    while len(picks) < min(n, B * H):
        picks.add((int(rng.integers(B)), int(rng.integers(H))))
    return sorted(picks)


def pool_from_records(records: torch.Tensor, p2l: torch.Tensor) -> torch.Tensor:
    """Test-side construction of a slot pool: pool[b,h,s] = records[b,h,p2l[b,h,s]]
    (zero for empty slots)."""
    idx = p2l.long().clamp_min(0)
    pool = torch.gather(records, 2, idx[..., None].expand(-1, -1, -1, records.shape[-1]))
    pool[p2l < 0] = 0
    return pool.contiguous()


def tie_exposed(scores_ora: np.ndarray, K: int, delta) -> np.ndarray:
    """Per unit: whether two adjacent ones of the oracle's K+1 best scores lie
    within `delta` (a scalar or a [B][H] array) of each other: only there can a
    GPU list order two blocks differently from the oracle."""
    B, H, NB = scores_ora.shape
    n = min(K + 1, NB)
    top = -np.sort(-scores_ora.reshape(B * H, NB), axis=1)[:, :n]
    dl = np.broadcast_to(np.asarray(delta, np.float64), (B, H)).reshape(B * H)
    out = np.zeros(B * H, bool)
    for u in range(B * H):
        s = top[u][np.isfinite(top[u])]
        if s.size >= 2:
            out[u] = bool(np.any(s[:-1] - s[1:] <= dl[u]))
    return out.reshape(B, H)


def rounding_scale(idx_gpu: np.ndarray, sc_gpu: np.ndarray, scores_ora: np.ndarray) -> float:
    """The largest difference between a score the GPU reports for a block of its
    list and the oracle's fp64 score of that block: the GPU's fp32 rounding
    scale of this call."""
    valid = idx_gpu >= 0
    ref = np.take_along_axis(scores_ora, np.where(valid, idx_gpu, 0).astype(np.int64), axis=2)
    err = np.abs(sc_gpu.astype(np.float64) - ref)
    return float(err[valid].max()) if valid.any() else 0.0


def check_swaps_within(idx_gpu, idx_ora, scores_ora, units, delta, what=""):
    """Every difference between the GPU's and the oracle's lists of the given
    units is between blocks whose oracle scores lie within `delta`."""
    for (b, h) in units:
        ig, io, s_row = idx_gpu[b, h], idx_ora[b, h], scores_ora[b, h]
        n = int((io >= 0).sum())
        kth = s_row[io[n - 1]]
        for j in set(ig[:n].tolist()) ^ set(io[:n].tolist()):
            assert abs(s_row[j] - kth) <= delta, (
                f"{what} unit ({b},{h}): block {j} swapped at the K-th score with a gap "
                f"{abs(s_row[j] - kth)} above the rounding scale {delta}")
        for r in range(n):
            assert abs(s_row[ig[r]] - s_row[io[r]]) <= delta, (
                f"{what} unit ({b},{h}) position {r}: gap {abs(s_row[ig[r]] - s_row[io[r]])} "
                f"above the rounding scale {delta}")


def summaries_equal_by_value(got: np.ndarray, ref: np.ndarray) -> bool:
    """Summaries compared by value: bit-identical, except that +0 and -0 are
    equal (a min or max of equal values may keep either sign of zero)."""
    if got.dtype == np.uint16:
        same = got == ref
        zero = ((got & 0x7FFF) == 0) & ((ref & 0x7FFF) == 0)
        return bool(np.all(same | zero))
    return bool(np.all(got == ref))


class OracleTwin:
    """The oracle's copy of one layer's resident state, stepped beside a GPU
    `Layer` on the same inputs and compared with it in full after every call.

    Attention is compared within the tolerance; the top-K list per unit within
    the tolerance at the K-th score (R21 of the readings: a list that differs
    must differ only among scores within TOPK_REL of each other); then the
    oracle evicts with the GPU's (validated) list, so that every unit's block
    maps, stamps and admissions are compared bit for bit at every step, also
    where the lists differed, and the two states never part."""

    def __init__(self, cfg, rec_cpu, ctx, summ=None):
        self.cfg = cfg
        self.rec = rec_cpu
        self.ctx = np.ascontiguousarray(np.asarray(ctx, np.int32))
        self.summ = oracle.summarize(rec_cpu, self.ctx, 16) if summ is None else summ
        B, H, NB = rec_cpu.shape[0], rec_cpu.shape[1], rec_cpu.shape[2]
        K = cfg.k_resident
        self.l2p = np.full((B, H, NB), -1, np.int32)
        self.p2l = np.full((B, H, K), -1, np.int32)
        self.ls = np.zeros((B, H, K), np.int32)
        self.unit_steps = 0
        self.differ = []
        self.exposed = 0
        self.eps = 0.0

    def check_summaries(self, layer, what=""):
        assert summaries_equal_by_value(host(layer.summ), self.summ), f"{what}: summaries differ"

    def _topk(self, layer, q_cpu, q_row, what):
        K = self.cfg.k_resident
        sc = oracle.block_scores(q_cpu, self.summ, self.ctx, 16, q_row=q_row)
        idx, _ = oracle.topk(sc, self.ctx, 16, K)
        ig, sg = i32(layer.topk_idx), host(layer.topk_score)
        differ_units = []
        check_topk(ig, sg, idx, sc, what=what, differ_units=differ_units)
        # stricter than the tolerance: every difference is explained by the
        # GPU's fp32 rounding (RANK_MARGIN times the largest error it reports
        # on any listed block of this call), and only units whose oracle
        # scores hold a gap that small can differ
        eps = rounding_scale(ig, sg, sc)
        delta = RANK_MARGIN * eps
        check_swaps_within(ig, idx, sc, differ_units, delta, what)
        exposed = tie_exposed(sc, K, delta)
        for (b, h) in differ_units:
            assert exposed[b, h], f"{what} unit ({b},{h}): lists differ without a near-tie"
        self.unit_steps += exposed.size
        self.exposed += int(exposed.sum())
        self.eps = max(self.eps, eps)
        self.differ += [(what, b, h) for (b, h) in differ_units]
        return ig

    def _maps(self, layer, admit, count, what):
        np.testing.assert_array_equal(i32(layer.l2p), self.l2p, err_msg=f"{what}: l2p")
        np.testing.assert_array_equal(i32(layer.p2l), self.p2l, err_msg=f"{what}: p2l")
        np.testing.assert_array_equal(i32(layer.last_sel), self.ls, err_msg=f"{what}: last_sel")
        np.testing.assert_array_equal(i32(layer.admit), admit, err_msg=f"{what}: admit")
        np.testing.assert_array_equal(i32(layer.admit_count), count, err_msg=f"{what}: admit_count")

    def cold_fill(self, layer, q_cpu, what=""):
        """After layer.cold_fill(q): the normal row's top-K into empty slots at step 0."""
        T = self._topk(layer, q_cpu, 0, f"{what} cold fill")
        self.l2p.fill(-1)
        self.p2l.fill(-1)
        self.ls.fill(0)
        K = self.cfg.k_resident
        admit, count = oracle.capped_evict(T, 0, K, self.l2p, self.p2l, self.ls)
        self._maps(layer, admit, count, f"{what} cold fill")

    def step(self, layer, q_cpu, step, m, what=""):
        """After layer.step(q, step, m): attention over the state before the
        step, then the draft row's top-K and the capped eviction."""
        out = oracle.attention(q_cpu, self.rec, self.p2l, self.ctx, 16)
        check_attention(layer.out, out, self.cfg.dtype, f"{what} step {step}")
        T = self._topk(layer, q_cpu, 1, f"{what} step {step}")
        admit, count = oracle.capped_evict(T, step, m, self.l2p, self.p2l, self.ls)
        self._maps(layer, admit, count, f"{what} step {step}")
        return admit, count

    def report(self):
        return (f"{self.unit_steps} unit-steps compared in full, {len(self.differ)} top-K lists "
                f"differed, each only between blocks within {RANK_MARGIN} x the fp32 rounding "
                f"scale (largest {self.eps:.3g}) of each other (bound: {self.exposed} unit-steps "
                f"with such a near-tie)")
