"""Comparison helpers for the GPU-vs-oracle parity tests (imported by tests only)."""
from __future__ import annotations

import numpy as np
import torch

import oracle

TOPK_REL = 1e-5      # swaps allowed within 1e-5 relative of the K-th score
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
               what="", exact=False):
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
