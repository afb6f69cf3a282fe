"""Top-K agreement study: how well the look-ahead selection predicts the
blocks the next step needs (pith.science paper page, "Core claim", and the
referee report on its Fig. 6, which compares the draft's predicted top-K set
with the exact top-K set of the true next query).

After the look-ahead step of step s (whose draft row stands in for step s+1)
the study compares, per (request, KV head) unit, the exact top-K E of the true
next query (row 0 of step s+1's queries; exact block scores from the keys)
with:
  pred      the step's own selection T_s (summary scan of the draft row);
  resident  the resident set after T_s's capped eviction (the hit rate of the
            next step; 1 - hit is the miss rate the fetch cap leaves);
  bound     the summary-scan top-K of the true next query (what the Quest
            bound alone loses);
  drift     the exact top-K of the draft row (what the draft's error alone
            loses);
  previous  the summary-scan top-K of the current query (the previous-query
            proxy the pages contrast the look-ahead with).
Each comparison is made on the whole exact list (K blocks) and on its `top`
best blocks (recall of the blocks that carry the attention; default 8, the
number of high-affinity blocks the synthetic workloads plant per unit).
Every step runs in the library's kernels; this module only orders the calls
and sums the per-unit counts.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

from . import lib
from .pipeline import Layer

METRICS = ("pred", "resident", "bound", "drift", "previous")


class AgreementStudy:
    def __init__(self, layer: Layer, top: int = 8):
        self.layer = layer
        self.top = max(1, min(top, layer.cfg.k_resident))
        B, H, K = layer.cfg.batch, layer.cfg.n_kv_heads, layer.cfg.k_resident
        dev = layer.device
        self.exact_idx = torch.full((B, H, K), -1, dtype=torch.int32, device=dev)
        self.exact_score = torch.zeros((B, H, K), dtype=torch.float32, device=dev)
        self.aux_idx = torch.full((B, H, K), -1, dtype=torch.int32, device=dev)
        self.aux_score = torch.zeros((B, H, K), dtype=torch.float32, device=dev)
        # "resident" is column 2 of the "pred" counts
        self.counts = {m + sfx: torch.zeros((B, H, 3), dtype=torch.int32, device=dev)
                       for m in METRICS if m != "resident" for sfx in ("", "@top")}

    def _count(self, name: str, pred: torch.Tensor, l2p: Optional[torch.Tensor] = None):
        sh = self.layer.shape
        lib.topk_agreement(sh, pred, self.exact_idx, self.counts[name], l2p=l2p)
        lib.topk_agreement(sh, pred, self.exact_idx, self.counts[name + "@top"], l2p=l2p,
                           exact_n=self.top)

    def step(self, records, q: torch.Tensor, q_next: torch.Tensor, step: int,
             max_admit: Optional[int] = None, keep_units: bool = False) -> Dict[str, np.ndarray]:
        """One look-ahead layer step (fused) and its prefetch from `records`,
        then the five comparisons.  Returns per metric the summed (n_exact,
        agreeing, resident) counts, or the per-unit counts with keep_units."""
        L, sh = self.layer, self.layer.shape
        L.step(q, step, max_admit)
        L.prefetch(records, max_admit)
        lib.exact_topk(sh, q_next, records, L.ctx_len, self.exact_idx, self.exact_score, q_row=0)
        self._count("pred", L.topk_idx, L.l2p)
        lib.score_topk(sh, q_next, L.summ, L.ctx_len, self.aux_idx, self.aux_score, q_row=0,
                       workspace=L.workspace)
        self._count("bound", self.aux_idx)
        lib.exact_topk(sh, q, records, L.ctx_len, self.aux_idx, self.aux_score, q_row=1)
        self._count("drift", self.aux_idx)
        lib.score_topk(sh, q, L.summ, L.ctx_len, self.aux_idx, self.aux_score, q_row=0,
                       workspace=L.workspace)
        self._count("previous", self.aux_idx)
        if keep_units:
            out = {m: c.cpu().numpy().copy() for m, c in self.counts.items()}
        else:
            out = {m: c.sum(dim=(0, 1)).cpu().numpy() for m, c in self.counts.items()}
        out["resident"] = out["pred"]
        out["resident@top"] = out["pred@top"]
        return out


def summarize_counts(per_step: List[Dict[str, np.ndarray]], top: int = 8) -> dict:
    """Mean and worst step of each fraction: agreement (column 1 / column 0)
    for every metric, hit rate (column 2 / column 0) for `resident`; keys
    `<metric>` (whole lists) and `<metric>_top<n>` (the exact list's n best)."""
    out = {}
    for m in METRICS:
        col = 2 if m == "resident" else 1
        for sfx, name in (("", m), ("@top", f"{m}_top{top}")):
            fr = [float(c[m + sfx][col]) / max(1.0, float(c[m + sfx][0])) for c in per_step]
            out[name] = {"mean": round(float(np.mean(fr)), 5), "min": round(float(np.min(fr)), 5)}
    return out


def run_study(layer: Layer, records, queries: Sequence[torch.Tensor], steps: int,
              max_admit: Optional[int] = None, first_step: int = 1, top: int = 8) -> dict:
    """`queries[s]` is step s's [B][2][Hq][d] query tensor; steps
    first_step .. first_step+steps-1 run, each compared with the next."""
    st = AgreementStudy(layer, top)
    per = []
    for s in range(first_step, first_step + steps):
        per.append(st.step(records, queries[s], queries[s + 1], s, max_admit))
    return summarize_counts(per, st.top)
