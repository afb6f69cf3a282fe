"""Seeded synthetic inputs for the look-ahead sparse decode step.

This module only draws random numbers and lays them out.  It holds none of the
method's arithmetic (no summaries, scores, selection, eviction or attention), so
that both the HIP path and the CPU oracle can be fed the very same bytes from it.

Recipes (stated again in the design notes):
  * keys and values are i.i.d. N(0, 1); tokens at or past a request's context
    length are zero;
  * queries drift between decode steps as AR(1): q[s+1] = rho*q[s] +
    sqrt(1-rho^2)*eps; step s uses q[s] as its normal row and q[s+1] plus
    N(0, draft_sigma) noise as its draft row (the speculative lookahead);
  * "planted" blocks: a few blocks per (request, KV head) whose valid keys are
    shifted by planted_shift along the unit vector of the summed next-step query
    of the KV head's query group;
  * lognormal context lengths with the requested mean, clipped.

Block record layout, one per (request, KV head, logical block):
  keys   [S][d]  (token-major)      elements [0, S*d)
  values [d][S]  (transposed)       elements [S*d, 2*S*d)
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
import torch

from .configs import Config

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    return g


def context_lengths(cfg: Config, seed: Optional[int] = None) -> np.ndarray:
    """Per-request context lengths (int32, [B])."""
    seed = cfg.seed if seed is None else seed
    if cfg.ctx is not None:
        return np.full(cfg.batch, cfg.ctx, dtype=np.int32)
    mean, sigma, lo, hi = cfg.ctx_lognormal
    rng = np.random.default_rng([seed, 11])
    mu = math.log(mean) - 0.5 * sigma * sigma
    x = rng.lognormal(mu, sigma, cfg.batch)
    return np.clip(np.rint(x), lo, hi).astype(np.int32)


def query_sequence(cfg: Config, n: int, seed: Optional[int] = None,
                   device="cpu") -> torch.Tensor:
    """q[1..n] as an fp32 tensor [n][B][Hq][d] (index 0 holds q[1])."""
    seed = cfg.seed if seed is None else seed
    g = _gen(device, seed * 7919 + 1)
    shape = (cfg.batch, cfg.n_q_heads, cfg.head_dim)
    out = torch.empty((n,) + shape, dtype=torch.float32, device=device)
    out[0] = torch.randn(shape, generator=g, device=device)
    a = math.sqrt(max(0.0, 1.0 - cfg.rho * cfg.rho))
    for s in range(1, n):
        eps = torch.randn(shape, generator=g, device=device)
        out[s] = cfg.rho * out[s - 1] + a * eps
    return out


def step_queries(cfg: Config, qseq: torch.Tensor, step: int,
                 seed: Optional[int] = None) -> torch.Tensor:
    """Query tensor [B][2][Hq][d] (storage dtype) for decode step `step` >= 1:
    row 0 = q[step] (normal), row 1 = q[step+1] + N(0, draft_sigma) (draft)."""
    seed = cfg.seed if seed is None else seed
    device = qseq.device
    g = _gen(device, seed * 104729 + step)
    normal = qseq[step - 1]
    noise = torch.randn(normal.shape, generator=g, device=device)
    draft = qseq[step] + cfg.draft_sigma * noise
    q = torch.stack([normal, draft], dim=1)
    return q.to(TORCH_DTYPE[cfg.dtype]).contiguous()


def planted_directions(cfg: Config, q_next: torch.Tensor) -> torch.Tensor:
    """Unit vector of the summed next-step query per (request, KV head): [B][Hkv][d]."""
    grp = q_next.reshape(cfg.batch, cfg.n_kv_heads, cfg.group, cfg.head_dim).sum(dim=2)
    return grp / grp.norm(dim=-1, keepdim=True).clamp_min(1e-30)


def records(cfg: Config, ctx: np.ndarray, nbmax: int, seed: Optional[int] = None,
            device="cpu", planted_dir: Optional[torch.Tensor] = None,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Block records [B][Hkv][NBmax][2*S*d] in the storage dtype."""
    seed = cfg.seed if seed is None else seed
    B, H, S, d = cfg.batch, cfg.n_kv_heads, cfg.block_size, cfg.head_dim
    dt = TORCH_DTYPE[cfg.dtype]
    if out is None:
        out = torch.empty((B, H, nbmax, 2 * S * d), dtype=dt, device=device)
    g = _gen(device, seed * 15485863 + 3)
    tok = torch.arange(nbmax * S, device=device).reshape(nbmax, S)
    for b in range(B):
        L = int(ctx[b])
        x = torch.randn((H, nbmax, 2, S * d), generator=g, device=device)
        valid = (tok < L).to(torch.float32)                        # [NB][S]
        kpart = x[:, :, 0].view(H, nbmax, S, d)
        vpart = x[:, :, 1].view(H, nbmax, d, S)
        kpart.mul_(valid[None, :, :, None])
        vpart.mul_(valid[None, :, None, :])
        nb = min(nbmax, -(-L // S))
        if cfg.planted and planted_dir is not None and nb > 0:
            r = torch.rand((H, nbmax), generator=g, device=device)
            r[:, nb:] = 2.0
            sel = torch.argsort(r, dim=1)[:, :min(cfg.planted, nb)]   # distinct blocks
            for h in range(H):
                blk = sel[h]
                add = cfg.planted_shift * planted_dir[b, h].to(torch.float32)
                kpart[h, blk] += valid[blk][:, :, None] * add[None, None, :]
        out[b].copy_(x.view(H, nbmax, 2 * S * d).to(dt))
    return out


def new_tokens(cfg: Config, n: int, seed: int, device="cpu", integer: bool = False):
    """Keys and values of n decode steps' new tokens, each [n][B][Hkv][d] in the
    storage dtype: N(0, 1) like the records, or small integers in [-3, 3]
    (frequent ties, for the summary tie rule)."""
    B, H, d = cfg.batch, cfg.n_kv_heads, cfg.head_dim
    g = _gen(device, seed * 7919 + 11)
    if integer:
        kv = torch.randint(-3, 4, (2, n, B, H, d), generator=g, device=device).to(torch.float32)
    else:
        kv = torch.randn((2, n, B, H, d), generator=g, device=device)
    kv = kv.to(TORCH_DTYPE[cfg.dtype])
    return kv[0].contiguous(), kv[1].contiguous()


def empty_state(cfg: Config, nbmax: int, device="cpu"):
    """(l2p [B][Hkv][NBmax], p2l [B][Hkv][K], last_sel [B][Hkv][K]), all int32."""
    B, H, K = cfg.batch, cfg.n_kv_heads, cfg.k_resident
    l2p = torch.full((B, H, nbmax), -1, dtype=torch.int32, device=device)
    p2l = torch.full((B, H, K), -1, dtype=torch.int32, device=device)
    last = torch.zeros((B, H, K), dtype=torch.int32, device=device)
    return l2p, p2l, last


def random_state(cfg: Config, ctx: np.ndarray, nbmax: int, seed: int,
                 fill: float = 1.0, stamp_max: int = 4):
    """Random resident sets (CPU tensors): each (request, KV head) holds
    round(fill*min(K, NB_b)) distinct logical blocks in random slots, with random
    stamps in [0, stamp_max).  l2p is the inverse of p2l."""
    B, H, K, S = cfg.batch, cfg.n_kv_heads, cfg.k_resident, cfg.block_size
    rng = np.random.default_rng([seed, 29])
    l2p = np.full((B, H, nbmax), -1, dtype=np.int32)
    p2l = np.full((B, H, K), -1, dtype=np.int32)
    last = rng.integers(0, max(1, stamp_max), size=(B, H, K), dtype=np.int32)
    for b in range(B):
        nb = min(nbmax, -(-int(ctx[b]) // S))
        n = int(round(fill * min(K, nb)))
        for h in range(H):
            blocks = rng.choice(nb, size=n, replace=False) if n else np.zeros(0, np.int64)
            slots = rng.choice(K, size=n, replace=False) if n else np.zeros(0, np.int64)
            p2l[b, h, slots] = blocks
            l2p[b, h, blocks] = slots
    return torch.from_numpy(l2p), torch.from_numpy(p2l), torch.from_numpy(last)


def integer_inputs(cfg: Config, ctx: np.ndarray, nbmax: int, seed: int,
                   lo: int = -3, hi: int = 3, device="cpu"):
    """Small-integer keys, values and queries ([lo, hi]) for the cases where every
    sum the method forms is exact in fp32, so ties are frequent and the top-K
    order must agree bit for bit.  Returns (records, q)."""
    B, H, S, d, Hq = cfg.batch, cfg.n_kv_heads, cfg.block_size, cfg.head_dim, cfg.n_q_heads
    dt = TORCH_DTYPE[cfg.dtype]
    g = _gen("cpu", seed * 31 + 7)
    rec = torch.randint(lo, hi + 1, (B, H, nbmax, 2, S * d), generator=g).to(torch.float32)
    tok = torch.arange(nbmax * S).reshape(nbmax, S)
    for b in range(B):
        valid = (tok < int(ctx[b])).to(torch.float32)
        rec[b, :, :, 0].view(H, nbmax, S, d).mul_(valid[None, :, :, None])
        rec[b, :, :, 1].view(H, nbmax, d, S).mul_(valid[None, :, None, :])
    q = torch.randint(lo, hi + 1, (B, 2, Hq, d), generator=g).to(torch.float32)
    rec = rec.reshape(B, H, nbmax, 2 * S * d).to(dt).to(device)
    return rec, q.to(dt).to(device)


def integer_queries(cfg: Config, n: int, seed: int, lo: int = -3, hi: int = 3, device="cpu"):
    """n independent small-integer query tensors [B][2][Hq][d] (storage dtype)."""
    g = _gen("cpu", seed * 131 + 17)
    q = torch.randint(lo, hi + 1, (n, cfg.batch, 2, cfg.n_q_heads, cfg.head_dim), generator=g)
    return [x.to(TORCH_DTYPE[cfg.dtype]).to(device).contiguous() for x in q.to(torch.float32)]
