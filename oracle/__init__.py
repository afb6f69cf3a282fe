"""Python handle on the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg use it; the product path never does.  It takes numpy arrays (or
CPU torch tensors), and bf16 data as raw uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16 = 0, 1


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so (no GPU code involved)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-shared", "-fPIC",
             os.path.join(_HERE, "oracle.c"), "-o", tmp, "-lpthread", "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def load(path: str):
    """Opens a build of oracle.c and declares its functions' signatures."""
    L = ctypes.CDLL(path)
    P, I, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
    L.ora_summarize.argtypes = [I, I, I, I, I, I, P, P, P, P, I, I]
    L.ora_block_scores.argtypes = [I, I, I, I, I, I, I, P, I, P, P, P, P, I, I]
    L.ora_topk.argtypes = [I, I, I, I, I, P, P, P, P, P, I]
    L.ora_max_admit.argtypes = [D, I]
    L.ora_max_admit.restype = I
    L.ora_capped_evict.argtypes = [I, I, I, I, P, ctypes.c_int32, ctypes.c_int32,
                                   P, P, P, P, P, P, I]
    L.ora_attention.argtypes = [I, I, I, I, I, I, I, I, P, P, P, P, D, P, P, I, I]
    L.ora_prefetch.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, I]
    L.ora_append.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P]
    L.ora_exact_block_scores.argtypes = [I, I, I, I, I, I, I, P, I, P, P, P, P, I, I]
    for f in (L.ora_summarize, L.ora_block_scores, L.ora_topk, L.ora_capped_evict,
              L.ora_attention, L.ora_prefetch, L.ora_append, L.ora_exact_block_scores):
        f.restype = None
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = load(LIB_PATH)
    return _lib


# ---------------------------------------------------------------------------
def as_np(x) -> np.ndarray:
    """numpy view of a CPU tensor or array; bf16 becomes its uint16 bit pattern."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach()
            if x.device.type != "cpu":
                x = x.cpu()
            if x.dtype == torch.bfloat16:
                return x.contiguous().view(torch.int16).numpy().view(np.uint16)
            return x.contiguous().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(x)


def dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle takes float32 or bf16 bit patterns, got {a.dtype}")


def bf16_to_f64(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_f64(a: np.ndarray) -> np.ndarray:
    return bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _units(units: Optional[Sequence[int]]):
    if units is None:
        return None, 0
    u = np.ascontiguousarray(np.asarray(units, dtype=np.int32))
    return u, len(u)


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# ---------------------------------------------------------------------------
def summarize(records, ctx_len, block_size: int, summ=None, units=None, nthreads=None):
    rec = as_np(records)
    B, H, NB, E = rec.shape
    S = block_size
    d = E // (2 * S)
    ctx = np.ascontiguousarray(as_np(ctx_len).astype(np.int32))
    if summ is None:
        summ = np.zeros((B, H, NB, 2, d), dtype=rec.dtype)
    u, nu = _units(units)
    lib().ora_summarize(B, H, NB, S, d, dtype_code(rec), _ptr(rec), _ptr(ctx), _ptr(summ),
                        _ptr(u), nu, nthreads or default_threads())
    return summ


def block_scores(q, summ, ctx_len, block_size: int, q_row: int = 1, units=None,
                 nthreads=None, scores=None):
    qa, sa = as_np(q), as_np(summ)
    B, H, NB, _, d = sa.shape
    Hq = qa.shape[2]
    ctx = np.ascontiguousarray(as_np(ctx_len).astype(np.int32))
    if scores is None:
        scores = np.full((B, H, NB), np.nan, dtype=np.float64)
    u, nu = _units(units)
    lib().ora_block_scores(B, Hq, H, NB, block_size, d, dtype_code(sa), _ptr(qa), q_row,
                           _ptr(sa), _ptr(ctx), _ptr(scores), _ptr(u), nu,
                           nthreads or default_threads())
    return scores


def exact_block_scores(q, records, ctx_len, block_size: int, q_row: int = 0, units=None,
                       nthreads=None, scores=None):
    """Exact block scores from the keys: sum over the KV head's query heads of
    the largest logit over the block's valid tokens ([B][H][NBmax], -inf past
    the context)."""
    qa, rec = as_np(q), as_np(records)
    B, H, NB, E = rec.shape
    d = E // (2 * block_size)
    Hq = qa.shape[2]
    ctx = np.ascontiguousarray(as_np(ctx_len).astype(np.int32))
    if scores is None:
        scores = np.full((B, H, NB), np.nan, dtype=np.float64)
    u, nu = _units(units)
    lib().ora_exact_block_scores(B, Hq, H, NB, block_size, d, dtype_code(rec), _ptr(qa), q_row,
                                 _ptr(rec), _ptr(ctx), _ptr(scores), _ptr(u), nu,
                                 nthreads or default_threads())
    return scores


def agreement(pred_idx, exact_idx, l2p=None, exact_n=None):
    """Per unit (n_exact, |pred & exact|, |exact & resident|) over the first
    exact_n entries of the exact top-K list (all by default): its valid
    entries, how many of them the predicted list holds, and how many are
    resident by the slot map l2p (-1 where l2p is None)."""
    P = np.asarray(as_np(pred_idx), np.int64)
    X = np.asarray(as_np(exact_idx), np.int64)
    if exact_n is not None:
        X = X[..., :exact_n]
    B, H, _ = X.shape
    out = np.zeros((B, H, 3), np.int32)
    for b in range(B):
        for h in range(H):
            ex = {int(j) for j in X[b, h] if j >= 0}
            pr = {int(j) for j in P[b, h] if j >= 0}
            out[b, h, 0] = len(ex)
            out[b, h, 1] = len(ex & pr)
            if l2p is None:
                out[b, h, 2] = -1
            else:
                lp = as_np(l2p)[b, h]
                out[b, h, 2] = sum(1 for j in ex if lp[j] >= 0)
    return out


def topk(scores, ctx_len, block_size: int, K: int, units=None, idx=None, val=None):
    sc = np.ascontiguousarray(scores, dtype=np.float64)
    B, H, NB = sc.shape
    ctx = np.ascontiguousarray(as_np(ctx_len).astype(np.int32))
    if idx is None:
        idx = np.full((B, H, K), -1, dtype=np.int32)
    if val is None:
        val = np.full((B, H, K), -np.inf, dtype=np.float64)
    u, nu = _units(units)
    lib().ora_topk(B, H, NB, block_size, K, _ptr(sc), _ptr(ctx), _ptr(idx), _ptr(val),
                   _ptr(u), nu)
    return idx, val


def max_admit(cap: float, K: int) -> int:
    return int(lib().ora_max_admit(float(cap), int(K)))


def capped_evict(topk_idx, step: int, max_admit_: int, l2p, p2l, last_sel, units=None):
    """In-place on the given int32 numpy arrays; returns (admit, admit_count)."""
    T = np.ascontiguousarray(as_np(topk_idx), dtype=np.int32)
    for a in (l2p, p2l, last_sel):
        assert isinstance(a, np.ndarray) and a.dtype == np.int32 and a.flags.c_contiguous
    B, H, K = p2l.shape
    NB = l2p.shape[2]
    admit = np.full((B, H, K, 3), -1, dtype=np.int32)
    count = np.zeros((B, H), dtype=np.int32)
    u, nu = _units(units)
    lib().ora_capped_evict(B, H, NB, K, _ptr(T), int(step), int(max_admit_), _ptr(l2p),
                           _ptr(p2l), _ptr(last_sel), _ptr(admit), _ptr(count), _ptr(u), nu)
    return admit, count


def attention(q, records, p2l, ctx_len, block_size: int, scale: Optional[float] = None,
              units=None, nthreads=None, out=None):
    qa, rec = as_np(q), as_np(records)
    B, _, Hq, d = qa.shape
    H, NB = rec.shape[1], rec.shape[2]
    pa = np.ascontiguousarray(as_np(p2l), dtype=np.int32)
    K = pa.shape[2]
    ctx = np.ascontiguousarray(as_np(ctx_len).astype(np.int32))
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if out is None:
        out = np.full((B, 2, Hq, d), np.nan, dtype=np.float64)
    u, nu = _units(units)
    lib().ora_attention(B, Hq, H, NB, block_size, d, K, dtype_code(qa), _ptr(qa), _ptr(rec),
                        _ptr(pa), _ptr(ctx), float(scale), _ptr(out), _ptr(u), nu,
                        nthreads or default_threads())
    return out


def prefetch(records, pool, admit, admit_count, block_size: int, units=None):
    """Copies admitted records into `pool` (a numpy array, modified in place)."""
    rec = as_np(records)
    B, H, NB, E = rec.shape
    d = E // (2 * block_size)
    K = pool.shape[2]
    ad = np.ascontiguousarray(as_np(admit), dtype=np.int32)
    ac = np.ascontiguousarray(as_np(admit_count), dtype=np.int32)
    u, nu = _units(units)
    lib().ora_prefetch(B, H, NB, block_size, d, K, dtype_code(rec), _ptr(rec), _ptr(pool),
                       _ptr(ad), _ptr(ac), _ptr(u), nu)
    return pool


def append(k_new, v_new, records, summ, ctx_len, block_size: int, pool=None, l2p=None):
    """In place on the numpy arrays records, summ, ctx_len (and pool)."""
    kn, vn = as_np(k_new), as_np(v_new)
    for a in (records, summ, ctx_len):
        assert isinstance(a, np.ndarray) and a.flags.c_contiguous
    B, H, NB, E = records.shape
    d = E // (2 * block_size)
    K = pool.shape[2] if pool is not None else 0
    l2 = None if l2p is None else np.ascontiguousarray(l2p, dtype=np.int32)
    lib().ora_append(B, H, NB, block_size, d, K, dtype_code(records), _ptr(kn), _ptr(vn),
                     _ptr(records), _ptr(pool), _ptr(l2), _ptr(summ), _ptr(ctx_len))


def layer_step(q, records, summ, ctx_len, block_size: int, K: int, step: int,
               max_admit_: int, l2p, p2l, last_sel, scale=None, units=None, nthreads=None):
    """One look-ahead layer step in the order the method runs it: attention of
    both rows over the current resident set, then the draft scores, top-K and
    capped eviction.  Returns (out, topk_idx, topk_score, admit, admit_count)."""
    out = attention(q, records, p2l, ctx_len, block_size, scale, units, nthreads)
    sc = block_scores(q, summ, ctx_len, block_size, 1, units, nthreads)
    idx, val = topk(sc, ctx_len, block_size, K, units)
    admit, count = capped_evict(idx, step, max_admit_, l2p, p2l, last_sel, units)
    return out, idx, val, admit, count
