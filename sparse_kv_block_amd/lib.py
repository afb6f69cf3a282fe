"""Thin ctypes binding over liboasis.so (include/oasis.h).

Argument marshalling only: it checks tensor devices, dtypes, contiguity and
sizes against the shape (so that no kernel is launched over a buffer smaller
than its grid assumes), then passes raw pointers and the current HIP stream.
Every step runs in the HIP library; there is no fallback.  Importing this
module raises if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from .configs import Config

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("OASIS_LIBRARY") or os.path.join(PKG, "liboasis.so")

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_HIP = 0, 1, 2, 3
F32, BF16 = 0, 1
GATHER, MEMCPY = 0, 1

# every symbol include/oasis.h declares
SYMBOLS = ("oasis_abi_version", "oasis_last_error", "oasis_cap_to_max_admit",
           "oasis_record_bytes", "oasis_summary_bytes", "oasis_host_to_device_ptr",
           "oasis_summarize", "oasis_lookahead_attn", "oasis_score_topk",
           "oasis_capped_evict", "oasis_prefetch", "oasis_layer_step",
           "oasis_layer_step_workspace_bytes", "oasis_dense_attn", "oasis_dense_attn_workspace_bytes",
           "oasis_append_token", "oasis_exact_topk", "oasis_topk_agreement",
           "oasis_layer_step_noalloc")


class OasisError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[oasis status {status}] {msg}")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
                ("k_resident", ctypes.c_int32), ("dtype", ctypes.c_int32)]

    @staticmethod
    def of(cfg: Config, max_blocks: int, batch: Optional[int] = None) -> "Shape":
        return Shape(cfg.batch if batch is None else batch, cfg.n_q_heads, cfg.n_kv_heads,
                     cfg.head_dim, cfg.block_size, max_blocks, cfg.k_resident,
                     F32 if cfg.dtype == "f32" else BF16)

    def units(self) -> int:
        return self.batch * self.n_kv_heads

    def torch_dtype(self):
        return torch.float32 if self.dtype == F32 else torch.bfloat16

    def record_elems(self) -> int:
        return 2 * self.block_size * self.head_dim


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run `python -m sparse_kv_block_amd.build` "
                          "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    SP = ctypes.POINTER(Shape)
    sig = {
        "oasis_abi_version": ([], I32),
        "oasis_last_error": ([], ctypes.c_char_p),
        "oasis_cap_to_max_admit": ([ctypes.c_double, I32], I32),
        "oasis_record_bytes": ([SP], ctypes.c_size_t),
        "oasis_summary_bytes": ([SP], ctypes.c_size_t),
        "oasis_host_to_device_ptr": ([P, ctypes.POINTER(P)], I32),
        "oasis_summarize": ([SP, P, P, P, P], I32),
        "oasis_lookahead_attn": ([SP, P, P, P, P, F, P, P], I32),
        "oasis_score_topk": ([SP, P, I32, P, P, P, P, P, ctypes.c_size_t, P], I32),
        "oasis_capped_evict": ([SP, P, I32, I32, P, P, P, P, P, P], I32),
        "oasis_prefetch": ([SP, P, P, P, P, I32, I32, P, P, P, P], I32),
        "oasis_layer_step": ([SP, P, P, P, P, F, I32, I32, P, P, P, P, P, P, P, P, P,
                              ctypes.c_size_t, P], I32),
        "oasis_layer_step_workspace_bytes": ([SP], ctypes.c_size_t),
        "oasis_layer_step_noalloc": ([SP, P, P, P, P, F, I32, I32, P, P, P, P, P, P, P, P, P], I32),
        "oasis_dense_attn": ([SP, P, P, P, F, P, P, ctypes.c_size_t, P], I32),
        "oasis_dense_attn_workspace_bytes": ([SP], ctypes.c_size_t),
        "oasis_append_token": ([SP, P, P, P, P, P, P, P, P], I32),
        "oasis_exact_topk": ([SP, P, I32, P, P, P, P, P], I32),
        "oasis_topk_agreement": ([SP, P, P, P, I32, P, P], I32),
    }
    for name, (args, res) in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    return L


_lib = _load()


def raw():
    return _lib


def last_error() -> str:
    return _lib.oasis_last_error().decode()


def _check(status: int):
    if status != OK:
        raise OasisError(status, last_error())


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, name: str, dtype, numel: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, the shape needs {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _any(t: torch.Tensor, name: str, dtype, numel: int):
    """A device tensor, or a pinned host tensor passed through its device mapping."""
    if isinstance(t, torch.Tensor) and t.device.type == "cpu":
        if t.dtype != dtype or not t.is_contiguous() or t.numel() != numel:
            raise ValueError(f"{name}: wrong dtype, layout or size")
        if not t.is_pinned():
            raise ValueError(f"{name}: host memory must be pinned")
        return ctypes.c_void_p(host_device_ptr(t))
    return _dev(t, name, dtype, numel)


def host_device_ptr(t: torch.Tensor) -> int:
    out = ctypes.c_void_p()
    _check(_lib.oasis_host_to_device_ptr(ctypes.c_void_p(t.data_ptr()), ctypes.byref(out)))
    return out.value


def cap_to_max_admit(cap: float, k_resident: int) -> int:
    return int(_lib.oasis_cap_to_max_admit(float(cap), int(k_resident)))


def record_bytes(shape: Shape) -> int:
    return int(_lib.oasis_record_bytes(ctypes.byref(shape)))


I32 = torch.int32


def summarize(shape: Shape, records, ctx_len, summ, stream=None):
    dt, U, NB, d = shape.torch_dtype(), shape.units(), shape.max_blocks, shape.head_dim
    _check(_lib.oasis_summarize(
        ctypes.byref(shape), _any(records, "records", dt, U * NB * shape.record_elems()),
        _dev(ctx_len, "ctx_len", I32, shape.batch), _dev(summ, "summ", dt, U * NB * 2 * d),
        _stream(stream)))


def append_token(shape: Shape, k_new, v_new, records, summ, ctx_len, pool=None, l2p=None,
                 stream=None):
    """Decode append of one token per request (see oasis_append_token)."""
    dt, U, NB, d = shape.torch_dtype(), shape.units(), shape.max_blocks, shape.head_dim
    if (pool is None) != (l2p is None):
        raise ValueError("pool and l2p must both be given or both be None")
    pp = None if pool is None else _dev(pool, "pool", dt, U * shape.k_resident * shape.record_elems())
    lp = None if l2p is None else _dev(l2p, "l2p", I32, U * NB)
    _check(_lib.oasis_append_token(
        ctypes.byref(shape), _dev(k_new, "k_new", dt, U * d), _dev(v_new, "v_new", dt, U * d),
        _any(records, "records", dt, U * NB * shape.record_elems()), pp, lp,
        _dev(summ, "summ", dt, U * NB * 2 * d), _dev(ctx_len, "ctx_len", I32, shape.batch),
        _stream(stream)))


def lookahead_attn(shape: Shape, q, pool, p2l, ctx_len, out, scale: float = 0.0, stream=None):
    dt, U, K, d = shape.torch_dtype(), shape.units(), shape.k_resident, shape.head_dim
    qn = shape.batch * 2 * shape.n_q_heads * d
    _check(_lib.oasis_lookahead_attn(
        ctypes.byref(shape), _dev(q, "q", dt, qn), _dev(pool, "pool", dt, U * K * shape.record_elems()),
        _dev(p2l, "p2l", I32, U * K), _dev(ctx_len, "ctx_len", I32, shape.batch), float(scale),
        _dev(out, "out", dt, qn), _stream(stream)))


def score_topk(shape: Shape, q, summ, ctx_len, topk_idx, topk_score, q_row: int = 1, stream=None,
               workspace=None):
    """Summary scan + top-K (see oasis_score_topk); `workspace` as for layer_step
    (needed when max_blocks exceeds one 1024-block scan part)."""
    dt, U, K, d = shape.torch_dtype(), shape.units(), shape.k_resident, shape.head_dim
    _check(_lib.oasis_score_topk(
        ctypes.byref(shape), _dev(q, "q", dt, shape.batch * 2 * shape.n_q_heads * d), int(q_row),
        _dev(summ, "summ", dt, U * shape.max_blocks * 2 * d),
        _dev(ctx_len, "ctx_len", I32, shape.batch), _dev(topk_idx, "topk_idx", I32, U * K),
        _dev(topk_score, "topk_score", torch.float32, U * K), *_workspace(shape, workspace),
        _stream(stream)))


def exact_topk(shape: Shape, q, records, ctx_len, topk_idx, topk_score, q_row: int = 0,
               stream=None):
    """Top-K of the exact block scores (see oasis_exact_topk)."""
    dt, U, K, d = shape.torch_dtype(), shape.units(), shape.k_resident, shape.head_dim
    _check(_lib.oasis_exact_topk(
        ctypes.byref(shape), _dev(q, "q", dt, shape.batch * 2 * shape.n_q_heads * d), int(q_row),
        _any(records, "records", dt, U * shape.max_blocks * shape.record_elems()),
        _dev(ctx_len, "ctx_len", I32, shape.batch), _dev(topk_idx, "topk_idx", I32, U * K),
        _dev(topk_score, "topk_score", torch.float32, U * K), _stream(stream)))


def topk_agreement(shape: Shape, pred_idx, exact_idx, counts, l2p=None,
                   exact_n: Optional[int] = None, stream=None):
    """Per-unit (n_exact, agreeing, resident) counts over the first exact_n
    entries of the exact list (all K by default; see oasis_topk_agreement)."""
    U, K = shape.units(), shape.k_resident
    lp = None if l2p is None else _dev(l2p, "l2p", I32, U * shape.max_blocks)
    _check(_lib.oasis_topk_agreement(
        ctypes.byref(shape), _dev(pred_idx, "pred_idx", I32, U * K),
        _dev(exact_idx, "exact_idx", I32, U * K), lp, int(K if exact_n is None else exact_n),
        _dev(counts, "counts", I32, U * 3), _stream(stream)))


def capped_evict(shape: Shape, topk_idx, step: int, max_admit: int, l2p, p2l, last_sel, admit,
                 admit_count, stream=None):
    U, K = shape.units(), shape.k_resident
    _check(_lib.oasis_capped_evict(
        ctypes.byref(shape), _dev(topk_idx, "topk_idx", I32, U * K), int(step), int(max_admit),
        _dev(l2p, "l2p", I32, U * shape.max_blocks), _dev(p2l, "p2l", I32, U * K),
        _dev(last_sel, "last_sel", I32, U * K), _dev(admit, "admit", I32, U * K * 3),
        _dev(admit_count, "admit_count", I32, U), _stream(stream)))


def prefetch(shape: Shape, records, pool, admit, admit_count, max_admit: int, mode: int = GATHER,
             host_staging=None, side_stream=None, wait_before=None, done=None):
    dt, U, K = shape.torch_dtype(), shape.units(), shape.k_resident
    stg = None
    if mode == MEMCPY:
        n = U * (3 * K + 1)
        if (host_staging is None or host_staging.device.type != "cpu" or not host_staging.is_pinned()
                or host_staging.dtype != I32 or host_staging.numel() < n):
            raise ValueError(f"MEMCPY mode needs a pinned int32 host_staging of >= {n} elements")
        stg = ctypes.c_void_p(host_staging.data_ptr())
    side = torch.cuda.current_stream() if side_stream is None else side_stream
    # torch creates an event's hipEvent_t only when torch first records it: an
    # event torch never recorded has handle 0.  `wait_before` in that state
    # has nothing to wait for; `done` is created here (recorded once on the
    # side stream) so that the library can record it and waiters see it.
    wait = None
    if wait_before is not None and wait_before.cuda_event:
        wait = ctypes.c_void_p(wait_before.cuda_event)
    fin = None
    if done is not None:
        if not done.cuda_event:
            done.record(side)
        if not done.cuda_event:
            raise RuntimeError("could not create the completion event")
        fin = ctypes.c_void_p(done.cuda_event)
    _check(_lib.oasis_prefetch(
        ctypes.byref(shape), _any(records, "records", dt, U * shape.max_blocks * shape.record_elems()),
        _dev(pool, "pool", dt, U * K * shape.record_elems()), _dev(admit, "admit", I32, U * K * 3),
        _dev(admit_count, "admit_count", I32, U), int(max_admit), int(mode), stg,
        _stream(side), wait, fin))


def _workspace(shape: Shape, ws):
    need = layer_step_workspace_bytes(shape)
    if need == 0:
        return None, 0
    if ws is None:
        raise ValueError(f"this shape needs a {need}-byte layer-step workspace")
    if ws.device.type != "cuda" or not ws.is_contiguous() or ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace must be a contiguous device tensor of >= {need} bytes")
    return ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size()


def layer_step_workspace_bytes(shape: Shape) -> int:
    return int(_lib.oasis_layer_step_workspace_bytes(ctypes.byref(shape)))


def layer_step_workspace(shape: Shape, device="cuda"):
    """A zero-filled workspace for layer_step (None when the shape needs none)."""
    n = layer_step_workspace_bytes(shape)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def layer_step(shape: Shape, q, pool, summ, ctx_len, step: int, max_admit: int, out, topk_idx,
               topk_score, l2p, p2l, last_sel, admit, admit_count, scale: float = 0.0, stream=None,
               workspace=None):
    dt, U, K, d = shape.torch_dtype(), shape.units(), shape.k_resident, shape.head_dim
    qn = shape.batch * 2 * shape.n_q_heads * d
    _check(_lib.oasis_layer_step(
        ctypes.byref(shape), _dev(q, "q", dt, qn), _dev(pool, "pool", dt, U * K * shape.record_elems()),
        _dev(summ, "summ", dt, U * shape.max_blocks * 2 * d), _dev(ctx_len, "ctx_len", I32, shape.batch),
        float(scale), int(step), int(max_admit), _dev(out, "out", dt, qn),
        _dev(topk_idx, "topk_idx", I32, U * K), _dev(topk_score, "topk_score", torch.float32, U * K),
        _dev(l2p, "l2p", I32, U * shape.max_blocks), _dev(p2l, "p2l", I32, U * K),
        _dev(last_sel, "last_sel", I32, U * K), _dev(admit, "admit", I32, U * K * 3),
        _dev(admit_count, "admit_count", I32, U), *_workspace(shape, workspace), _stream(stream)))


def layer_step_noalloc(shape: Shape, q, pool, summ, ctx_len, step: int, max_admit: int, out,
                       topk_idx, topk_score, l2p, p2l, last_sel, admit, admit_count,
                       scale: float = 0.0, stream=None):
    """The fused step with the library's own device scratch (no workspace; see
    oasis_layer_step_noalloc)."""
    dt, U, K, d = shape.torch_dtype(), shape.units(), shape.k_resident, shape.head_dim
    qn = shape.batch * 2 * shape.n_q_heads * d
    _check(_lib.oasis_layer_step_noalloc(
        ctypes.byref(shape), _dev(q, "q", dt, qn), _dev(pool, "pool", dt, U * K * shape.record_elems()),
        _dev(summ, "summ", dt, U * shape.max_blocks * 2 * d), _dev(ctx_len, "ctx_len", I32, shape.batch),
        float(scale), int(step), int(max_admit), _dev(out, "out", dt, qn),
        _dev(topk_idx, "topk_idx", I32, U * K), _dev(topk_score, "topk_score", torch.float32, U * K),
        _dev(l2p, "l2p", I32, U * shape.max_blocks), _dev(p2l, "p2l", I32, U * K),
        _dev(last_sel, "last_sel", I32, U * K), _dev(admit, "admit", I32, U * K * 3),
        _dev(admit_count, "admit_count", I32, U), _stream(stream)))


def dense_attn_workspace(shape: Shape, device="cuda"):
    n = int(_lib.oasis_dense_attn_workspace_bytes(ctypes.byref(shape)))
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def dense_attn(shape: Shape, q, records, ctx_len, out, workspace, scale: float = 0.0, stream=None):
    """Dense comparator: attention over every valid token of `records` (device)."""
    dt, U, d = shape.torch_dtype(), shape.units(), shape.head_dim
    qn = shape.batch * 2 * shape.n_q_heads * d
    need = int(_lib.oasis_dense_attn_workspace_bytes(ctypes.byref(shape)))
    if workspace.device.type != "cuda" or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"dense attention needs a device workspace of >= {need} bytes")
    _check(_lib.oasis_dense_attn(
        ctypes.byref(shape), _dev(q, "q", dt, qn),
        _dev(records, "records", dt, U * shape.max_blocks * shape.record_elems()),
        _dev(ctx_len, "ctx_len", I32, shape.batch), float(scale), _dev(out, "out", dt, qn),
        ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
        _stream(stream)))
