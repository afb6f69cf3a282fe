"""The C-ABI library loads, exports every symbol its header declares, and
rejects bad arguments before touching a GPU (no compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "oasis.h")


@pytest.fixture(scope="module")
def L():
    from sparse_kv_block_amd import lib
    return lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(oasis_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) == 19
    so = ctypes.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(so, n), n
    assert sorted(L.SYMBOLS) == names


def test_version_and_helpers(L, ora):
    raw = L.raw()
    assert raw.oasis_abi_version() == 8
    for cap, K in [(0.0, 128), (0.01, 128), (0.05, 128), (0.2, 128), (1.0, 128), (0.25, 8),
                   (2.0, 16), (-1.0, 8), (0.3, 10), (0.7, 10)]:
        assert L.cap_to_max_admit(cap, K) == ora.max_admit(cap, K), (cap, K)
    s = L.Shape(128, 32, 8, 128, 16, 1024, 128, L.BF16)
    assert L.record_bytes(s) == 8192
    assert raw.oasis_summary_bytes(ctypes.byref(s)) == 128 * 8 * 1024 * 512


def shape(**kw):
    from sparse_kv_block_amd import lib
    base = dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16, max_blocks=64,
                k_resident=8, dtype=lib.BF16)
    base.update(kw)
    return lib.Shape(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(n_q_heads=6, n_kv_heads=4), 1),
    (dict(n_kv_heads=0), 1),
    (dict(batch=-1), 1),
    (dict(max_blocks=0), 1),
    (dict(k_resident=0), 1),
    (dict(head_dim=96), 2),
    (dict(block_size=32), 2),
    (dict(max_blocks=8193), 2),
    (dict(k_resident=257), 2),
    (dict(n_q_heads=34, n_kv_heads=2), 2),
    (dict(dtype=7), 2),
    (dict(batch=(1 << 21) + 1, n_kv_heads=2, n_q_heads=2), 2),     # more than 2^22 units
])
def test_bad_shapes_are_rejected(L, kw, status):
    raw = L.raw()
    s = shape(**kw)
    p = ctypes.c_void_p(16)   # never dereferenced: validation fails first
    assert raw.oasis_summarize(ctypes.byref(s), p, p, p, None) == status
    assert "oasis_summarize" in L.last_error()
    assert raw.oasis_score_topk(ctypes.byref(s), p, 1, p, p, p, p, None, 0, None) == status
    assert raw.oasis_layer_step(ctypes.byref(s), p, p, p, p, 0.0, 1, 6, p, p, p, p, p, p, p, p,
                                p, 1 << 30, None) == status


def test_null_pointers_and_bad_scalars(L):
    raw = L.raw()
    s = shape()
    p = ctypes.c_void_p(16)
    assert raw.oasis_summarize(None, p, p, p, None) == L.ERR_INVALID
    assert raw.oasis_summarize(ctypes.byref(s), None, p, p, None) == L.ERR_INVALID
    assert "records is NULL" in L.last_error()
    assert raw.oasis_exact_topk(ctypes.byref(s), p, 2, p, p, p, p, None) == L.ERR_INVALID
    assert "q_row" in L.last_error()
    assert raw.oasis_topk_agreement(ctypes.byref(s), p, None, p, 4, p, None) == L.ERR_INVALID
    assert "exact_idx is NULL" in L.last_error()
    assert raw.oasis_topk_agreement(ctypes.byref(s), p, p, p, 9, p, None) == L.ERR_INVALID
    assert "exact_n" in L.last_error()
    assert raw.oasis_score_topk(ctypes.byref(s), p, 2, p, p, p, p, None, 0, None) == L.ERR_INVALID
    assert raw.oasis_capped_evict(ctypes.byref(s), p, 1, -1, p, p, p, p, p, None) == L.ERR_INVALID
    assert raw.oasis_lookahead_attn(ctypes.byref(s), p, p, p, p, float("nan"), p, None) == L.ERR_INVALID
    assert raw.oasis_prefetch(ctypes.byref(s), p, p, p, p, 6, 5, None, None, None, None) == L.ERR_INVALID
    assert raw.oasis_prefetch(ctypes.byref(s), p, p, p, p, 6, L.MEMCPY, None, None, None,
                              None) == L.ERR_INVALID
    assert "host_staging" in L.last_error()
    assert raw.oasis_append_token(ctypes.byref(s), p, p, p, p, None, p, p, None) == L.ERR_INVALID
    assert "both" in L.last_error()
    assert raw.oasis_append_token(ctypes.byref(s), p, p, None, None, None, p, p, None) == L.ERR_INVALID
    assert "records is NULL" in L.last_error()


def test_empty_batch_is_a_no_op(L):
    raw = L.raw()
    s = shape(batch=0)
    assert raw.oasis_summarize(ctypes.byref(s), None, None, None, None) == L.OK
    assert raw.oasis_append_token(ctypes.byref(s), *([None] * 7), None) == L.OK
    assert raw.oasis_layer_step(ctypes.byref(s), *([None] * 4), 0.0, 1, 6, *([None] * 8), None, 0,
                                None) == L.OK


def test_layer_step_workspace_contract(L):
    raw = L.raw()
    short = shape(max_blocks=1024, k_resident=128, batch=4)
    assert L.layer_step_workspace_bytes(short) == 0
    long = shape(max_blocks=8192, k_resident=128, batch=64, n_kv_heads=8, n_q_heads=32)
    need = L.layer_step_workspace_bytes(long)
    parts, units = 1 + 8192 // 1024, 64 * 8          # attention part + 1024-block scan parts
    # per unit: every part's list (keys and block indices), the last part's
    # 1024 unselected keys and the arrival word
    assert need >= units * (2 * parts * 128 * 4 + 1024 * 4 + 8)
    assert need < 7 * 2**20
    p = ctypes.c_void_p(4096)
    args = [p] * 4 + [0.0, 1, 6] + [p] * 8
    assert raw.oasis_layer_step(ctypes.byref(long), *args, None, need, None) == L.ERR_INVALID
    assert "workspace is NULL" in L.last_error()
    assert raw.oasis_layer_step(ctypes.byref(long), *args, p, need - 1, None) == L.ERR_INVALID
    assert "needed" in L.last_error()
    assert raw.oasis_layer_step(ctypes.byref(long), *args, ctypes.c_void_p(4096 + 16), need,
                                None) == L.ERR_INVALID
    assert "aligned" in L.last_error()


def test_binding_refuses_cpu_tensors(L):
    import torch
    s = shape(batch=1, n_q_heads=2, n_kv_heads=1, head_dim=64, max_blocks=4, k_resident=2, dtype=L.F32)
    x = torch.zeros(1 * 4 * 2 * 16 * 64)
    with pytest.raises(ValueError):
        L.summarize(s, torch.zeros(4 * 2 * 16 * 64 + 1), torch.zeros(1, dtype=torch.int32),
                    torch.zeros(4 * 2 * 64))
    with pytest.raises(ValueError):
        L.lookahead_attn(s, torch.zeros(1 * 2 * 2 * 64), x, torch.zeros(2, dtype=torch.int32),
                         torch.zeros(1, dtype=torch.int32), torch.zeros(256))
