"""The host-link budget model (host arithmetic only)."""
import math

from sparse_kv_block_amd import capmodel as cm


def test_bytes_per_step_matches_the_pages_cap_001_figure():
    # agihunt.info summary, fetch-cap ablation: 0.30 GB per step at cap 0.01.
    # 36 layers x 128 requests x 8 KV heads, one 8 KiB bf16 record per admission
    # (m = floor(0.01 * 128) = 1).
    b = cm.bytes_per_step(36, 128 * 8, 1, 2 * 16 * 128 * 2)
    assert b == 301_989_888
    assert round(b / 1e9, 2) == 0.30


def test_largest_hidden_admit():
    # 10 GB/s for 1 ms moves 10 MB; one admission per unit of 10 units x 1
    # layer x 100 kB is 1 MB, so 10 fit; clamped to K.
    assert cm.largest_hidden_admit(10e9, 1e-3, 1, 10, 100_000, 128) == 10
    assert cm.largest_hidden_admit(10e9, 1e-3, 1, 10, 100_000, 4) == 4
    assert cm.largest_hidden_admit(10e9, 0.99e-3, 1, 10, 100_000, 128) == 9
    assert cm.largest_hidden_admit(0.0, 1e-3, 1, 10, 100_000, 128) == 0
    # the quota that hides moves no more than the window allows, one more would not
    bw, win, L, U, rec = 55.9e9, 36 * 275e-6, 36, 1024, 8192
    m = cm.largest_hidden_admit(bw, win, L, U, rec, 128)
    assert cm.bytes_per_step(L, U, m, rec) / bw <= win < cm.bytes_per_step(L, U, m + 1, rec) / bw


def test_predicted_step():
    assert cm.predicted_step_s(1.0, 5e9, 10e9) == 1.0
    assert cm.predicted_step_s(1.0, 20e9, 10e9) == 2.0
    assert cm.predicted_step_s(1.0, 20e9, 10e9, overlap=False) == 3.0
    assert math.isinf(cm.predicted_step_s(1.0, 1.0, 0.0))
