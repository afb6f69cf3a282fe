"""bench.py's command-line contract: one GPU only, and the single JSON line it
prints (metric, value, roofline and CPU-oracle objects).  The GPU case runs a
short bench in a child process."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_algorithmic_bytes_of_the_16k_layer_step():
    sys.path.insert(0, ROOT)
    import bench
    from sparse_kv_block_amd import gen
    from sparse_kv_block_amd.configs import QWEN3_8B_16K
    algo = bench.algorithmic_bytes(QWEN3_8B_16K, gen.context_lengths(QWEN3_8B_16K))
    # resident KV + summaries + q/out + maps + context lengths, one launch; per
    # unit the maps move p2l and stamps read and written (4 K ints), 2m slot
    # updates, K (index, score) pairs, K admission triples and their count
    # (residency comes from p2l: no slot lookup per top-K entry)
    K, m = 128, 6
    maps_per_unit = 4 * K * 4 + 2 * m * 4 + K * 8 + K * 12 + 4
    assert maps_per_unit == 4_660
    assert algo["total"] == 1_073_741_824 + 536_870_912 + 4_194_304 + 1024 * maps_per_unit + 512
    assert bench.kernel_name(QWEN3_8B_16K) == "layer_step_kernel<bf16, d=128, 1 row tile>"


@pytest.mark.gpu
def test_bench_prints_one_json_line_with_roofline_and_oracle_baseline():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "5", "--warmup", "5",
           "--settle-seconds", "0", "--no-pcie", "--cpu-seconds", "1"]
    print("[bench contract]", " ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, lines
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 5
    assert d["unit"] == "layer-steps/s" and d["value"] > 0 and d["higher_is_better"] is True
    assert d["config"]["workload"].startswith("qwen3_8b_16k")
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert 0 < rf["frac"] < 1
    assert d["achievable"]["copy_GBps"] > 0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    assert cb["single_thread"]["value"] > 0 and cb["cpu_model"]
