"""bench.py's command-line contract on the CPU: more than one GPU is refused
with a message before anything touches a GPU, and the measurement helpers
behave (FLOP count, kernel-code hash)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n],
                             capture_output=True, text=True, timeout=60)
        assert res.returncode == 2
        assert "one GPU" in res.stderr
        assert res.stdout == ""


def test_prefill_flop_count():
    sys.path.insert(0, ROOT)
    import bench

    # 4*B*H*Sq*Sk*D, halved when causal: 1.374e11 at the LLaMA-7B shape
    assert bench.prefill_flops(1, 32, 4096, 4096, 128, True) == 4.0 * 32 * 4096 * 4096 * 128 / 2
    assert bench.prefill_flops(8, 16, 256, 256, 64, False) == 4.0 * 8 * 16 * 256 * 256 * 64


def test_kernel_hash_ignores_comments(tmp_path, monkeypatch):
    # the stored counter figures stay valid across comment edits and are
    # retired by any code change
    import shutil

    sys.path.insert(0, ROOT)
    import bench

    csrc = tmp_path / "exact_attention_54_amd" / "csrc"
    shutil.copytree(os.path.join(ROOT, "exact_attention_54_amd", "csrc"), csrc)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    with open(csrc / "fa_device.hpp", "a") as f:
        f.write("\n// a new comment line\n\n   \n")
    assert bench.kernel_source_hash() == h0
    with open(csrc / "fa_device.hpp", "a") as f:
        f.write("constexpr int kUnused = 1;  // code\n")
    assert bench.kernel_source_hash() != h0


def test_cpu_baseline_fields_on_a_tiny_sample():
    # the oracle leg records what it ran on: CPU model, affinity cores, BLAS
    # threads (set before numpy's import), and the median of three runs when
    # a run is short
    from types import SimpleNamespace

    import numpy as np

    sys.path.insert(0, ROOT)
    import bench

    g = np.random.default_rng(0)
    w3 = SimpleNamespace(B=1, H=2, Sq=64, Sk=64, D=32, scale=0.2)
    w4 = SimpleNamespace(B=2, H=2, Sq=1, Sk=128, D=32, scale=0.2)
    pre = [g.standard_normal((1, 2, 64, 32)).astype(np.float16) for _ in range(3)]
    dec = [g.standard_normal((2, 2, n, 32)).astype(np.float16) for n in (1, 128, 128)]
    out = bench.cpu_baseline((w3, *pre), (w4, *dec), budget_s=1.0)
    assert out["kind"] == "oracle" and out["unit"] == "TFLOPS" and out["value"] > 0
    assert out["decode_value"] > 0 and out["decode_unit"] == "GB/s"
    assert out["affinity_cores"] == len(os.sched_getaffinity(0))
    assert out["cores"] == out["blas_threads"] >= 1
    assert out["cpu_model"]
    assert "median of 3" in out["sample"]


def test_median_time_runs_once_when_long():
    sys.path.insert(0, ROOT)
    import bench

    calls = []
    t, n = bench.median_time(lambda: calls.append(1), single_run_s=0.0)
    assert n == 1 and len(calls) == 1
    t, n = bench.median_time(lambda: calls.append(1), single_run_s=10.0)
    assert n == 3 and len(calls) == 4
