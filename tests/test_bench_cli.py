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
