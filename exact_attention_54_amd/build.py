"""Builds the gfx950 HIP library in-tree with hipcc.

    python -m exact_attention_54_amd.build        # or __graft_entry__.build()

Produces ``exact_attention_54_amd/libfa_hip.so`` from ``csrc/fa_api.hip``
(the C ABI of ``include/fa.h`` plus every kernel), the streaming-read /
MFMA loop probes ``exact_attention_54_amd/libroofline_probe.so`` from
``csrc/roofline_probe.hip`` that bench.py reports as context, the test-only
MFMA layout probe ``tests/hip/libmfma_probe.so``, and the host-side checks
of the LDS layouts ``tests/hip/libswizzle_check.so`` and of the split
prefill's index arithmetic ``tests/hip/libsplit_check.so``.  Always
recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa_hip.so")

ARCH = "gfx950"
COMPILE_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
COMMON_FLAGS = COMPILE_FLAGS + ["-shared"]


def hipcc() -> str:
    exe = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError(f"hipcc not found ({exe})")
    return exe


def compile_shared(sources, out, include_dirs=(), extra=(), verbose=False):
    cmd = [hipcc(), *COMMON_FLAGS, *extra]
    for d in include_dirs:
        cmd += ["-I", d]
    tmp = out + ".tmp"
    cmd += list(sources) + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature name; that warning is expected
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


PROBE_SRC = os.path.join(ROOT, "tests", "hip", "mfma_probe.hip")
PROBE_LIB = os.path.join(ROOT, "tests", "hip", "libmfma_probe.so")


# The compiler's iterative ILP scheduler orders the prefill's MFMA, exp and
# LDS work better than the default (3% on the LLaMA-shaped prefill, 1% on
# the backward, 3% slower on the D = 512 Split-D forward; all bit-identical).
LIB_FLAGS = ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]


# The library's translation units and the flags each adds to LIB_FLAGS: the
# D = 256 prefill kernels keep their MFMA results in VGPRs (see
# csrc/fa_fwd256.hip), which the two-wavefront-per-SIMD kernels do not want.
LIB_UNITS = [
    ("fa_api.hip", []),
    ("fa_fwd256.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form"]),
]


def run_hipcc(cmd, verbose=False):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature name; that warning is expected
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))


def build_library(verbose: bool = False) -> str:
    """Each unit compiled to an object with its own flags, then linked."""
    objs = []
    for name, extra in LIB_UNITS:
        obj = os.path.join(CSRC, os.path.splitext(name)[0] + ".o")
        cmd = [hipcc(), *COMPILE_FLAGS, *LIB_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c",
               os.path.join(CSRC, name), "-o", obj]
        run_hipcc(cmd, verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    run_hipcc([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    for obj in objs:
        os.remove(obj)
    os.replace(tmp, LIB)
    return LIB


def build_test_probe(verbose: bool = False) -> str:
    """The MFMA lane-layout probe used by tests/test_mfma_probe.py."""
    return compile_shared([PROBE_SRC], PROBE_LIB, verbose=verbose)


ROOFLINE_SRC = os.path.join(CSRC, "roofline_probe.hip")
ROOFLINE_LIB = os.path.join(PKG, "libroofline_probe.so")


def build_roofline_probe(verbose: bool = False) -> str:
    """Plain HBM-read and MFMA-loop kernels that bench.py times for context."""
    return compile_shared([ROOFLINE_SRC], ROOFLINE_LIB, verbose=verbose)


SWIZZLE_SRC = os.path.join(ROOT, "tests", "hip", "swizzle_check.hip")
SWIZZLE_LIB = os.path.join(ROOT, "tests", "hip", "libswizzle_check.so")


def build_swizzle_check(verbose: bool = False) -> str:
    """Host-side check of the kernels' LDS layouts, used by tests/test_swizzle.py."""
    return compile_shared([SWIZZLE_SRC], SWIZZLE_LIB, include_dirs=[CSRC], verbose=verbose)


SPLIT_SRC = os.path.join(ROOT, "tests", "hip", "split_check.hip")
SPLIT_LIB = os.path.join(ROOT, "tests", "hip", "libsplit_check.so")


def build_split_check(verbose: bool = False) -> str:
    """Host-side check of the split prefill's index arithmetic, used by tests/test_split_index.py."""
    return compile_shared([SPLIT_SRC], SPLIT_LIB, include_dirs=[CSRC], verbose=verbose)


def build_all(verbose: bool = False):
    return [build_library(verbose), build_test_probe(verbose), build_roofline_probe(verbose),
            build_swizzle_check(verbose), build_split_check(verbose)]


if __name__ == "__main__":
    print(build_all(verbose="-v" in sys.argv))
