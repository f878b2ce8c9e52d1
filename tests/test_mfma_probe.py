"""Pins the 32x32x16 fp16 MFMA lane layout the kernels assume (GPU).

Lane l supplies A[l % 32][8 * (l // 32) + t] and B[8 * (l // 32) + t][l % 32]
(t = 0..7) and receives C[8 * (j // 4) + 4 * (l // 32) + j % 4][l % 32] in
accumulator register j.  Small-integer operands make every product exact.
"""
import ctypes
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hip", "libmfma_probe.so")


def test_mfma_32x32x16_layout():
    import torch

    assert torch.cuda.is_available(), "GPU test needs a GPU"
    assert os.path.exists(PROBE), "probe library not built"
    lib = ctypes.CDLL(PROBE)
    lib.probe_mfma_32x32x16.restype = ctypes.c_int
    lib.probe_mfma_32x32x16.argtypes = [ctypes.c_void_p] * 3

    rng = np.random.Generator(np.random.PCG64(7))
    A = rng.integers(-8, 9, size=(32, 16)).astype(np.float16)
    B = rng.integers(-8, 9, size=(16, 32)).astype(np.float16)
    a_regs = np.empty((64, 8), np.float16)
    b_regs = np.empty((64, 8), np.float16)
    for l in range(64):
        for t in range(8):
            a_regs[l, t] = A[l % 32, 8 * (l // 32) + t]
            b_regs[l, t] = B[8 * (l // 32) + t, l % 32]
    dev = torch.device("cuda:0")
    a_d = torch.from_numpy(a_regs).to(dev)
    b_d = torch.from_numpy(b_regs).to(dev)
    c_d = torch.zeros((64, 16), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    assert lib.probe_mfma_32x32x16(a_d.data_ptr(), b_d.data_ptr(), c_d.data_ptr()) == 0
    c_regs = c_d.cpu().numpy()
    C = A.astype(np.float64) @ B.astype(np.float64)
    got = np.empty((32, 32))
    for l in range(64):
        for j in range(16):
            got[8 * (j // 4) + 4 * (l // 32) + j % 4, l % 32] = c_regs[l, j]
    np.testing.assert_array_equal(got, C)


def test_permlane32_swap_exchanges_wave_halves():
    """xhalf_max / xhalf_sum rely on v_permlane32_swap(x, x) returning the
    low half of x broadcast to both halves and the high half likewise."""
    import torch

    assert torch.cuda.is_available(), "GPU test needs a GPU"
    lib = ctypes.CDLL(PROBE)
    lib.probe_permlane32_swap.restype = ctypes.c_int
    lib.probe_permlane32_swap.argtypes = [ctypes.c_void_p] * 3
    dev = torch.device("cuda:0")
    x = torch.arange(1000, 1064, dtype=torch.int32, device=dev)
    lo = torch.zeros(64, dtype=torch.int32, device=dev)
    hi = torch.zeros(64, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    assert lib.probe_permlane32_swap(x.data_ptr(), lo.data_ptr(), hi.data_ptr()) == 0
    xs = list(range(1000, 1064))
    assert lo.cpu().tolist() == xs[:32] + xs[:32]
    assert hi.cpu().tolist() == xs[32:] + xs[32:]


ROOFLINE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "exact_attention_54_amd",
                        "libroofline_probe.so")


def test_roofline_probes_run():
    # the context probes bench.py times: a read stream over a known buffer
    # (every thread's fold lands in the sink) and a short MFMA loop
    import torch

    assert os.path.exists(ROOFLINE), "roofline probe library not built"
    lib = ctypes.CDLL(ROOFLINE)
    lib.probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.probe_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    buf = torch.zeros(1 << 20, dtype=torch.int32, device=dev)
    sink = torch.full((4 * 256,), -1.0, dtype=torch.float32, device=dev)
    assert lib.probe_stream_read(buf.data_ptr(), buf.numel() * 4, 4, sink.data_ptr(), None) == 0
    torch.cuda.synchronize()
    assert (sink == 0).all()  # XOR of zeros
    assert lib.probe_stream_read(buf.data_ptr(), 10, 4, sink.data_ptr(), None) == 1  # not a multiple of 16
    assert lib.probe_mfma_loop(4, 3, sink.data_ptr(), None) == 0
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all()
