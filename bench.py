"""Throughput of the exact-attention hot path on one MI355X.

One step = the whole path once over one batch of synthetic fp16 N(0,1) input:
  * causal prefill fa_fwd on the LLaMA-7B-shaped workload
    (B, H, Sq, Sk, D) = (1, 32, 4096, 4096, 128), scale 1/sqrt(128);
  * split-KV decoding fa_decode_splitkv on (16, 32, 1, 8192, 128),
    num_splits chosen by the library to fill the CUs.
After the timed steps, paged decoding (fa_decode_paged) of the same K / V in
16-token pages, and packed variable-length causal prefill (fa_fwd_varlen) of
16 sequences of 256..4096 tokens (with the same batch zero-padded through
fa_fwd for comparison), and the backward pass (fa_bwd) of the causal
prefill, are timed on their own and reported beside the step figures.
Inputs are resident in HBM before the timed region.  Prefill throughput
counts 4*B*H*Sq*Sk*D FLOPs halved for the causal mask; decode throughput
counts the bytes of K and V read.  rank 0 prints one JSON line on stdout;
progress goes to stderr.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

# The oracle's BLAS uses every core this process may run on, fixed before
# numpy is first imported (an explicit setting in the environment is kept).
AFFINITY_CORES = len(os.sched_getaffinity(0))
for _var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_var, str(AFFINITY_CORES))

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP16_TFLOPS = 2516.6   # MI355X dense fp16 MFMA (256 CU x 4096 FLOP/clk x 2.4 GHz)
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
METRIC = "attn fwd TFLOPS (causal prefill D=128) + decode K/V GB/s, % of roofline"
KERNEL_SOURCES = ["fa_device.hpp", "fa_fwd_kernel.hpp", "fa_splitd_kernel.hpp", "fa_decode_kernel.hpp", "fa_bwd_kernel.hpp",
                  "fa_api.hip", "fa_fwd256.hip"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash():
    """Hash of the kernel sources' code and the library's compiler flags: //
    comments, trailing blanks and empty lines are left out, so that a
    comment edit keeps the stored counter figures valid while any code or
    flag change retires them."""
    from exact_attention_54_amd import build as fa_build

    h = hashlib.sha256()
    h.update(repr((fa_build.COMPILE_FLAGS, fa_build.LIB_FLAGS, fa_build.LIB_UNITS)).encode())
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "exact_attention_54_amd", "csrc", name), encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(kernel_keys, src_hash):
    """HBM bytes per call (summed over the listed kernels) from the committed
    rocprofv3 counter summary, only if it was taken on the current kernel
    sources; None otherwise."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    total = 0
    for key in kernel_keys:
        entry = data.get(key)
        if not entry or entry.get("source_hash") != src_hash:
            return None
        total += entry["bytes_per_launch"]
    return total


def prefill_flops(B, H, Sq, Sk, D, causal):
    f = 4.0 * B * H * Sq * Sk * D
    return f / 2 if causal else f


_HIP = None


def _hip_runtime():
    """The HIP runtime this process already runs on (torch's copy)."""
    global _HIP
    if _HIP is None:
        import ctypes

        path = next((ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln), "libamdhip64.so")
        lib = ctypes.CDLL(path)
        lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        _HIP = lib
    return _HIP


class TimingEvent:
    """A HIP event for timing only, recorded on torch's current stream (the
    stream the library launches on).  It is created with
    hipEventDisableSystemFence: recording it performs no system-scope memory
    fence, so timed kernels are not separated by L2 write-backs and
    invalidations, as they are by torch.cuda.Event's default events.  The
    elapsed times are read after torch.cuda.synchronize()."""

    FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self, torch):
        import ctypes

        self._ct = ctypes
        self.hip = _hip_runtime()
        self.ev = ctypes.c_void_p()
        assert self.hip.hipEventCreateWithFlags(ctypes.byref(self.ev), self.FLAGS) == 0
        self.stream = torch.cuda.current_stream().cuda_stream

    def record(self):
        assert self.hip.hipEventRecord(self.ev, self.stream) == 0

    def elapsed_time(self, end):
        t = self._ct.c_float()
        assert self.hip.hipEventElapsedTime(self._ct.byref(t), self.ev, end.ev) == 0
        return t.value

    def __del__(self):
        if getattr(self, "ev", None):
            self.hip.hipEventDestroy(self.ev)


def settle(torch, fn, args, warmup=None):
    """Runs fn untimed until the clocks have settled under its own load (the
    main step's spin-up, at most 200 ms per line), then the warmup calls: a
    line that follows a different workload, or idle time, otherwise starts
    at that workload's clocks (measured: the D = 256 causal prefill takes
    56.6-58.0 us per call in steady state, 59-64 us right after the
    backward, 63-64 us after 0.2 s idle)."""
    t0, n = time.perf_counter(), 0
    while (time.perf_counter() - t0) * 1e3 < min(args.spinup_ms, 200.0):
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    for _ in range(args.warmup if warmup is None else warmup):
        fn()
    torch.cuda.synchronize()


def time_launches(torch, fn, n):
    """Average duration of one call of fn, HIP timing events on the current stream."""
    start = TimingEvent(torch)
    end = TimingEvent(torch)
    torch.cuda.synchronize()
    start.record()
    for _ in range(n):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / n * 1e-3  # seconds


def roofline_context(torch, dev, buf, cus, warmup):
    """Times the plain read-stream and MFMA-loop probes (HIP events)."""
    import ctypes

    lib = ctypes.CDLL(os.path.join(ROOT, "exact_attention_54_amd", "libroofline_probe.so"))
    lib.probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.probe_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.probe_empty_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    st = torch.cuda.current_stream(dev).cuda_stream
    nbytes = buf.numel() * buf.element_size()
    rblocks, mblocks, iters = 16 * cus, 2 * cus, 4096
    sink = torch.empty(max(rblocks, mblocks) * 256, dtype=torch.float32, device=dev)

    def read():
        assert lib.probe_stream_read(buf.data_ptr(), nbytes, rblocks, sink.data_ptr(), st) == 0

    def mfma():
        assert lib.probe_mfma_loop(mblocks, iters, sink.data_ptr(), st) == 0

    def empty():  # the grid of the small (8, 16, 256, 256, 64) prefill: 256 blocks of 256 threads
        assert lib.probe_empty_launch(256, 256, sink.data_ptr(), st) == 0

    for _ in range(max(warmup, 3)):
        read()
        mfma()
        empty()
    t_read = time_launches(torch, read, 10)
    t_mfma = time_launches(torch, mfma, 10)
    # back-to-back empty launches from Python are host-bound, so 50 of them
    # are captured in a graph and the replay is timed: launch cost on the GPU
    side = torch.cuda.Stream(device=dev)  # default priority
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        empty()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gst = torch.cuda.current_stream(dev).cuda_stream
        for _ in range(50):
            assert lib.probe_empty_launch(256, 256, sink.data_ptr(), gst) == 0
    graph.replay()
    t_empty = time_launches(torch, graph.replay, 5) / 50
    mfma_flops = mblocks * 4 * iters * 8 * 32768.0   # 4 wavefronts per block, 8 MFMAs per round
    return {"context_stream_read_gbps": round(nbytes / t_read / 1e9, 1),
            "context_mfma_loop_tflops": round(mfma_flops / t_mfma / 1e12, 1),
            "context_empty_launch_us": round(t_empty * 1e6, 2)}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info

        n = [p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"]
        if n:
            return max(n)
    except Exception:
        pass
    return int(os.environ.get("OPENBLAS_NUM_THREADS", AFFINITY_CORES))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def median_time(fn, single_run_s=10.0):
    """Wall time of fn(): one run if it takes at least single_run_s, else the
    median of three."""
    t0 = time.perf_counter()
    fn()
    t = [time.perf_counter() - t0]
    if t[0] < single_run_s:
        for _ in range(2):
            t0 = time.perf_counter()
            fn()
            t.append(time.perf_counter() - t0)
    return sorted(t)[len(t) // 2], len(t)


def cpu_baseline(pre, dec, budget_s=10.0):
    """The fp64 oracle timed on a bounded sample of the same two workloads:
    whole (b, h) slices of the prefill and whole batch entries of the decode,
    as many as one run of about budget_s allows.  The fp16 -> fp64 widening
    happens before the timer; each figure is the median of three runs (one
    run if it takes over 10 s)."""
    import numpy as np

    import oracle

    (w3, q3, k3, v3), (w4, q4, k4, v4) = pre, dec
    # prefill: the first `heads` heads, sized from the time of one head
    q64, k64, v64 = (np.ascontiguousarray(x, dtype=np.float64) for x in (q3, k3, v3))
    t0 = time.perf_counter()
    oracle.attention(q64[:, :1], k64[:, :1], v64[:, :1], True, w3.scale)
    heads = max(1, min(w3.H, int(budget_s / max(time.perf_counter() - t0, 1e-6))))
    t_pre, runs_pre = median_time(
        lambda: oracle.attention(q64[:, :heads], k64[:, :heads], v64[:, :heads], True, w3.scale))
    del q64, k64, v64
    pre_tflops = prefill_flops(1, heads, w3.Sq, w3.Sk, w3.D, True) / t_pre / 1e12
    # decode: the first `nb` batch entries, sized the same way
    t0 = time.perf_counter()
    q1, k1, v1 = (np.ascontiguousarray(x[:1], dtype=np.float64) for x in (q4, k4, v4))
    oracle.attention(q1, k1, v1, False, w4.scale)
    nb = max(1, min(w4.B, int(budget_s / max(time.perf_counter() - t0, 1e-6))))
    del q1, k1, v1
    q64, k64, v64 = (np.ascontiguousarray(x[:nb], dtype=np.float64) for x in (q4, k4, v4))
    t_dec, runs_dec = median_time(lambda: oracle.attention(q64, k64, v64, False, w4.scale))
    del q64, k64, v64
    dec_gbps = 2.0 * nb * w4.H * w4.Sk * w4.D * 2 / t_dec / 1e9
    return {
        "value": round(pre_tflops, 6),
        "unit": "TFLOPS",
        "cores": blas_threads(),
        "kind": "oracle",
        "sample": f"prefill: {heads} of {w3.H} heads of the causal (1,32,4096,4096,128) workload, "
                  f"{t_pre:.2f} s (median of {runs_pre}); decode: {nb} of {w4.B} batch entries of "
                  f"(16,32,1,8192,128), {t_dec:.2f} s (median of {runs_dec}); fp64 numpy, inputs widened "
                  "to fp64 before the timer",
        "decode_value": round(dec_gbps, 4),
        "decode_unit": "GB/s",
        "cpu_model": cpu_model(),
        "affinity_cores": AFFINITY_CORES,
        "blas_threads": blas_threads(),
        "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--spinup-ms", type=float, default=300.0,
                    help="before the warmup steps, run untimed steps for this long so the GPU clocks have "
                         "left their idle state (they take ~10 ms of load to ramp up)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-splits", type=int, default=0, help="0 = library's automatic choice")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run 3 plain device copies of this many MiB (untimed), so a "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE pass over this command can be scaled by "
                         "what the counters read for a transfer of known size")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the prefill "
              "shards over heads and the decode over keys, and no multi-GPU path is built", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import exact_attention_54_amd as fa
    from workloads import (make_qkv, PAGED_BLOCK_SIZE, PAGED_PERM_SEED, VARLEN_B, VARLEN_D, VARLEN_H, VARLEN_LEN_SEED,
                           VARLEN_MAX, VARLEN_MIN, VARLEN_SEED, WORKLOADS, make_varlen, paged_layout,
                           varlen_lengths, workload_inputs)

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    w3, w4 = WORKLOADS["llama7b_prefill"], WORKLOADS["decode_8k"]

    log("generating inputs")
    pre_host = workload_inputs(w3)
    dec_host = workload_inputs(w4)
    q3, k3, v3 = (torch.from_numpy(x).to(dev) for x in pre_host)
    q4, k4, v4 = (torch.from_numpy(x).to(dev) for x in dec_host)
    o3 = torch.empty_like(q3)
    l3 = torch.empty((w3.B, w3.H, w3.Sq), dtype=torch.float32, device=dev)
    o4 = torch.empty_like(q4)
    l4 = torch.empty((w4.B, w4.H, 1), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    ns = args.decode_splits if args.decode_splits > 0 else fa.fa_decode_auto_splits(w4.B, w4.H, w4.Sk, cus)

    def prefill():
        fa.fa_fwd(q3, k3, v3, o3, l3, causal=True, scale=w3.scale)

    def decode():
        fa.fa_decode_splitkv(q4, k4, v4, o4, l4, scale=w4.scale, num_splits=ns)

    def step():
        prefill()
        decode()

    # clock spin-up: from idle the GPU needs ~10 ms of load before its clocks
    # settle, so a short warmup alone would leave the first timed steps slow
    t0, n_spin = time.perf_counter(), 0
    while (time.perf_counter() - t0) * 1e3 < args.spinup_ms:
        step()
        n_spin += 1
        if n_spin % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    log(f"spin-up: {n_spin} untimed steps in {(time.perf_counter() - t0) * 1e3:.0f} ms")
    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    # one event between consecutive launches inside the timed loop: launch
    # j runs between events j and j + 1, so the per-kernel averages are taken
    # under the same conditions as the step time, and the first and last
    # events bracket the whole timed region
    ev = [TimingEvent(torch) for _ in range(2 * args.steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(args.steps):
        prefill()
        ev[2 * i + 1].record()
        decode()
        ev[2 * i + 2].record()
    torch.cuda.synchronize()
    ms_per_step = ev[0].elapsed_time(ev[-1]) / args.steps
    t_pre = sum(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(args.steps)) / args.steps * 1e-3
    t_dec = sum(ev[2 * i + 1].elapsed_time(ev[2 * i + 2]) for i in range(args.steps)) / args.steps * 1e-3
    flops = prefill_flops(w3.B, w3.H, w3.Sq, w3.Sk, w3.D, True)
    kv_bytes = 2.0 * w4.B * w4.H * w4.Sk * w4.D * 2
    tflops = flops / t_pre / 1e12
    gbps = kv_bytes / t_dec / 1e9
    log(f"step {ms_per_step * 1e3:.1f} us; prefill {t_pre * 1e6:.1f} us = {tflops:.1f} TFLOPS; "
        f"decode {t_dec * 1e6:.1f} us = {gbps:.1f} GB/s (ns={ns})")
    t_pre_hot = time_launches(torch, prefill, args.steps)
    log(f"prefill back-to-back (K/V cache-warm): {t_pre_hot * 1e6:.1f} us = {flops / t_pre_hot / 1e12:.1f} TFLOPS")

    # The same decode in its two-kernel form: the smallest power-of-two split
    # count that gives every CU 8 phase-one workgroups of 256 threads (the
    # partitions that fill the CUs), then the log-sum-exp merge kernel; with
    # a caller workspace, so the call allocates nothing.  Timed back to back.
    ns2 = 1
    while w4.B * w4.H * ns2 < 8 * cus:
        ns2 *= 2
    ws2 = torch.empty(fa.fa_decode_workspace_bytes(w4.B, w4.H, w4.D, ns2), dtype=torch.uint8, device=dev)
    o4b, l4b = torch.empty_like(o4), torch.empty_like(l4)

    def decode_two_kernel():
        fa.fa_decode_splitkv_ws(q4, k4, v4, ws2, o4b, l4b, scale=w4.scale, num_splits=ns2)

    settle(torch, decode_two_kernel, args)
    t_dec2 = time_launches(torch, decode_two_kernel, args.steps)
    gbps2 = kv_bytes / t_dec2 / 1e9
    log(f"decode two-kernel form (ns={ns2}, caller workspace): {t_dec2 * 1e6:.1f} us = {gbps2:.1f} GB/s")
    del ws2, o4b, l4b

    # Paged decoding of the same K / V, held in 16-token pages in a seeded
    # random physical order (built on the GPU, untimed); timed back to back.
    bs = PAGED_BLOCK_SIZE
    max_blocks = w4.Sk // bs
    tables, nb = paged_layout(w4.B, max_blocks, PAGED_PERM_SEED)
    td = torch.from_numpy(tables).to(dev)
    idx = td.reshape(-1).long()
    kc = torch.empty((nb, w4.H, bs, w4.D), dtype=torch.float16, device=dev)
    vc = torch.empty_like(kc)
    kc[idx] = k4.view(w4.B, w4.H, max_blocks, bs, w4.D).permute(0, 2, 1, 3, 4).reshape(-1, w4.H, bs, w4.D)
    vc[idx] = v4.view(w4.B, w4.H, max_blocks, bs, w4.D).permute(0, 2, 1, 3, 4).reshape(-1, w4.H, bs, w4.D)
    sl = torch.full((w4.B,), w4.Sk, dtype=torch.int32, device=dev)
    op4 = torch.empty_like(o4)
    lp4 = torch.empty_like(l4)

    def paged():
        fa.fa_decode_paged(q4, kc, vc, td, sl, op4, lp4, scale=w4.scale, num_splits=ns)

    settle(torch, paged, args)
    t_paged = time_launches(torch, paged, args.steps)
    gbps_paged = kv_bytes / t_paged / 1e9
    log(f"paged decode (block_size {bs}, random page order): {t_paged * 1e6:.1f} us = {gbps_paged:.1f} GB/s")
    del kc, vc

    # Packed variable-length causal prefill: 16 sequences of 256..4096 tokens
    # (LLaMA-7B heads), timed back to back, and the same batch zero-padded to
    # its longest sequence through fa_fwd, the padding the packed layout avoids.
    lens = varlen_lengths(VARLEN_B, VARLEN_MIN, VARLEN_MAX, VARLEN_LEN_SEED)
    vq, vk, vv, cu_q, cu_k = make_varlen(lens, VARLEN_H, VARLEN_D, VARLEN_SEED)
    vq, vk, vv, cqd, ckd = (torch.from_numpy(x).to(dev) for x in (vq, vk, vv, cu_q, cu_k))
    vo = torch.empty_like(vq)
    vl = torch.empty((VARLEN_H, vq.shape[0]), dtype=torch.float32, device=dev)
    Lmax = int(lens.max())
    vscale = VARLEN_D ** -0.5

    def varlen():
        fa.fa_fwd_varlen(vq, vk, vv, cqd, ckd, Lmax, Lmax, vo, vl, causal=True, scale=vscale)

    pads = [torch.zeros((VARLEN_B, VARLEN_H, Lmax, VARLEN_D), dtype=torch.float16, device=dev) for _ in range(3)]
    for b in range(VARLEN_B):
        s0, n = int(cu_q[b]), int(lens[b])
        for dst, src in zip(pads, (vq, vk, vv)):
            dst[b, :, :n] = src[s0:s0 + n].permute(1, 0, 2)
    po = torch.empty_like(pads[0])
    pl = torch.empty((VARLEN_B, VARLEN_H, Lmax), dtype=torch.float32, device=dev)

    def padded():
        fa.fa_fwd(pads[0], pads[1], pads[2], po, pl, causal=True, scale=vscale)

    settle(torch, varlen, args)
    t_var = time_launches(torch, varlen, args.steps)
    settle(torch, padded, args)
    t_pad = time_launches(torch, padded, args.steps)
    flops_var = float(sum(4.0 * VARLEN_H * int(n) * int(n) * VARLEN_D / 2 for n in lens))
    tflops_var = flops_var / t_var / 1e12
    log(f"varlen prefill ({VARLEN_B} sequences, {int(lens.sum())} tokens): {t_var * 1e6:.1f} us = "
        f"{tflops_var:.1f} TFLOPS; padded to {Lmax}: {t_pad * 1e6:.1f} us")
    del pads, po, pl, vq, vk, vv, vo, vl

    # Backward of the causal prefill (fa_bwd: D, dK/dV, dQ kernels) from the
    # forward's o and lse with a seeded fp16 dO, timed back to back.
    do3 = torch.from_numpy(make_qkv(w3.B, w3.H, w3.Sq, 1, w3.D, 13)[0]).to(dev)
    prefill()
    dq3, dk3, dv3 = torch.empty_like(q3), torch.empty_like(k3), torch.empty_like(v3)

    def backward():
        fa.fa_bwd(q3, k3, v3, o3, l3, do3, dq3, dk3, dv3, causal=True, scale=w3.scale)

    settle(torch, backward, args)
    t_bwd = time_launches(torch, backward, args.steps)
    tflops_bwd = 2.5 * flops / t_bwd / 1e12
    log(f"backward (causal prefill shape): {t_bwd * 1e6:.1f} us = {tflops_bwd:.1f} TFLOPS (2.5 x forward FLOPs)")
    del dq3, dk3, dv3, do3

    # The D = 256 causal prefill (1,16,2048,2048,256) and the Split-D forward
    # on the large-head shapes (D = 512 and 1024), both masks, timed back to
    # back; FLOPs counted as for the prefill above.
    w5 = WORKLOADS["d256_prefill"]
    q5, k5, v5 = (torch.from_numpy(x).to(dev) for x in workload_inputs(w5))
    o5 = torch.empty_like(q5)
    l5 = torch.empty((w5.B, w5.H, w5.Sq), dtype=torch.float32, device=dev)

    # split grids take a workspace: allocated once, as a serving loop would
    # (fa_fwd_ws; fa_fwd would take it from the stream-ordered pool per call)
    ws5_bytes = fa.fa_fwd_workspace_bytes(w5.B, w5.H, w5.Sq, w5.Sk, w5.D, True, cus)
    ws5 = torch.empty(ws5_bytes, dtype=torch.uint8, device=dev) if ws5_bytes else None

    def d256():
        fa.fa_fwd_ws(q5, k5, v5, ws5, o5, l5, causal=True, scale=w5.scale)

    settle(torch, d256, args)
    t_d256 = time_launches(torch, d256, args.steps)
    tflops_d256 = prefill_flops(w5.B, w5.H, w5.Sq, w5.Sk, w5.D, True) / t_d256 / 1e12
    log(f"D=256 causal prefill (1,16,2048,2048,256): {t_d256 * 1e6:.1f} us = {tflops_d256:.1f} TFLOPS")

    # Batch-1 decoding (one sequence, as a latency-bound server step): 32
    # heads over 8K keys and 8 heads over 32K keys, the library's split
    # choice, two kernels (partitions, then their merge) per call.
    small_dec = {}
    for sb, sh, ssk in ((1, 32, 8192), (1, 8, 32768)):
        qb, kb_, vb_ = (torch.from_numpy(x).to(dev) for x in make_qkv(sb, sh, 1, ssk, 128, seed=40 + sh))
        ob = torch.empty_like(qb)
        lb = torch.empty((sb, sh, 1), dtype=torch.float32, device=dev)

        def dec1(qb=qb, kb_=kb_, vb_=vb_, ob=ob, lb=lb):
            fa.fa_decode_splitkv(qb, kb_, vb_, ob, lb, scale=128 ** -0.5)

        settle(torch, dec1, args, max(args.warmup, 3))
        t_b = time_launches(torch, dec1, args.steps)
        tag = f"decode_b{sb}_h{sh}_k{ssk // 1024}k"
        small_dec[tag + "_us"] = round(t_b * 1e6, 2)
        small_dec[tag + "_gbps"] = round(2 * sb * sh * ssk * 128 * 2 / t_b / 1e9, 1)
        small_dec[tag + "_splits"] = fa.fa_decode_auto_splits(sb, sh, ssk, cus)
        log(f"batch-1 decode ({sb},{sh},1,{ssk},128): {t_b * 1e6:.1f} us = {small_dec[tag + '_gbps']} GB/s "
            f"({small_dec[tag + '_splits']} partitions)")
        del qb, kb_, vb_, ob, lb

    # One GPU's share of the LLaMA-7B-shaped prefill sharded by heads over 8
    # GPUs: 4 of the 32 heads, (1, 4, 4096, 4096, 128) causal.  128 query
    # tiles leave most CUs idle, so fa_fwd splits the key ranges of the
    # heaviest ones (fa_fwd_key_splits parts) and merges them.
    hs = 4
    qs_, ks_, vs_ = (x[:, :hs].contiguous() for x in (q3, k3, v3))
    os_ = torch.empty_like(qs_)
    ls_ = torch.empty((1, hs, w3.Sq), dtype=torch.float32, device=dev)

    wss_bytes = fa.fa_fwd_workspace_bytes(1, hs, w3.Sq, w3.Sk, w3.D, True, cus)
    wss = torch.empty(wss_bytes, dtype=torch.uint8, device=dev) if wss_bytes else None

    def shard():
        fa.fa_fwd_ws(qs_, ks_, vs_, wss, os_, ls_, causal=True, scale=w3.scale)

    settle(torch, shard, args)
    t_shard = time_launches(torch, shard, args.steps)
    tflops_shard = prefill_flops(1, hs, w3.Sq, w3.Sk, w3.D, True) / t_shard / 1e12
    shard_parts = fa.fa_fwd_key_splits(1, hs, w3.Sq, w3.Sk, w3.D, True, cus)
    log(f"head-shard prefill (1,{hs},4096,4096,128): {t_shard * 1e6:.1f} us = {tflops_shard:.1f} TFLOPS "
        f"({shard_parts} key parts)")
    del q5, k5, v5, o5, l5
    # the small (8,16,256,256,64) shape, both masks: launch-sized work
    w2 = WORKLOADS["small"]
    q2, k2, v2 = (torch.from_numpy(x).to(dev) for x in workload_inputs(w2))
    o2 = torch.empty_like(q2)
    l2 = torch.empty((w2.B, w2.H, w2.Sq), dtype=torch.float32, device=dev)
    small = {}
    for causal in (False, True):
        def small_fwd():
            fa.fa_fwd(q2, k2, v2, o2, l2, causal=causal, scale=w2.scale)

        settle(torch, small_fwd, args)
        t = time_launches(torch, small_fwd, args.steps)
        tag = "small_prefill_" + ("causal" if causal else "full")
        small[tag + "_us"] = round(t * 1e6, 2)
        small[tag + "_tflops"] = round(prefill_flops(w2.B, w2.H, w2.Sq, w2.Sk, w2.D, causal) / t / 1e12, 3)
        log(f"small (8,16,256,256,64) causal={causal}: {t * 1e6:.1f} us per call")
    del q2, k2, v2, o2, l2
    splitd = {}
    for name in ("d512_prefill", "d1024_prefill"):
        w = WORKLOADS[name]
        qx, kx, vx = (torch.from_numpy(x).to(dev) for x in workload_inputs(w))
        ox = torch.empty_like(qx)
        lx = torch.empty((w.B, w.H, w.Sq), dtype=torch.float32, device=dev)
        for causal in (False, True):
            # key parts need a workspace: allocated once (fa_fwd_ws)
            wsx_bytes = fa.fa_fwd_workspace_bytes(w.B, w.H, w.Sq, w.Sk, w.D, causal, cus)
            wsx = torch.empty(wsx_bytes, dtype=torch.uint8, device=dev) if wsx_bytes else None

            def large_head():
                fa.fa_fwd_ws(qx, kx, vx, wsx, ox, lx, causal=causal, scale=w.scale)

            settle(torch, large_head, args)
            t = time_launches(torch, large_head, args.steps)
            tf = prefill_flops(w.B, w.H, w.Sq, w.Sk, w.D, causal) / t / 1e12
            tag = f"{name}_{'causal' if causal else 'full'}"
            splitd[tag + "_us"] = round(t * 1e6, 2)
            splitd[tag + "_tflops"] = round(tf, 3)
            log(f"split-D {name} causal={causal}: {t * 1e6:.1f} us = {tf:.1f} TFLOPS")
        del qx, kx, vx, ox, lx

    # Context, not the metric: what a plain 16-byte non-temporal read stream
    # (over the 1 GiB K cache) and a plain register-only fp16 MFMA loop reach
    # on this GPU right now (exact_attention_54_amd/csrc/roofline_probe.hip).
    context = roofline_context(torch, dev, k4, cus, args.warmup)
    log(f"context: plain HBM read stream {context['context_stream_read_gbps']:.1f} GB/s; "
        f"plain fp16 MFMA loop {context['context_mfma_loop_tflops']:.1f} TFLOPS; "
        f"empty 256 x 256 launch {context['context_empty_launch_us']:.2f} us")

    src_hash = kernel_source_hash()
    roof_pre = {
        "kernel": "fwd_kernel<128,32,causal>",
        "bound": "mfma",
        "achieved": round(tflops, 3),
        "peak": PEAK_FP16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(tflops / PEAK_FP16_TFLOPS, 4),
        "traffic": measured_traffic(["fwd_kernel<128,32,causal>"], src_hash),
    }
    # one partition: a single kernel splits the keys over the 16 wavefronts
    # of a 1024-thread workgroup and merges them in LDS
    dec_kernels = ["decode_partial_kernel<128>"] + ([] if ns == 1 else ["decode_merge_kernel<128>"])
    roof_dec = {
        "kernel": "decode_partial_kernel<128,1024,final>" if ns == 1 else " + ".join(dec_kernels),
        "bound": "hbm",
        "achieved": round(gbps, 2),
        "peak": PEAK_HBM_GBPS,
        "unit": "GB/s",
        "frac": round(gbps / PEAK_HBM_GBPS, 4),
        "traffic": measured_traffic(dec_kernels, src_hash),
    }
    dominant, other = (roof_pre, roof_dec) if t_pre >= t_dec else (roof_dec, roof_pre)

    out = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": "causal prefill (B,H,Sq,Sk,D)=(1,32,4096,4096,128) + split-KV decode "
                        "(16,32,1,8192,128)",
            "prefill_frac_of_peak": round(tflops / PEAK_FP16_TFLOPS, 4),
            "decode_gbps": round(gbps, 2),
            "decode_frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4),
            "decode_num_splits": ns,
            "prefill_us": round(t_pre * 1e6, 2),
            "decode_us": round(t_dec * 1e6, 2),
            "prefill_us_back_to_back": round(t_pre_hot * 1e6, 2),
            "decode_two_kernel_splits": ns2,
            "decode_two_kernel_us": round(t_dec2 * 1e6, 2),
            "decode_two_kernel_gbps": round(gbps2, 2),
            "decode_two_kernel_frac_of_peak": round(gbps2 / PEAK_HBM_GBPS, 4),
            "paged_decode_gbps": round(gbps_paged, 2),
            "paged_decode_frac_of_peak": round(gbps_paged / PEAK_HBM_GBPS, 4),
            "paged_decode_us": round(t_paged * 1e6, 2),
            "paged_block_size": bs,
            "varlen_prefill_tflops": round(tflops_var, 3),
            "varlen_prefill_frac_of_peak": round(tflops_var / PEAK_FP16_TFLOPS, 4),
            "varlen_prefill_us": round(t_var * 1e6, 2),
            "varlen_tokens": int(lens.sum()),
            "varlen_padded_us": round(t_pad * 1e6, 2),
            "backward_tflops": round(tflops_bwd, 3),
            "backward_frac_of_peak": round(tflops_bwd / PEAK_FP16_TFLOPS, 4),
            "backward_us": round(t_bwd * 1e6, 2),
            "d256_prefill_tflops": round(tflops_d256, 3),
            "d256_prefill_frac_of_peak": round(tflops_d256 / PEAK_FP16_TFLOPS, 4),
            "d256_prefill_us": round(t_d256 * 1e6, 2),
            "d256_key_parts": fa.fa_fwd_key_splits(w5.B, w5.H, w5.Sq, w5.Sk, w5.D, True, cus),
            "head_shard_prefill_tflops": round(tflops_shard, 3),
            "head_shard_prefill_frac_of_peak": round(tflops_shard / PEAK_FP16_TFLOPS, 4),
            "head_shard_prefill_us": round(t_shard * 1e6, 2),
            "head_shard_key_parts": shard_parts,
            **small_dec,
            **small,
            **context,
            **{"splitd_" + k: x for k, x in splitd.items()},
            "accumulate": "fp32",
            "kernel_source_hash": src_hash,
        },
        "roofline": dominant,
        "roofline_other": other,
    }
    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * 2**20 // 2
        x = torch.ones(n, dtype=torch.float16, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        out["config"]["copy_calibration_bytes"] = n * 2
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline((w3, *pre_host), (w4, *dec_host))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
