// Roofline context probes timed by bench.py (not part of the attention path):
// what a plain HBM read stream and a plain fp16 MFMA loop reach on this
// GPU, so that the attention kernels' rates can be read against what the
// chip sustains as well as against its published peaks.
//
//   probe_stream_read  reads `bytes` (a multiple of 16) with 16-byte
//                      non-temporal loads, one contiguous span per block,
//                      and folds them into one value per thread (written to
//                      `sink`, so nothing is dead code).
//   probe_mfma_loop    every wavefront runs `iters` rounds of 8 independent
//                      v_mfma_f32_32x32x16_f16 (32768 FLOP each) on register
//                      operands and writes one value per lane to `sink`.
//   probe_empty_launch a grid that does no work (thread 0 of each block
//                      writes one float to `sink`): what a launch of that
//                      shape costs by itself, the floor under the smallest
//                      attention grids.
//
// All are asynchronous on `stream` and return 0, or 1 if the launch failed.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kStreamThreads = 256;
constexpr int kMfmaThreads = 256;

// Each block streams one contiguous span, 8 loads of 16 bytes in flight per
// lane (the access pattern of the decode kernels).
__global__ void __launch_bounds__(kStreamThreads) stream_read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                                     float* __restrict__ sink) {
  constexpr int U = 8;
  const size_t span = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t begin = (size_t)blockIdx.x * span;
  const size_t end = begin + span < n16 ? begin + span : n16;
  size_t i = begin + threadIdx.x;
  unsigned acc = 0;
  for (; i + (U - 1) * kStreamThreads < end; i += U * kStreamThreads) {
    u32x4 r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) r[u] = __builtin_nontemporal_load(p + i + u * kStreamThreads);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= r[u][0] ^ r[u][1] ^ r[u][2] ^ r[u][3];
  }
  for (; i < end; i += kStreamThreads) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  sink[(size_t)blockIdx.x * kStreamThreads + threadIdx.x] = (float)acc;
}

__global__ void __launch_bounds__(kMfmaThreads, 2) mfma_loop_kernel(float* __restrict__ sink, int iters) {
  const int lane = threadIdx.x & 63;
  h8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (_Float16)(0.001f * (lane + e));
    b[e] = (_Float16)(0.002f * (lane - e));
  }
  f32x16 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[k][j] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[k][j];
  sink[(size_t)blockIdx.x * kMfmaThreads + threadIdx.x] = s;
}

__global__ void empty_kernel(float* __restrict__ sink) {
  if (threadIdx.x == 0) sink[blockIdx.x] = 0.f;
}

}  // namespace

extern "C" {

// buf: device memory of `bytes` bytes (16-byte aligned, bytes % 16 == 0);
// sink: device floats, one per thread of `blocks` x 256.
int probe_stream_read(const void* buf, size_t bytes, int blocks, float* sink, void* stream) {
  if (!buf || !sink || bytes % 16 != 0 || blocks < 1 || (reinterpret_cast<uintptr_t>(buf) & 15) != 0) return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kStreamThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// sink: device floats, one per thread of `blocks` x 256.
int probe_mfma_loop(int blocks, int iters, float* sink, void* stream) {
  if (!sink || blocks < 1 || iters < 1) return 1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(kMfmaThreads), 0, static_cast<hipStream_t>(stream), sink,
                     iters);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// sink: device floats, one per block; threads a multiple of 64, at most 1024.
int probe_empty_launch(int blocks, int threads, float* sink, void* stream) {
  if (!sink || blocks < 1 || threads < 64 || threads > 1024 || threads % 64 != 0) return 1;
  hipLaunchKernelGGL(empty_kernel, dim3(blocks), dim3(threads), 0, static_cast<hipStream_t>(stream), sink);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // extern "C"
