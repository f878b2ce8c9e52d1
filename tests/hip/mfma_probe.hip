// Test-only probe of the gfx950 32x32x16 fp16 MFMA lane layout.  One
// wavefront loads the per-lane operand registers given by the host, runs
// one v_mfma_f32_32x32x16_f16 and stores the 16 accumulator registers of
// every lane.  The host decides which matrix element each register holds;
// the test checks that the product lands where the layout says.
#include <hip/hip_runtime.h>

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(64) probe_kernel(const h8* a, const h8* b, f32x16* c) {
  const int l = threadIdx.x;  // exactly 64 lanes, arrays hold 64 entries each
  f32x16 acc = {};
  acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[l], b[l], acc, 0, 0, 0);
  c[l] = acc;
}

extern "C" int probe_mfma_32x32x16(const void* a_regs, const void* b_regs, void* c_regs) {
  // a_regs, b_regs: 64 x 8 fp16; c_regs: 64 x 16 fp32 (device memory)
  hipLaunchKernelGGL(probe_kernel, dim3(1), dim3(64), 0, 0, static_cast<const h8*>(a_regs),
                     static_cast<const h8*>(b_regs), static_cast<f32x16*>(c_regs));
  if (hipGetLastError() != hipSuccess) return 1;
  return hipDeviceSynchronize() == hipSuccess ? 0 : 2;
}

// v_permlane32_swap with both operands = x: returns (x of lanes 0..31 in
// both halves, x of lanes 32..63 in both halves).
__global__ void __launch_bounds__(64) permlane_kernel(const unsigned* x, unsigned* lo, unsigned* hi) {
  const int l = threadIdx.x;  // exactly 64 lanes, arrays hold 64 entries each
  const auto r = __builtin_amdgcn_permlane32_swap(x[l], x[l], false, false);
  lo[l] = r[0];
  hi[l] = r[1];
}

extern "C" int probe_permlane32_swap(const void* x, void* lo, void* hi) {
  hipLaunchKernelGGL(permlane_kernel, dim3(1), dim3(64), 0, 0, static_cast<const unsigned*>(x),
                     static_cast<unsigned*>(lo), static_cast<unsigned*>(hi));
  if (hipGetLastError() != hipSuccess) return 1;
  return hipDeviceSynchronize() == hipSuccess ? 0 : 2;
}
