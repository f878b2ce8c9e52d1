// The D = 256 instantiations of fa::fwd_kernel, in a translation unit of
// their own: this one is compiled with the MFMA results in VGPRs
// (-mllvm -amdgpu-mfma-vgpr-form).  At D = 256 a wavefront has its SIMD's
// whole register file; with Q pinned to the accumulation registers (see
// fwd_kernel) and O, S and P in VGPRs, the loop moves nothing between the
// two register files.  The default MFMA form put O and S in AGPRs and spent
// ~44 register moves per key tile reading S back for the softmax; the other
// kernels (two wavefronts per SIMD, 256 registers each) do best with the
// default form, hence the separate unit.  fa_api.hip declares these
// instantiations extern and launches them.
#include "fa_fwd_kernel.hpp"

namespace fa {

#define FA_FWD256_INSTANCE(CAUSAL, VARLEN, KSPLIT)                                                               \
  template __global__ void fwd_kernel<256, 32, 4, CAUSAL, VARLEN, KSPLIT>(                                       \
      const _Float16* __restrict__, const _Float16* __restrict__, const _Float16* __restrict__,                  \
      _Float16* __restrict__, float* __restrict__, int, int, int, int, float, VarlenArgs, KeySplit);

FA_FWD256_INSTANCE(false, false, false)
FA_FWD256_INSTANCE(true, false, false)
FA_FWD256_INSTANCE(false, false, true)
FA_FWD256_INSTANCE(true, false, true)
FA_FWD256_INSTANCE(false, true, false)
FA_FWD256_INSTANCE(true, true, false)

#undef FA_FWD256_INSTANCE

}  // namespace fa
