// Exact attention forward (prefill) for gfx950, FlashAttention-2 loop order.
//
// One workgroup = 4 wavefronts = BM = 128 query rows ("Split-Q"; the loop
// inversion of "Adaptive High-Performance Attention Kernels in CUDA",
// Architectural Progression, Stage 3: outer query tile, inner key/value
// stream, output accumulator in registers).  Each wavefront owns 32 query
// rows for the whole kernel.
//
// Per key/value tile of BN keys:
//   S^T = K Q^T   on v_mfma_f32_32x32x16_f16 with K from LDS as the A
//                 operand and the wavefront's Q rows (registers) as B.  The
//                 transposed product puts one query row in each lane (lanes
//                 l and l+32 share a row), so the row max needs one
//                 cross-half exchange and the row sum none until the end.
//   online softmax  m_new = max(m, rowmax), p = 2^(s*c - m_new),
//                 alpha = 2^(m - m_new), l = alpha*l + rowsum(p), O *= alpha,
//                 with c = scale*log2(e) folded into one FMA per score
//                 ("FlashAttention-2 MMA", Technical Details, Online Softmax).
//   O^T += V^T P^T  P is rounded to fp16 in registers and used directly as
//                 the B operand: the accumulator layout of S^T lists keys
//                 8*(j/4) + 4*(l/32) + j%4, and the contraction index is
//                 free to permute as long as V^T uses the same order, so V
//                 is written to LDS transposed ([d][key]) with key bits 2
//                 and 3 swapped; each lane then reads its 8 keys as one
//                 16-byte LDS load.
// Key/value tiles are double-buffered in LDS: the next tile's global loads
// (16-byte, coalesced) are issued before the current tile's MFMAs and
// written to the other LDS stage afterwards (Lever C of the same page).
// Both LDS arrays use the XOR swizzle of fa::swz (Lever B).
// Causal: key tiles wholly above the diagonal of the workgroup are never
// visited, wavefronts skip tiles above their own rows, and only tiles that
// cross the diagonal evaluate the mask (Lever A).  Query tiles are issued
// heaviest first so the triangular work packs well onto the CUs.
#pragma once

#include "fa_device.hpp"

namespace fa {

template <int D, int BN>
struct FwdCfg {
  static constexpr int NWAVES = 4;
  static constexpr int THREADS = 64 * NWAVES;
  static constexpr int BM = 32 * NWAVES;
  static constexpr int KCH = D / 8;   // 16-byte chunks per K row in LDS
  static constexpr int VCH = BN / 8;  // 16-byte chunks per V^T row in LDS
  static constexpr int NKB = BN / 32; // 32-key blocks per tile
  static constexpr int NDB = D / 32;  // 32-wide d blocks of the output
  static constexpr int K_TILE_BYTES = BN * D * 2;
  static constexpr int V_TILE_BYTES = D * BN * 2;
  static constexpr int STAGE_BYTES = K_TILE_BYTES + V_TILE_BYTES;
  static constexpr int EPI_BYTES = NWAVES * 32 * D * 2;
  static constexpr int LDS_BYTES = (2 * STAGE_BYTES > EPI_BYTES) ? 2 * STAGE_BYTES : EPI_BYTES;
  static constexpr int K_PER_THREAD = BN * KCH / THREADS;     // 16-byte K chunks per thread
  static constexpr int V_BLOCKS = (BN / 4) * (D / 8);          // 4-key x 8-d V blocks per tile
  static constexpr int V_PER_THREAD = (V_BLOCKS + THREADS - 1) / THREADS;
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert(BN * KCH % THREADS == 0, "K tile must split evenly over the workgroup");
  static_assert(LDS_BYTES <= 65536, "static LDS budget");
};

// Position of key `k` (0..BN-1) inside a V^T row: bits 2 and 3 swapped.
__device__ __forceinline__ int vt_pos(int k) {
  return (k & ~0xC) | ((k & 4) << 1) | ((k & 8) >> 1);
}

template <int D, int BN, bool CAUSAL>
__global__ void __launch_bounds__(256)
fwd_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
           const _Float16* __restrict__ V, _Float16* __restrict__ O, float* __restrict__ LSE,
           int Sq, int Sk, int BH, int nqt, float c2) {
  using C = FwdCfg<D, BN>;
  __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int r32 = lane & 31;
  const int hh = lane >> 5;

  // Work item: consecutive workgroup ids walk all (batch, head) slices of
  // one query-tile rank before the next rank, so the dispatcher sees the
  // heaviest causal tiles first and, with B*H a multiple of 8, every tile
  // of a slice runs on the same XCD (workgroups are dealt to XCDs round
  // robin by id) and shares its L2.
  const int rank = blockIdx.x / BH;
  const int bh = blockIdx.x - rank * BH;
  const int qt = CAUSAL ? (nqt - 1 - rank) : rank;
  const int q0 = qt * C::BM;
  const int qw = q0 + 32 * w;            // first query row of this wavefront
  const int qi = qw + r32;               // query row held by this lane
  const size_t qoff = (size_t)bh * Sq * D;
  const size_t koff = (size_t)bh * Sk * D;

  // Q fragment: B operand of S^T = K Q^T, 8 consecutive d per lane and step.
  h8 qreg[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 t = {0u, 0u, 0u, 0u};
    if (qi < Sq) t = *reinterpret_cast<const u32x4*>(Q + qoff + (size_t)qi * D + 16 * ks + 8 * hh);
    qreg[ks] = as_h8(t);
  }

  const int nkt_all = (Sk + BN - 1) / BN;
  const int nkt = CAUSAL ? min(nkt_all, (min(q0 + C::BM, Sk) + BN - 1) / BN) : nkt_all;

  // Global -> register staging of one K/V tile.
  u32x4 kst[C::K_PER_THREAD];
  u32x4 vst[C::V_PER_THREAD][4];
  auto gload = [&](int kt) {
    const int kbase = kt * BN;
#pragma unroll
    for (int u = 0; u < C::K_PER_THREAD; ++u) {
      const int ci = tid + C::THREADS * u;
      const int r = ci / C::KCH, c = ci % C::KCH;
      const int key = kbase + r;
      u32x4 t = {0u, 0u, 0u, 0u};
      if (key < Sk) t = *reinterpret_cast<const u32x4*>(K + koff + (size_t)key * D + c * 8);
      kst[u] = t;
    }
#pragma unroll
    for (int u = 0; u < C::V_PER_THREAD; ++u) {
      const int bi = tid + C::THREADS * u;
      if (C::V_BLOCKS % C::THREADS != 0 && bi >= C::V_BLOCKS) continue;
      const int kg = bi / (D / 8), dc = bi % (D / 8);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int key = kbase + 4 * kg + rr;
        u32x4 t = {0u, 0u, 0u, 0u};
        if (key < Sk) t = *reinterpret_cast<const u32x4*>(V + koff + (size_t)key * D + dc * 8);
        vst[u][rr] = t;
      }
    }
  };
  // Register -> LDS stage: K row-major swizzled, V transposed to [d][key].
  auto lstore = [&](int st) {
    char* Ks = smem + st * C::STAGE_BYTES;
    char* Vs = Ks + C::K_TILE_BYTES;
#pragma unroll
    for (int u = 0; u < C::K_PER_THREAD; ++u) {
      const int ci = tid + C::THREADS * u;
      const int r = ci / C::KCH, c = ci % C::KCH;
      *reinterpret_cast<u32x4*>(Ks + swz<C::KCH>(r, c)) = kst[u];
    }
#pragma unroll
    for (int u = 0; u < C::V_PER_THREAD; ++u) {
      const int bi = tid + C::THREADS * u;
      if (C::V_BLOCKS % C::THREADS != 0 && bi >= C::V_BLOCKS) continue;
      const int kg = bi / (D / 8), dc = bi % (D / 8);
      const int p = vt_pos(4 * kg);         // 4 consecutive keys stay consecutive
      const int cp = p >> 3, hoff = (p & 7) * 2;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dw = e >> 1;
        const bool hi = (e & 1) != 0;
        u32x2 out;
        out.x = pack_halves(vst[u][0][dw], vst[u][1][dw], hi);
        out.y = pack_halves(vst[u][2][dw], vst[u][3][dw], hi);
        *reinterpret_cast<u32x2*>(Vs + swz<C::VCH>(8 * dc + e, cp) + hoff) = out;
      }
    }
  };

  f32x16 oacc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[db][j] = 0.f;
  float m_run = kNegInf;  // running row max of s*c (log2 units)
  float l_run = 0.f;      // this lane's share of the running row sum

  gload(0);
  lstore(0);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nkt) gload(kt + 1);

    const int kbase = kt * BN;
    const bool active = (qw < Sq) && (!CAUSAL || kbase <= qw + 31);
    if (active) {
      const char* Ks = smem + st * C::STAGE_BYTES;
      const char* Vs = Ks + C::K_TILE_BYTES;

      f32x16 sacc[C::NKB];
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
        for (int j = 0; j < 16; ++j) sacc[kb][j] = 0.f;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const h8 a = *reinterpret_cast<const h8*>(Ks + swz<C::KCH>(32 * kb + r32, 2 * ks + hh));
          sacc[kb] = mfma_32x32x16(a, qreg[ks], sacc[kb]);
        }
      }

      const bool need_mask = (kbase + BN > Sk) || (CAUSAL && kbase + BN - 1 > qw);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = kbase + 32 * kb + 8 * (j >> 2) + 4 * hh + (j & 3);
            if (key >= Sk || (CAUSAL && key > qi)) sacc[kb][j] = kNegInf;
          }
      }

      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sacc[kb][j]);
      mx = xhalf_max(mx);
      const float m_new = fmaxf(m_run, mx * c2);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = exp2_fast(m_run - m_use);

      h8 pop[C::NKB][2];
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float p = exp2_fast(__builtin_fmaf(sacc[kb][j], c2, -m_use));
          psum += p;
          pop[kb][j >> 3][j & 7] = (_Float16)p;
        }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha;

#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            const h8 a = *reinterpret_cast<const h8*>(Vs + swz<C::VCH>(32 * db + r32, 4 * kb + 2 * k2 + hh));
            oacc[db] = mfma_32x32x16(a, pop[kb][k2], oacc[db]);
          }
    }

    if (kt + 1 < nkt) lstore(st ^ 1);
    __syncthreads();
  }

  // Epilogue: O = acc / l, LSE = (m + log2 l) * ln 2.  The O^T fragment is
  // transposed through LDS so each row leaves as coalesced 16-byte stores.
  const float l_tot = xhalf_sum(l_run);
  const float inv = 1.f / l_tot;
  char* Os = smem + w * (32 * D * 2);
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      const int d0 = 32 * db + 8 * jg + 4 * hh;
      h4 val;
      val[0] = (_Float16)(oacc[db][4 * jg + 0] * inv);
      val[1] = (_Float16)(oacc[db][4 * jg + 1] * inv);
      val[2] = (_Float16)(oacc[db][4 * jg + 2] * inv);
      val[3] = (_Float16)(oacc[db][4 * jg + 3] * inv);
      *reinterpret_cast<h4*>(Os + swz<C::KCH>(r32, d0 >> 3) + (d0 & 7) * 2) = val;
    }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < (32 * D / 8) / 64; ++u) {
    const int ci = lane + 64 * u;
    const int row = ci / C::KCH, c = ci % C::KCH;
    const int qrow = qw + row;
    if (qrow < Sq)
      *reinterpret_cast<u32x4*>(O + qoff + (size_t)qrow * D + c * 8) =
          *reinterpret_cast<const u32x4*>(Os + swz<C::KCH>(row, c));
  }
  if (hh == 0 && qi < Sq) LSE[(size_t)bh * Sq + qi] = (m_run + __builtin_log2f(l_tot)) * kLn2;
}

}  // namespace fa
