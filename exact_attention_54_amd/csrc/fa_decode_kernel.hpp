// Split-KV decoding for gfx950: one query row per (batch, head), the key
// range cut into num_splits contiguous partitions ("Adaptive High-Performance
// Attention Kernels in CUDA", Advanced Production Features, 1. Split-K
// FlashDecoding; "FlashAttention-2 MMA", Supported Dispatch Strategies,
// Split-KV).
//
// Phase one (decode_partial_kernel): one workgroup per (slice, partition).
// The work is a stream of K and V rows that are each used once, so it is
// bound by HBM bandwidth, not by arithmetic: no MFMA, and the loads are
// non-temporal.  A key row of D fp16 values is read by LPK = min(16, D/8)
// lanes with 16-byte loads, so each wavefront instruction moves 64 x 16
// contiguous bytes (4 key rows at D = 128).  Every lane keeps an independent online softmax over the keys
// of its slot; the 4 x SLOTS slot states of a workgroup are merged through
// LDS at the end into one normalised partial output O_s and lse_s.
//
// Phase two (decode_merge_kernel): per slice, lse = ln sum_s exp(lse_s) and
// O = sum_s exp(lse_s - lse) O_s, rounded to fp16.
#pragma once

#include "fa_device.hpp"

namespace fa {

template <int D>
struct DecCfg {
  static constexpr int THREADS = 256;
  static constexpr int NWAVES = THREADS / 64;
  static constexpr int LPK = (D / 8 < 16) ? D / 8 : 16;  // lanes per key row
  static constexpr int CPL = (D / 8) / LPK;              // 16-byte chunks per lane
  static constexpr int SLOTS = 64 / LPK;                 // key rows per wavefront load
  static constexpr int U = 4;                            // loads in flight per lane and tensor
  static constexpr int KEYS_PER_WAVE_ITER = SLOTS * U;
  static constexpr int KEYS_PER_WG_ITER = NWAVES * KEYS_PER_WAVE_ITER;
  static constexpr int NSTATE = NWAVES * SLOTS;          // independent softmax states per workgroup
};

// ws_o: [BH, ns, D] fp32, ws_lse: [BH, ns] fp32 (natural log).
template <int D>
__global__ void __launch_bounds__(256)
decode_partial_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
                      const _Float16* __restrict__ V, float* __restrict__ ws_o,
                      float* __restrict__ ws_lse, int Sk, int ns, int chunk, float c2) {
  using C = DecCfg<D>;
  __shared__ float s_m[C::NSTATE];
  __shared__ float s_l[C::NSTATE];
  __shared__ __attribute__((aligned(16))) float s_acc[C::NSTATE][D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int slot = lane / C::LPK;
  const int dl = lane % C::LPK;
  const int bh = blockIdx.x / ns;
  const int s = blockIdx.x - bh * ns;
  const int k0 = s * chunk;
  const int k1 = min(Sk, k0 + chunk);
  float* out_o = ws_o + ((size_t)bh * ns + s) * D;

  if (k0 >= k1) {  // empty partition: weight zero in the merge
    for (int d = tid; d < D; d += C::THREADS) out_o[d] = 0.f;
    if (tid == 0) ws_lse[(size_t)bh * ns + s] = kNegInf;
    return;
  }

  const _Float16* qp = Q + (size_t)bh * D;
  const _Float16* kp = K + (size_t)bh * Sk * D;
  const _Float16* vp = V + (size_t)bh * Sk * D;

  float qf[C::CPL][8];
#pragma unroll
  for (int c = 0; c < C::CPL; ++c) {
    const h8 t = as_h8(*reinterpret_cast<const u32x4*>(qp + (dl + c * C::LPK) * 8));
#pragma unroll
    for (int e = 0; e < 8; ++e) qf[c][e] = (float)t[e];
  }

  float m_run = kNegInf, l_run = 0.f;
  float acc[C::CPL][8];
#pragma unroll
  for (int c = 0; c < C::CPL; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[c][e] = 0.f;

  for (int base = k0 + w * C::KEYS_PER_WAVE_ITER; base < k1; base += C::KEYS_PER_WG_ITER) {
    u32x4 kr[C::U][C::CPL], vr[C::U][C::CPL];
#pragma unroll
    for (int u = 0; u < C::U; ++u) {
      const int key = base + u * C::SLOTS + slot;
#pragma unroll
      for (int c = 0; c < C::CPL; ++c) {
        u32x4 tk = {0u, 0u, 0u, 0u}, tv = {0u, 0u, 0u, 0u};
        if (key < k1) {
          // read once: non-temporal loads keep the stream from evicting
          // useful cache lines (measured ~13% more HBM bandwidth)
          const size_t off = (size_t)key * D + (dl + c * C::LPK) * 8;
          tk = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + off));
          tv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + off));
        }
        kr[u][c] = tk;
        vr[u][c] = tv;
      }
    }
    float sc[C::U];
#pragma unroll
    for (int u = 0; u < C::U; ++u) {
      float part = 0.f;
#pragma unroll
      for (int c = 0; c < C::CPL; ++c) {
        const h8 kh = as_h8(kr[u][c]);
#pragma unroll
        for (int e = 0; e < 8; ++e) part = __builtin_fmaf(qf[c][e], (float)kh[e], part);
      }
#pragma unroll
      for (int off = 1; off < C::LPK; off <<= 1) part += __shfl_xor(part, off);
      const int key = base + u * C::SLOTS + slot;
      sc[u] = (key < k1) ? part : kNegInf;
    }
    float mx = sc[0];
#pragma unroll
    for (int u = 1; u < C::U; ++u) mx = fmaxf(mx, sc[u]);
    const float m_new = fmaxf(m_run, mx * c2);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2_fast(m_run - m_use);
    l_run *= alpha;
#pragma unroll
    for (int c = 0; c < C::CPL; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[c][e] *= alpha;
#pragma unroll
    for (int u = 0; u < C::U; ++u) {
      const float p = exp2_fast(__builtin_fmaf(sc[u], c2, -m_use));
      l_run += p;
#pragma unroll
      for (int c = 0; c < C::CPL; ++c) {
        const h8 vh = as_h8(vr[u][c]);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[c][e] = __builtin_fmaf(p, (float)vh[e], acc[c][e]);
      }
    }
    m_run = m_new;
  }

  // Merge the NSTATE slot states of this workgroup.
  const int st = w * C::SLOTS + slot;
  if (dl == 0) {
    s_m[st] = m_run;
    s_l[st] = l_run;
  }
#pragma unroll
  for (int c = 0; c < C::CPL; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) s_acc[st][(dl + c * C::LPK) * 8 + e] = acc[c][e];
  __syncthreads();

  float M = kNegInf;
#pragma unroll
  for (int i = 0; i < C::NSTATE; ++i) M = fmaxf(M, s_m[i]);
  for (int d = tid; d < D; d += C::THREADS) {
    float den = 0.f, num = 0.f;
#pragma unroll
    for (int i = 0; i < C::NSTATE; ++i) {
      const float wgt = exp2_fast(s_m[i] - M);  // 0 for a slot that saw no key
      den += wgt * s_l[i];
      num += wgt * s_acc[i][d];
    }
    out_o[d] = num / den;
    if (d == 0) ws_lse[(size_t)bh * ns + s] = (M + __builtin_log2f(den)) * kLn2;
  }
}

template <int D>
__global__ void __launch_bounds__(256)
decode_merge_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_lse,
                    _Float16* __restrict__ O, float* __restrict__ LSE, int ns) {
  const int bh = blockIdx.x;
  const float* lp = ws_lse + (size_t)bh * ns;
  const float* op = ws_o + (size_t)bh * ns * D;
  float M = kNegInf;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, lp[s]);
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float den = 0.f, num = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float wgt = exp2_fast((lp[s] - M) * kLog2e);
      den += wgt;
      num += wgt * op[(size_t)s * D + d];
    }
    O[(size_t)bh * D + d] = (_Float16)(num / den);
    if (d == 0) LSE[bh] = M + __builtin_logf(den);
  }
}

}  // namespace fa
