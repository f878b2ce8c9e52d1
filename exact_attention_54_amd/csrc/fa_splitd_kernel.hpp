// Exact attention forward for large heads (D = 512, 1024): Split-D.
//
// "FlashAttention-2 MMA", Supported Dispatch Strategies, 3. Split-D:
// partition the head dimension across parallel workers for head dims above
// 256.  Here the workers are the NW = D / 128 wavefronts of one workgroup,
// which share 32 query rows and each own one 128-wide slice of D:
//   * wavefront w computes the partial scores S_w^T = K[:, slice w] Q[:, slice w]^T
//     of a 32-key tile with its Q slice in registers;
//   * the NW partials are summed through LDS in a fixed order, so every
//     wavefront holds the same full S^T and takes the same online-softmax
//     decisions (running max, sum, rescale);
//   * wavefront w accumulates only its slice of the output,
//     O[:, slice w]^T += V[:, slice w]^T P, exactly like the D = 128 kernel.
// No product is computed twice.  K and V tiles (32 keys x D) stream through
// LDS with direct 16-byte copies, double-buffered at D = 512 and single-
// buffered at D = 1024 (LDS holds one 64 KiB K and V pair plus the partial
// scores).
#pragma once

#include "fa_device.hpp"

namespace fa {

template <int D>
struct SplitDCfg {
  static constexpr int NW = D / 128;
  static constexpr int THREADS = 64 * NW;
  static constexpr int BN = 32;
  static constexpr int C = D / 8;                    // 16-byte chunks per row
  static constexpr int TILE = BN * D * 2;            // one K or V tile
  static constexpr int NS = (D <= 512) ? 2 : 1;      // stages
  static constexpr int RED = NW * 64 * 16 * 4;       // partial scores, 16 fp32 per lane per wavefront
  static constexpr int BYTES = NS * 2 * TILE + RED;
  static_assert(BYTES <= 163840, "LDS budget");
  static_assert(TILE % (1024 * NW) == 0, "tile split");
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(64 * (D / 128), 1)
fwd_splitd_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
                  const _Float16* __restrict__ V, _Float16* __restrict__ O, float* __restrict__ LSE,
                  int Sq, int Sk, int BH, int nqt, float c2) {
  using C = SplitDCfg<D>;
  constexpr int NW = C::NW;
  __shared__ __attribute__((aligned(1024))) char smem[C::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // the D slice of this wavefront
  const int r32 = lane & 31;
  const int hh = lane >> 5;

  const int rank = blockIdx.x / BH;
  const int bh = blockIdx.x - rank * BH;
  const int qt = CAUSAL ? (nqt - 1 - rank) : rank;  // heaviest first
  const int q0 = qt * 32;
  const int qi = q0 + r32;

  const auto rq = make_rsrc(Q + (size_t)bh * Sq * D, (uint32_t)Sq * D * 2);
  const u32x4 rk = rsrc_words(K + (size_t)bh * Sk * D, (uint32_t)Sk * D * 2);
  const u32x4 rv = rsrc_words(V + (size_t)bh * Sk * D, (uint32_t)Sk * D * 2);
  const auto ro = make_rsrc(O + (size_t)bh * Sq * D, (uint32_t)Sq * D * 2);

  // this lane's query row, D slice w, as the B operand of S^T = K Q^T
  h8 qreg[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    qreg[ks] = as_h8(buf_load16(rq, ((uint32_t)qi * D + 128 * w + 16 * ks + 8 * hh) * 2u));

  const int nkt_all = (Sk + C::BN - 1) / C::BN;
  const int nkt = CAUSAL ? min(nkt_all, (min(q0 + 32, Sk) + C::BN - 1) / C::BN) : nkt_all;

  // direct copies: 1 KiB block b of a tile is filled by wavefront b % NW
  constexpr int BPW = C::TILE / 1024 / NW;
  uint32_t gk[BPW], gv[BPW];
#pragma unroll
  for (int u = 0; u < BPW; ++u) {
    const int p = (w + u * NW) * 1024 + lane * 16;
    int r, c;
    swz_inv<C::C>(p >> 8, (p >> 4) & 15, r, c);
    gk[u] = (uint32_t)(r * D + c * 8) * 2;
    vswz_inv<C::C>(p >> 8, (p >> 4) & 15, r, c);
    gv[u] = (uint32_t)(r * D + c * 8) * 2;
  }
  const uint32_t lds0 = lds_addr_of(smem);
  auto load_tile = [&](int kt, int st) {
    const uint32_t tb = (uint32_t)kt * C::TILE;
    const uint32_t base = lds0 + st * 2 * C::TILE;
#pragma unroll
    for (int u = 0; u < BPW; ++u) {
      dma16(rk, base + (w + u * NW) * 1024, tb + gk[u]);
      dma16(rv, base + C::TILE + (w + u * NW) * 1024, tb + gv[u]);
    }
  };
  float* red = reinterpret_cast<float*>(smem + C::NS * 2 * C::TILE);

  const int ti = lane & 15;
  const int tg = (lane >> 4) & 1;
  const int v_key = 4 * hh + (ti >> 2);
  const int v_chunk = 2 * tg + ((ti & 3) >> 1);
  const int v_half = (ti & 1) * 8;

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[db][j] = 0.f;
  float m_run = kNegInf, l_run = 0.f;

  if (nkt > 0) load_tile(0, 0);
  for (int kt = 0; kt < nkt; ++kt) {
    const int st = (C::NS == 2) ? (kt & 1) : 0;
    wait_vmem_all();
    __syncthreads();  // tile kt has landed; last tile's readers are done
    if (C::NS == 2 && kt + 1 < nkt) load_tile(kt + 1, st ^ 1);
    const char* Ks = smem + st * 2 * C::TILE;
    const char* Vs = Ks + C::TILE;

    // partial S^T over this wavefront's D slice
    f32x16 s;
#pragma unroll
    for (int j = 0; j < 16; ++j) s[j] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const h8 a = *reinterpret_cast<const h8*>(Ks + swz<C::C>(r32, 16 * w + 2 * ks + hh));
      s = mfma_32x32x16(a, qreg[ks], s);
    }
#pragma unroll
    for (int j = 0; j < 16; j += 4)
      *reinterpret_cast<f32x4*>(red + ((w * 64 + lane) * 16 + j)) = f32x4{s[j], s[j + 1], s[j + 2], s[j + 3]};
    __syncthreads();
    // full S^T: the partials summed in wavefront order (the same in every
    // wavefront, so all of them see bit-identical scores)
#pragma unroll
    for (int j = 0; j < 16; ++j) s[j] = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww)
#pragma unroll
      for (int j = 0; j < 16; j += 4) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(red + ((ww * 64 + lane) * 16 + j));
        s[j] += t[0];
        s[j + 1] += t[1];
        s[j + 2] += t[2];
        s[j + 3] += t[3];
      }
    // mask: key kt*32 + 8(j/4) + 4 hh + j%4 against Sk and the diagonal
    const int kbase = kt * C::BN + 4 * hh;
    const int lim = CAUSAL ? min(Sk - kbase - 1, qi - kbase) : Sk - kbase - 1;
    if (kt * C::BN + C::BN > Sk || (CAUSAL && kt * C::BN + C::BN - 1 > q0)) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (8 * (j >> 2) + (j & 3) > lim) s[j] = kNegInf;
    }
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < 16; j += 2) mx = fmaxf(fmaxf(mx, s[j]), s[j + 1]);
    const float m_new = fmaxf(m_run, xhalf_max(mx) * c2);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2_fast(m_run - m_use);
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha;
    m_run = m_new;
    h8 pop[2];
    const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int j = 0; j < 16; j += 2) {
      h2 pr;
      pr[0] = (_Float16)exp2_fast(__builtin_fmaf(s[j], c2, -m_use));
      pr[1] = (_Float16)exp2_fast(__builtin_fmaf(s[j + 1], c2, -m_use));
      l_run = dot2(pr, ones, l_run);
      pop[j >> 3][j & 7] = pr[0];
      pop[j >> 3][(j & 7) + 1] = pr[1];
    }
    // O[:, slice w]^T += V[:, slice w]^T P, V read transposed in the
    // accumulator's key order
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int key = 16 * k2 + v_key;
        const int chunk = 16 * w + 4 * db + v_chunk;
        const h4v lo = lds_read_tr16(Vs + vswz<C::C>(key, chunk) + v_half);
        const h4v hi = lds_read_tr16(Vs + vswz<C::C>(key + 8, chunk) + v_half);
        const h8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        oacc[db] = mfma_32x32x16(a, pop[k2], oacc[db]);
      }
    if (C::NS == 1 && kt + 1 < nkt) {
      __syncthreads();  // single stage: every wavefront is done with tile kt
      load_tile(kt + 1, 0);
    }
  }

  // epilogue: O = acc / l for this wavefront's slice, LSE from wavefront 0
  const float l_tot = xhalf_sum(l_run);
  const float inv = 1.f / l_tot;
  __syncthreads();
  char* tile = smem + w * (32 * 128 * 2);
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      const int d0 = 32 * db + 8 * jg + 4 * hh;
      h4 val;
      val[0] = (_Float16)(oacc[db][4 * jg + 0] * inv);
      val[1] = (_Float16)(oacc[db][4 * jg + 1] * inv);
      val[2] = (_Float16)(oacc[db][4 * jg + 2] * inv);
      val[3] = (_Float16)(oacc[db][4 * jg + 3] * inv);
      *reinterpret_cast<h4*>(tile + swz<16>(r32, d0 >> 3) + (d0 & 7) * 2) = val;
    }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < (32 * 128 / 8) / 64; ++u) {
    const int ci = lane + 64 * u;
    const int row = ci / 16, c = ci % 16;
    buf_store16(ro, ((uint32_t)(q0 + row) * D + 128 * w + c * 8) * 2u,
                *reinterpret_cast<const u32x4*>(tile + swz<16>(row, c)));
  }
  if (w == 0 && hh == 0 && qi < Sq) LSE[(size_t)bh * Sq + qi] = (m_run + __builtin_log2f(l_tot)) * kLn2;
}

}  // namespace fa
