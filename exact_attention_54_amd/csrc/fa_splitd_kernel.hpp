// Exact attention forward for large heads (D = 512, 1024): Split-D.
//
// "FlashAttention-2 MMA", Supported Dispatch Strategies, 3. Split-D:
// partition the head dimension across parallel workers for head dims above
// 256.  Here the workers are the NW = D / 128 wavefronts of one workgroup,
// which share 32 query rows and each own one 128-wide slice of D:
//   * wavefront w computes the partial scores S_w^T = K[:, slice w] Q[:, slice w]^T
//     of a 32-key tile with its Q slice in registers;
//   * the NW partials meet in LDS: wavefront w sums the w-th 1/NW of the
//     tile over all partials (in wavefront order), then every wavefront
//     reads the whole sum, so all of them hold the same full S^T and take
//     the same online-softmax decisions;
//   * wavefront w accumulates only its slice of the output,
//     O[:, slice w]^T += V[:, slice w]^T P, exactly like the D = 128 kernel.
// No product is computed twice.  K and V tiles (32 keys x D) stream through
// LDS by direct 16-byte copies, one buffer each: K of the next tile is
// copied while the scores are reduced and P V runs, V of the next tile while
// the next scores are formed.
//
// When the grid of (query tile, slice) work items is too small to fill the
// chip, the key range is also split ("Split-KV", same page, 2.) into ns
// contiguous parts; each part writes a normalised partial output and its
// log-sum-exp, and the split-KV merge kernel combines them exactly as for
// decoding ("Adaptive High-Performance Attention Kernels in CUDA", Advanced
// Production Features 1).
#pragma once

#include "fa_device.hpp"
#include "fa_fwd_kernel.hpp"

namespace fa {

template <int D>
struct SplitDCfg {
  static constexpr int NW = D / 128;
  static constexpr int THREADS = 64 * NW;
  static constexpr int BN = 32;
  static constexpr int C = D / 8;              // 16-byte chunks per row
  static constexpr int TILE = BN * D * 2;      // one K or V tile
  static constexpr int RED = NW * 64 * 16 * 4; // partial scores, 16 fp32 per lane per wavefront
  static constexpr int BYTES = 2 * TILE + RED;
  static constexpr int BPW = TILE / 1024 / NW; // 1 KiB copy blocks per wavefront and tile
  static constexpr int PER = 1024 / NW / 64;   // floats of the sum each lane produces
  static_assert(BYTES <= 163840, "LDS budget");
  static_assert(TILE % (1024 * NW) == 0, "tile split");
  static_assert(BPW < 16, "outstanding copies must fit the vmcnt field");
  static_assert(PER == 2 || PER == 4, "reduction piece");
};

// Float offset of element j of lane L's 16 partial scores: chunk-major,
// 16-byte chunk c of every lane in one contiguous 1 KiB run, so the 64 lanes
// writing (or reading back) one chunk touch 64 consecutive 16-byte slots.
// (A lane-major layout with the chunks XOR-permuted reads without bank
// conflicts on gfx950 but costs 8 conflict cycles per 16-byte write, as
// measured with SQ_LDS_BANK_CONFLICT.)  The flat offsets 0..1023 also
// partition the tile for the reduce-scatter into contiguous pieces.
__device__ __forceinline__ int red_off(int L, int j) { return (j >> 2) * 256 + L * 4 + (j & 3); }

// RUNS: the grid is split into runs of key tiles, as fwd_kernel does for
// D = 256 (KeySplit, fa_fwd_kernel.hpp): 32-row query tiles in split_order,
// one run per workgroup, each run a few segments, cut tiles written as fp32
// partials for fwd_split_merge_kernel.  Otherwise work item = key part s of
// a query tile (ns parts of equal length, merged by fwd_merge_kernel).
template <int D, bool CAUSAL, bool RUNS = false>
__global__ void __launch_bounds__(64 * (D / 128), 1)
fwd_splitd_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
                  const _Float16* __restrict__ V, _Float16* __restrict__ O, float* __restrict__ LSE,
                  int Sq, int Sk, int BH, int nqt, int ns, float c2, float* __restrict__ ws_o,
                  float* __restrict__ ws_lse, KeySplit ksp = {}) {
  using C = SplitDCfg<D>;
  constexpr int NW = C::NW;
  __shared__ __attribute__((aligned(1024))) char smem[C::BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // the D slice of this wavefront
  const int r32 = lane & 31;
  const int hh = lane >> 5;

  // parts: key part s of query-tile rank `rank` of slice bh
  int s = (int)(blockIdx.x % (unsigned)ns);
  int rank = (int)(blockIdx.x / (unsigned)ns) / BH;
  int bh = (int)(blockIdx.x / (unsigned)ns) - rank * BH;
  // runs: this workgroup's run (XCD-local, as in fwd_kernel)
  int run = 0, lin = 0, lin_end = 0;
  if constexpr (RUNS) {
    run = (int)(blockIdx.x & 7) * (int)(gridDim.x >> 3) + (int)(blockIdx.x >> 3);
    lin = (int)min(split_start(run, ksp.runs, ksp.total, ksp.bias), (long long)ksp.total);
    lin_end = (int)min(split_start(run + 1, ksp.runs, ksp.total, ksp.bias), (long long)ksp.total);
  }
  for (;;) {
  int seg_kb = 0, seg_ke = 0, seg_units = 0, tile_lin = 0;
  if constexpr (RUNS) {
    if (lin >= lin_end) return;
    bh = lin / ksp.units;
    const int off = lin - bh * ksp.units;
    int base = 0;
    for (int i = 0;; ++i) {
      rank = split_order(i, nqt);
      seg_units = fwd_tile_units(CAUSAL ? nqt - 1 - rank : rank, 32, C::BN, Sq, Sk, CAUSAL);
      if (off < base + seg_units || i == nqt - 1) break;
      base += seg_units;
    }
    seg_kb = off - base;
    seg_ke = min(seg_units, seg_kb + (lin_end - lin));
    tile_lin = lin - seg_kb;
    lin += seg_ke - seg_kb;
    s = 0;
  }
  const int qt = CAUSAL ? (nqt - 1 - rank) : rank;  // heaviest first
  const int q0 = qt * 32;
  const int qi = q0 + r32;

  const auto rq = make_rsrc(Q + (size_t)bh * Sq * D, (uint32_t)Sq * D * 2);
  const u32x4 rk = rsrc_words(K + (size_t)bh * Sk * D, (uint32_t)Sk * D * 2);
  const u32x4 rv = rsrc_words(V + (size_t)bh * Sk * D, (uint32_t)Sk * D * 2);

  // this lane's query row, D slice w, as the B operand of S^T = K Q^T
  h8 qreg[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    qreg[ks] = as_h8(buf_load16(rq, ((uint32_t)qi * D + 128 * w + 16 * ks + 8 * hh) * 2u));

  const int nkt_all = (Sk + C::BN - 1) / C::BN;
  const int nkt = CAUSAL ? min(nkt_all, (min(q0 + 32, Sk) + C::BN - 1) / C::BN) : nkt_all;
  const int kt0 = RUNS ? seg_kb : (int)((int64_t)s * nkt / ns);
  const int kt1 = RUNS ? seg_ke : (int)((int64_t)(s + 1) * nkt / ns);
  const bool cut = RUNS && (seg_kb > 0 || seg_ke < seg_units);  // a segment of a tile cut between runs

  // direct copies: 1 KiB block b of a tile is filled by wavefront b % NW
  uint32_t gk[C::BPW], gv[C::BPW];
#pragma unroll
  for (int u = 0; u < C::BPW; ++u) {
    const int p = (w + u * NW) * 1024 + lane * 16;
    int r, c;
    swz_inv<C::C>(p >> 8, (p >> 4) & 15, r, c);
    gk[u] = (uint32_t)(r * D + c * 8) * 2;
    vswz_inv<C::C>(p >> 8, (p >> 4) & 15, r, c);
    gv[u] = (uint32_t)(r * D + c * 8) * 2;
  }
  const uint32_t ldsk = lds_addr_of(smem);
  const uint32_t ldsv = ldsk + C::TILE;
  auto load_k = [&](int kt) {
#pragma unroll
    for (int u = 0; u < C::BPW; ++u) dma16(rk, ldsk + (w + u * NW) * 1024, (uint32_t)kt * C::TILE + gk[u]);
  };
  auto load_v = [&](int kt) {
#pragma unroll
    for (int u = 0; u < C::BPW; ++u) dma16(rv, ldsv + (w + u * NW) * 1024, (uint32_t)kt * C::TILE + gv[u]);
  };
  const char* Ks = smem;
  const char* Vs = smem + C::TILE;
  float* red = reinterpret_cast<float*>(smem + 2 * C::TILE);

  const int ti = lane & 15;
  const int tg = (lane >> 4) & 1;
  const int v_key = 4 * hh + (ti >> 2);
  const int v_chunk = 2 * tg + ((ti & 3) >> 1);
  const int v_half = (ti & 1) * 8;

  // the piece of the score tile this wavefront sums: PER consecutive floats
  // per lane starting at flat offset w * 1024 / NW + lane * PER (red_off is
  // chunk-major, so the pieces of consecutive lanes are contiguous)
  const int pofs = w * (1024 / NW) + lane * C::PER;

  f32x16 oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[db][j] = 0.f;
  float m_run = kNegInf, l_run = 0.f;

  if (kt0 < kt1) {
    load_k(kt0);
    load_v(kt0);
  }
  for (int kt = kt0; kt < kt1; ++kt) {
    const bool more = kt + 1 < kt1;
    wait_vmem_le<C::BPW>();  // K(kt) has landed (V(kt) may still be in flight)
    __syncthreads();

    // partial S^T over this wavefront's D slice
    f32x16 sc;
#pragma unroll
    for (int j = 0; j < 16; ++j) sc[j] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const h8 a = *reinterpret_cast<const h8*>(Ks + swz<C::C>(r32, 16 * w + 2 * ks + hh));
      sc = mfma_32x32x16(a, qreg[ks], sc);
    }
    float* mine = red + w * 1024;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *reinterpret_cast<f32x4*>(mine + red_off(lane, 4 * c)) =
          f32x4{sc[4 * c], sc[4 * c + 1], sc[4 * c + 2], sc[4 * c + 3]};
    __syncthreads();  // partials visible; every wavefront is done with K(kt)
    if (more) load_k(kt + 1);

    // reduce-scatter: this wavefront's piece summed over the partials in
    // wavefront order, written back in place of partial 0
    if constexpr (C::PER == 4) {
      f32x4 acc = *reinterpret_cast<const f32x4*>(red + pofs);
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(red + ww * 1024 + pofs);
        acc[0] += t[0];
        acc[1] += t[1];
        acc[2] += t[2];
        acc[3] += t[3];
      }
      *reinterpret_cast<f32x4*>(red + pofs) = acc;
    } else {
      f32x2 acc = *reinterpret_cast<const f32x2*>(red + pofs);
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) {
        const f32x2 t = *reinterpret_cast<const f32x2*>(red + ww * 1024 + pofs);
        acc[0] += t[0];
        acc[1] += t[1];
      }
      *reinterpret_cast<f32x2*>(red + pofs) = acc;
    }
    if (more)
      wait_vmem_le<C::BPW>();  // V(kt) has landed (K(kt+1) may still be in flight)
    else
      wait_vmem_all();
    __syncthreads();  // the full sum and V(kt) are visible

#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 t = *reinterpret_cast<const f32x4*>(red + red_off(lane, 4 * c));
      sc[4 * c] = t[0];
      sc[4 * c + 1] = t[1];
      sc[4 * c + 2] = t[2];
      sc[4 * c + 3] = t[3];
    }
    // mask: key kt*32 + 8(j/4) + 4 hh + j%4 against Sk and the diagonal
    const int kbase = kt * C::BN + 4 * hh;
    const int lim = CAUSAL ? min(Sk - kbase - 1, qi - kbase) : Sk - kbase - 1;
    if (kt * C::BN + C::BN > Sk || (CAUSAL && kt * C::BN + C::BN - 1 > q0)) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (8 * (j >> 2) + (j & 3) > lim) sc[j] = kNegInf;
    }
    // online softmax with the lazy reference max of the D = 128 kernel: the
    // reference moves only when a row max exceeds it by more than 2^8
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < 16; j += 2) mx = fmaxf(fmaxf(mx, sc[j]), sc[j + 1]);
    const float mt = xhalf_max(mx) * c2;
    const bool grow = mt > m_run + kLazyRescale;
    if (wave_any(grow)) {
      const float m_new = grow ? mt : m_run;
      const float alpha = exp2_fast(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;
    h8 pop[2];
    const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int j = 0; j < 16; j += 2) {
      h2 pr;
      pr[0] = (_Float16)exp2_fast(__builtin_fmaf(sc[j], c2, -m_use));
      pr[1] = (_Float16)exp2_fast(__builtin_fmaf(sc[j + 1], c2, -m_use));
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
    __syncthreads();  // every wavefront is done with V(kt) and the sum
    if (more) load_v(kt + 1);
  }

  const float l_tot = xhalf_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse = l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : kNegInf;
  if (cut) {
    // normalised fp32 partial O (this wavefront's slice) and the row's
    // log2-sum-exp, in the run's slot (split_slot) for the merge kernel
    if (qi < Sq) {
      const size_t slot = split_slot(run, tile_lin, ksp.runs, ksp.total, ksp.bias);
      float* dst = ksp.ws_o + (slot * 32 + r32) * D + 128 * w;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          const int d0 = 32 * db + 8 * jg + 4 * hh;
          *reinterpret_cast<f32x4*>(dst + d0) = f32x4{oacc[db][4 * jg] * inv, oacc[db][4 * jg + 1] * inv,
                                                      oacc[db][4 * jg + 2] * inv, oacc[db][4 * jg + 3] * inv};
        }
      if (w == 0 && hh == 0) ksp.ws_lse[slot * 32 + r32] = l_tot > 0.f ? m_run + __builtin_log2f(l_tot) : kNegInf;
    }
    __syncthreads();  // every wavefront is done with LDS before the next segment's copies
    continue;
  }
  if (!RUNS && ns > 1) {
    // partial for key part s: normalised O_s (fp32) and lse_s, rows of
    // [BH * Sq, ns, D]
    if (qi < Sq) {
      const size_t row = ((size_t)bh * Sq + qi) * ns + s;
      float* dst = ws_o + row * D + 128 * w;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int jg = 0; jg < 4; ++jg) {
          const int d0 = 32 * db + 8 * jg + 4 * hh;
          *reinterpret_cast<f32x4*>(dst + d0) = f32x4{oacc[db][4 * jg] * inv, oacc[db][4 * jg + 1] * inv,
                                                      oacc[db][4 * jg + 2] * inv, oacc[db][4 * jg + 3] * inv};
        }
      if (w == 0 && hh == 0) ws_lse[row] = lse;
    }
    return;
  }

  // epilogue: O = acc / l for this wavefront's slice through an LDS
  // transpose (16-byte coalesced stores), LSE from wavefront 0
  const auto ro = make_rsrc(O + (size_t)bh * Sq * D, (uint32_t)Sq * D * 2);
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
  if (w == 0 && hh == 0 && qi < Sq) LSE[(size_t)bh * Sq + qi] = lse;
  if constexpr (!RUNS) return;
  __syncthreads();  // the next segment refills LDS
  }
}

}  // namespace fa
