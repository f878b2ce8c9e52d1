// Exact attention backward for gfx950, from the forward's log-sum-exp.
//
// The pages' backward ("Adaptive High-Performance Attention Kernels in
// CUDA", Advanced Production Features, 2. Custom CUDA Backward Pass)
// recomputes S = Q K^T * scale and P = exp(S - m) / l from the forward
// statistics (here P = exp(S - LSE)), precomputes D_i = sum_d dO_id O_id and
// forms dS = P o (dP - D) with dP = dO V^T, never storing P.  Then
//   dV = P^T dO,   dK = scale * dS^T Q,   dQ = scale * dS K.
//
// Two kernels, no atomics, the dQ kernel first:
//   bwd_dq_kernel     one workgroup per (slice, 32*NW queries); each
//                     wavefront owns 32 queries (Q and dO rows in registers)
//                     and streams 64-key tiles of K and V through LDS:
//                     S^T = K Q^T and dP^T = V dO^T put one query in each
//                     lane, and dQ^T += K^T dS^T reads K transposed, like the
//                     forward reads V.  It forms D_i = dO_i . O_i (fp32) from
//                     the dO row it holds and writes D and the LSE in log2
//                     units for the next kernel.
//   bwd_dkdv_kernel   one workgroup per (slice, 32*NW keys); each wavefront
//                     owns 32 keys (K and V rows in registers) and streams
//                     32-query tiles of Q, dO, LSE and D through LDS:
//                     S = Q K^T and dP = dO V^T put one key in each lane, so
//                     P and dS feed dV^T += dO^T P and dK^T += Q^T dS
//                     straight from registers, with dO and Q read
//                     transposed from LDS in the matching (permuted) query
//                     order -- the forward's P V trick with queries and keys
//                     exchanged.
// Q/dO tiles (dkdv) and K tiles (dq) are read both row-wise and transposed,
// so they use bswz, an XOR swizzle conflict-free for both reads.  Tiles go
// HBM -> LDS with 16-byte direct copies one tile ahead of their use.
#pragma once

#include <type_traits>

#include "fa_device.hpp"

namespace fa {

// Row-major LDS layout read both by 16-byte row reads (16 consecutive rows,
// one chunk column) and by ds_read_b64_tr_b16 (4 consecutive rows x 4
// consecutive chunks): the XOR key swaps the two 2-bit halves of the row
// index, which keeps both groups of 16 chunks on 16 distinct 16-byte bank
// groups of a 256-byte line.  Rows of 4 chunks (D = 32) share a line four
// at a time, and XOR the chunk with the line index instead.
template <int C>
__host__ __device__ __forceinline__ uint32_t bswz(int r, int c) {
  static_assert(C == 4 || C == 8 || C == 16 || C == 32, "chunks per row");
  if constexpr (C >= 16) {
    const int line = r * (C / 16) + (c >> 4);
    const int slot = (c & 15) ^ (((r & 3) << 2) | ((r >> 2) & 3));
    return (uint32_t)(line * 256 + slot * 16);
  } else if constexpr (C == 8) {
    const int line = r >> 1;
    const int slot = (r & 1) * 8 + (c ^ (((line & 1) << 2) | ((line >> 1) & 3)));
    return (uint32_t)(line * 256 + slot * 16);
  } else {
    const int line = r >> 2;
    const int slot = (r & 3) * 4 + (c ^ (line & 3));
    return (uint32_t)(line * 256 + slot * 16);
  }
}
template <int C>
__host__ __device__ __forceinline__ void bswz_inv(int line, int slot, int& r, int& c) {
  if constexpr (C >= 16) {
    r = line / (C / 16);
    c = (line % (C / 16)) * 16 + (slot ^ (((r & 3) << 2) | ((r >> 2) & 3)));
  } else if constexpr (C == 8) {
    r = line * 2 + slot / 8;
    c = (slot % 8) ^ (((line & 1) << 2) | ((line >> 1) & 3));
  } else {
    r = line * 4 + slot / 4;
    c = (slot % 4) ^ (line & 3);
  }
}

// ------------------------------------------------------------- shared pieces

template <int D, int NW>
struct BwdCfg {
  static constexpr int THREADS = 64 * NW;
  static constexpr int KCH = D / 8;   // 16-byte chunks per row
  static constexpr int KS = D / 16;   // k-steps of a D contraction
  static constexpr int NDB = D / 32;  // 32-wide d blocks
};

// Transposed A operand (32 d x 16 contraction rows) of a 32x32x16 MFMA from a
// row-major [row][d] LDS tile: rows taken in the permuted order in which the
// 32x32 accumulator lists them (block r0 = 32 rows, k2 = which 16), d block
// db.  Same addressing as the forward's V reads.
template <int C, class Swz>
__device__ __forceinline__ h8 tr_operand(const char* base, int r0, int k2, int db, int lane, Swz swzf) {
  const int ti = lane & 15;
  const int tg = (lane >> 4) & 1;
  const int hh = lane >> 5;
  const int row = r0 + 16 * k2 + 4 * hh + (ti >> 2);
  const int chunk = 4 * db + 2 * tg + ((ti & 3) >> 1);
  const int half = (ti & 1) * 8;
  const h4v lo = lds_read_tr16(base + swzf(row, chunk) + half);
  const h4v hi = lds_read_tr16(base + swzf(row + 8, chunk) + half);
  return h8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Epilogue shared by the three outputs: an accumulator whose lane l holds
// column l%32 (a row of the output) and d = 32 db + 8(j/4) + 4(l/32) + j%4,
// scaled, rounded to fp16 and transposed through this wavefront's 32 x D
// LDS tile so each output row leaves as 16-byte stores (rows past `rows`
// are dropped by the buffer bounds).
template <int D>
__device__ __forceinline__ void store_rows(const f32x16 (&acc)[D / 32], float scale, char* tile,
                                           __amdgpu_buffer_rsrc_t rout, int row0, int lane) {
  constexpr int KCH = D / 8;
  const int r32 = lane & 31;
  const int hh = lane >> 5;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int jg = 0; jg < 4; ++jg) {
      const int d0 = 32 * db + 8 * jg + 4 * hh;
      h4 val;
      val[0] = (_Float16)(acc[db][4 * jg + 0] * scale);
      val[1] = (_Float16)(acc[db][4 * jg + 1] * scale);
      val[2] = (_Float16)(acc[db][4 * jg + 2] * scale);
      val[3] = (_Float16)(acc[db][4 * jg + 3] * scale);
      *reinterpret_cast<h4*>(tile + swz<KCH>(r32, d0 >> 3) + (d0 & 7) * 2) = val;
    }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < (32 * D / 8) / 64; ++u) {
    const int ci = lane + 64 * u;
    const int row = ci / KCH, c = ci % KCH;
    buf_store16(rout, ((uint32_t)(row0 + row) * D + c * 8) * 2u, *reinterpret_cast<const u32x4*>(tile + swz<KCH>(row, c)));
  }
}

// Workgroups per CU the register budget is sized for: two below D = 256;
// at D = 256 the fp32 gradient accumulators of a wavefront alone take 256
// registers per lane, so one (the wavefront then has the SIMD's whole
// register file).
template <int D>
constexpr int bwd_wg_per_cu() { return D > 128 ? 1 : 2; }

// --------------------------------------------------------------- dK and dV

// LDS: the workgroup's V rows (32 NW x D fp16, swz), then per stage a Q
// tile, a dO tile (32 x D fp16 each, bswz) and 32 LSE (log2 units) + 32 D
// values.
template <int D, int NW>
struct DkdvLds {
  static constexpr int VROWS = 32 * NW * D * 2;
  static constexpr int TILE = 32 * D * 2;
  static constexpr int STAGE = 2 * TILE + 256;
  static constexpr int BYTES = VROWS + 2 * STAGE;
};

// LDS bytes of a workgroup (dynamic LDS, passed at launch; above 64 KiB,
// at D = 256, the kernel must be allowed that much first).
template <int D, int NW>
constexpr int dkdv_lds_bytes() {
  return (DkdvLds<D, NW>::BYTES > NW * 32 * D * 2) ? DkdvLds<D, NW>::BYTES : NW * 32 * D * 2;
}

template <int D, int NW, bool CAUSAL>
__global__ void __launch_bounds__(64 * NW, bwd_wg_per_cu<D>())
bwd_dkdv_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K, const _Float16* __restrict__ V,
                const _Float16* __restrict__ dO, const float* __restrict__ L2, const float* __restrict__ Dv,
                _Float16* __restrict__ dK, _Float16* __restrict__ dV, int Sq, int Sk, int BH, int nkt, float scale) {
  using C = BwdCfg<D, NW>;
  using L = DkdvLds<D, NW>;
  extern __shared__ __attribute__((aligned(1024))) char smem[];  // dkdv_lds_bytes<D, NW>(), passed at launch

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31;
  const int hh = lane >> 5;
  const int kt = blockIdx.x / BH;
  const int bh = blockIdx.x - kt * BH;
  const int k0 = kt * 32 * NW;
  const int kw = k0 + 32 * w;  // first key of this wavefront
  const int key = kw + r32;    // the key this lane's accumulator columns belong to
  const float c2 = scale * kLog2e;

  const u32x4 rq = rsrc_words(Q + (size_t)bh * Sq * D, (uint32_t)Sq * D * 2);
  const u32x4 rdo = rsrc_words(dO + (size_t)bh * Sq * D, (uint32_t)Sq * D * 2);
  const auto rk = make_rsrc(K + (size_t)bh * Sk * D, (uint32_t)Sk * D * 2);
  const u32x4 rv = rsrc_words(V + (size_t)bh * Sk * D, (uint32_t)Sk * D * 2);
  const u32x4 rl = rsrc_words(L2 + (size_t)bh * Sq, (uint32_t)Sq * 4);
  const u32x4 rd = rsrc_words(Dv + (size_t)bh * Sq, (uint32_t)Sq * 4);

  // K rows of this wavefront as the B operand of S = Q K^T: lane l holds
  // d = 16 ks + 8 (l/32) .. +7 of key l%32.  The V rows, the B operand of
  // dP = dO V^T, are read from LDS in the same pattern (registers are the
  // scarcer resource here).
  h8 kreg[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks)
    kreg[ks] = as_h8(buf_load16(rk, ((uint32_t)key * D + 16 * ks + 8 * hh) * 2u));

  // Query tiles: all of them, or from the diagonal on when causal.
  const int qt0 = CAUSAL ? (k0 / 32) : 0;
  const int nqt = (Sq + 31) / 32;

  // Direct 16-byte HBM -> LDS copies of the 32 x D Q and dO tiles: 1 KiB
  // block b of a tile is filled by wavefront b % NW, lane l's 16 bytes
  // landing at 16 l of it, and the (row, chunk) that belongs there is found
  // through the inverse swizzle.  Rows past Sq read as zeros.
  constexpr int BLK = L::TILE / 1024;  // 1 KiB blocks per tile
  constexpr int BPW = (BLK + NW - 1) / NW;
  uint32_t go[BPW];
#pragma unroll
  for (int u = 0; u < BPW; ++u) {
    const int p = ((w + u * NW) % BLK) * 1024 + lane * 16;
    int r, c;
    bswz_inv<C::KCH>(p >> 8, (p >> 4) & 15, r, c);
    go[u] = (uint32_t)(r * D + c * 8) * 2;
  }
  const uint32_t lds0 = lds_addr_of(smem);
  // the workgroup's 32 NW V rows, copied once (rows past Sk read as zeros)
  {
    constexpr int VBLK = L::VROWS / 1024;
    static_assert(VBLK % NW == 0, "V rows split");
#pragma unroll
    for (int u = 0; u < VBLK / NW; ++u) {
      const int b = w + u * NW;
      const int p = b * 1024 + lane * 16;
      int r, c;
      swz_inv<C::KCH>(p >> 8, (p >> 4) & 15, r, c);
      dma16(rv, lds0 + b * 1024, (uint32_t)((k0 + r) * D + c * 8) * 2);
    }
  }
  const char* Vw = smem;  // V rows of this workgroup, [32 NW][D] swz
  auto load_stage = [&](int st, int q0) {
    const uint32_t base = lds0 + L::VROWS + st * L::STAGE;
    const uint32_t tb = (uint32_t)q0 * D * 2;
#pragma unroll
    for (int u = 0; u < BPW; ++u) {
      const int b = w + u * NW;
      if (b < BLK) {
        dma16(rq, base + b * 1024, tb + go[u]);
        dma16(rdo, base + L::TILE + b * 1024, tb + go[u]);
      }
    }
    // LSE (log2 units) to lanes 0..31, D to 32..63 of one 256-byte block;
    // padding rows read zeros and are masked where P is formed
    if (w == 0) {
      if (lane < 32) dma4(rl, base + 2 * L::TILE, (uint32_t)(q0 + lane) * 4);
      else dma4(rd, base + 2 * L::TILE, (uint32_t)(q0 + lane - 32) * 4);
    }
  };

  f32x16 dvt[C::NDB], dkt[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      dvt[db][j] = 0.f;
      dkt[db][j] = 0.f;
    }

  if (qt0 < nqt) load_stage(0, qt0 * 32);
  wait_vmem_all();
  __syncthreads();
  for (int qt = qt0; qt < nqt; ++qt) {
    const int st = (qt - qt0) & 1;
    // the other stage was released by the last barrier; its copies land
    // while this tile is computed
    if (qt + 1 < nqt) load_stage(st ^ 1, (qt + 1) * 32);
    const int q0 = qt * 32;
    const char* Qs = smem + L::VROWS + st * L::STAGE;
    const char* dOs = Qs + L::TILE;
    const float* lv = reinterpret_cast<const float*>(Qs + 2 * L::TILE);
    // a wavefront whose keys all come after the tile's last query sees none
    const bool active = !CAUSAL || kw <= q0 + 31;
    if (active && kw < Sk) {
      f32x16 s, dp;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        s[j] = 0.f;
        dp[j] = 0.f;
      }
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const h8 aq = *reinterpret_cast<const h8*>(Qs + bswz<C::KCH>(r32, 2 * ks + hh));
        s = mfma_32x32x16(aq, kreg[ks], s);
        const h8 ado = *reinterpret_cast<const h8*>(dOs + bswz<C::KCH>(r32, 2 * ks + hh));
        const h8 bv = *reinterpret_cast<const h8*>(Vw + swz<C::KCH>(32 * w + r32, 2 * ks + hh));
        dp = mfma_32x32x16(ado, bv, dp);
      }
      // accumulator j holds query q0 + 4 hh + c, c = 8(j/4) + j%4, of key
      // `key`; it is kept for lo <= c < hi (key < Sk, query < Sq, and
      // key <= query when causal), one unsigned compare against a constant.
      // Masked entries take exp2(-inf) = 0, without a branch.
      h8 pop[2], dsop[2];
      const int lo = CAUSAL ? max(key - q0 - 4 * hh, 0) : 0;
      const int hi = (key < Sk) ? max(min(Sq - q0 - 4 * hh, 32), lo) : lo;
      const unsigned span = (unsigned)(hi - lo);
#pragma unroll
      for (int jg = 0; jg < 4; ++jg) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lv + 8 * jg + 4 * hh);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(lv + 32 + 8 * jg + 4 * hh);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = 4 * jg + i;
          const bool keep = (unsigned)(8 * jg + i - lo) < span;
          const float p = exp2_fast(keep ? __builtin_fmaf(s[j], c2, -l4[i]) : kNegInf);
          const float ds = p * (dp[j] - d4[i]);
          pop[j >> 3][j & 7] = (_Float16)p;
          dsop[j >> 3][j & 7] = (_Float16)ds;
        }
      }
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          const h8 a_do = tr_operand<C::KCH>(dOs, 0, k2, db, lane, [](int r, int c) { return bswz<C::KCH>(r, c); });
          dvt[db] = mfma_32x32x16(a_do, pop[k2], dvt[db]);
          const h8 a_q = tr_operand<C::KCH>(Qs, 0, k2, db, lane, [](int r, int c) { return bswz<C::KCH>(r, c); });
          dkt[db] = mfma_32x32x16(a_q, dsop[k2], dkt[db]);
        }
    }
    wait_vmem_all();
    __syncthreads();  // this stage's readers are done; the next stage has landed
  }

  // dV = (dV^T)^T, dK = scale (dK^T)^T, each wavefront's 32 key rows
  char* tile = smem + w * (32 * D * 2);
  const auto rdv = make_rsrc(dV + (size_t)bh * Sk * D, (uint32_t)Sk * D * 2);
  const auto rdk = make_rsrc(dK + (size_t)bh * Sk * D, (uint32_t)Sk * D * 2);
  store_rows<D>(dvt, 1.f, tile, rdv, kw, lane);
  __syncthreads();
  store_rows<D>(dkt, scale, tile, rdk, kw, lane);
}

// -------------------------------------------------------------------- dQ

template <int D>
struct DqLds {
  static constexpr int BN = 64;
  static constexpr int TILE = BN * D * 2;
  static constexpr int BYTES = 4 * TILE;  // K0 K1 V0 V1
};

template <int D, int NW>
constexpr int dq_lds_bytes() {
  return (DqLds<D>::BYTES > NW * 32 * D * 2) ? DqLds<D>::BYTES : NW * 32 * D * 2;
}

template <int D, int NW, bool CAUSAL>
__global__ void __launch_bounds__(64 * NW, bwd_wg_per_cu<D>())
bwd_dq_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K, const _Float16* __restrict__ V,
              const _Float16* __restrict__ O, const _Float16* __restrict__ dO, const float* __restrict__ LSE,
              float* __restrict__ L2, float* __restrict__ Dv, _Float16* __restrict__ dQ, int Sq, int Sk, int BH,
              int nqt, float scale) {
  using C = BwdCfg<D, NW>;
  using L = DqLds<D>;
  constexpr int BN = L::BN;
  constexpr int NKB = BN / 32;
  extern __shared__ __attribute__((aligned(1024))) char smem[];  // dq_lds_bytes<D, NW>(), passed at launch

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r32 = lane & 31;
  const int hh = lane >> 5;
  const int rank = blockIdx.x / BH;
  const int bh = blockIdx.x - rank * BH;
  const int qt = CAUSAL ? (nqt - 1 - rank) : rank;  // heaviest first
  const int q0 = qt * 32 * NW;
  const int qw = q0 + 32 * w;
  const int qi = qw + r32;  // this lane's query
  const float c2 = scale * kLog2e;

  const auto rq = make_rsrc(Q + (size_t)bh * Sq * D, (uint32_t)Sq * D * 2);
  const auto rdo = make_rsrc(dO + (size_t)bh * Sq * D, (uint32_t)Sq * D * 2);
  const u32x4 rk = rsrc_words(K + (size_t)bh * Sk * D, (uint32_t)Sk * D * 2);
  const u32x4 rv = rsrc_words(V + (size_t)bh * Sk * D, (uint32_t)Sk * D * 2);

  const int nkt_all = (Sk + BN - 1) / BN;
  const int nkt = CAUSAL ? min(nkt_all, (min(q0 + 32 * NW, Sk) + BN - 1) / BN) : nkt_all;
  const int jlast = (qw >= Sq) ? -1 : (CAUSAL ? min(nkt - 1, (qw + 31) / BN) : nkt - 1);

  // Direct 16-byte HBM -> LDS copies of the 64 x D K (bswz) and V (swz)
  // tiles, 1 KiB blocks spread over the wavefronts as in the dK/dV kernel.
  constexpr int BLK = L::TILE / 1024;
  constexpr int BPW = (BLK + NW - 1) / NW;
  uint32_t gk[BPW], gv[BPW];
#pragma unroll
  for (int u = 0; u < BPW; ++u) {
    const int p = ((w + u * NW) % BLK) * 1024 + lane * 16;
    int r, c;
    bswz_inv<C::KCH>(p >> 8, (p >> 4) & 15, r, c);
    gk[u] = (uint32_t)(r * D + c * 8) * 2;
    swz_inv<C::KCH>(p >> 8, (p >> 4) & 15, r, c);
    gv[u] = (uint32_t)(r * D + c * 8) * 2;
  }
  const uint32_t lds0 = lds_addr_of(smem);
  auto load_stage = [&](int st, int kt) {
    const uint32_t tb = (uint32_t)kt * L::TILE;
#pragma unroll
    for (int u = 0; u < BPW; ++u) {
      const int b = w + u * NW;
      if (b < BLK) {
        dma16(rk, lds0 + st * L::TILE + b * 1024, tb + gk[u]);
        dma16(rv, lds0 + 2 * L::TILE + st * L::TILE + b * 1024, tb + gv[u]);
      }
    }
  };

  // Q and dO rows of this lane's query as the B operands of S^T = K Q^T and
  // dP^T = V dO^T (this lane's half of each 16-wide step), its LSE in log2
  // units and D = dO . O: this lane's half of the dot product, then the
  // other half's from lane ^ 32.  Both go to L2 / Dv for the dK/dV kernel.
  // The row loads and the first K / V tile copy are all issued before any
  // of them is waited for (one memory round trip before the loop).
  const auto ro = make_rsrc(O + (size_t)bh * Sq * D, (uint32_t)Sq * D * 2);
  const bool qvalid = qi < Sq;
  // read unconditionally (rows past Sq read row Sq - 1 and are not used), so
  // no branch around the load makes its use wait at once
  const float lse_in = LSE[(size_t)bh * Sq + min(qi, Sq - 1)];
  h8 qreg[C::KS], doreg[C::KS], oreg[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const uint32_t off = ((uint32_t)qi * D + 16 * ks + 8 * hh) * 2u;
    qreg[ks] = as_h8(buf_load16(rq, off));
    doreg[ks] = as_h8(buf_load16(rdo, off));
    oreg[ks] = as_h8(buf_load16(ro, off));
  }
  if (nkt > 0) load_stage(0, 0);
  __builtin_amdgcn_sched_barrier(0);  // the uses below stay after the copies' issue
  float dhalf = 0.f;
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) dhalf = __builtin_fmaf((float)oreg[ks][e], (float)doreg[ks][e], dhalf);
  const float dval = qvalid ? xhalf_sum(dhalf) : 0.f;
  const float lse2 = qvalid ? lse_in * kLog2e : __builtin_huge_valf();
  if (qvalid && hh == 0) {
    L2[(size_t)bh * Sq + qi] = lse2;
    Dv[(size_t)bh * Sq + qi] = dval;
  }

  f32x16 dqt[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) dqt[db][j] = 0.f;

  wait_vmem_all();
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nkt) load_stage(st ^ 1, kt + 1);
    const char* Ks = smem + st * L::TILE;
    const char* Vs = smem + 2 * L::TILE + st * L::TILE;
    if (kt <= jlast) {
      f32x16 s[NKB], dp[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          s[kb][j] = 0.f;
          dp[kb][j] = 0.f;
        }
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          const h8 ak = *reinterpret_cast<const h8*>(Ks + bswz<C::KCH>(32 * kb + r32, 2 * ks + hh));
          s[kb] = mfma_32x32x16(ak, qreg[ks], s[kb]);
          const h8 av = *reinterpret_cast<const h8*>(Vs + swz<C::KCH>(32 * kb + r32, 2 * ks + hh));
          dp[kb] = mfma_32x32x16(av, doreg[ks], dp[kb]);
        }
      }
      // accumulator j of block kb holds key kt*BN + 4 hh + c with
      // c = 32 kb + 8(j/4) + j%4; it is kept for c <= lim (key < Sk, and
      // key <= query when causal): one compare against a constant
      h8 dsop[NKB][2];
      const int kbase = kt * BN + 4 * hh;
      const int lim = CAUSAL ? min(Sk - 1, qi) - kbase : Sk - 1 - kbase;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const bool keep = 32 * kb + 8 * (j >> 2) + (j & 3) <= lim;
          const float p = exp2_fast(keep ? __builtin_fmaf(s[kb][j], c2, -lse2) : kNegInf);
          dsop[kb][j >> 3][j & 7] = (_Float16)(p * (dp[kb][j] - dval));
        }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int db = 0; db < C::NDB; ++db) {
            const h8 a = tr_operand<C::KCH>(Ks, 32 * kb, k2, db, lane, [](int r, int c) { return bswz<C::KCH>(r, c); });
            dqt[db] = mfma_32x32x16(a, dsop[kb][k2], dqt[db]);
          }
    }
    wait_vmem_all();
    __syncthreads();
  }

  char* tile = smem + w * (32 * D * 2);
  const auto rdq = make_rsrc(dQ + (size_t)bh * Sq * D, (uint32_t)Sq * D * 2);
  store_rows<D>(dqt, scale, tile, rdq, qw, lane);
}

}  // namespace fa
