// Exact attention forward (prefill) for gfx950, FlashAttention-2 loop order.
//
// One workgroup = NW wavefronts = BM = 32*NW query rows ("Split-Q"; the loop
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
//   online softmax  p = 2^(s*c - m), l += rowsum(p), with c = scale*log2(e)
//                 folded into one FMA per score ("FlashAttention-2 MMA",
//                 Technical Details, Online Softmax).  The reference max m
//                 is not taken per tile: a lane's share of the tile's row
//                 sum bounds every p it formed, so while that share stays
//                 <= 2^15 P is inside fp16's range at full relative
//                 precision and m stays.  When it does not (a row's first
//                 tile, or a row max that grew by ~2^15) m moves to the
//                 tile's row max, O and l are rescaled by 2^(m - m_new) and
//                 P is formed again.  Only rounding differs from moving m on
//                 every tile.
//   O^T += V^T P^T  P is rounded to fp16 in registers and used directly as
//                 the B operand: the accumulator layout of S^T lists keys
//                 8*(j/4) + 4*(l/32) + j%4, and the contraction index is
//                 free to permute as long as V^T uses the same order.  V
//                 stays row-major in LDS and each lane gathers its 8 keys of
//                 one d column with two ds_read_b64_tr_b16.
// Data movement: K and V tiles go straight from HBM to LDS with 16-byte
// buffer loads (no register staging), double-buffered, K one tile ahead of
// V (Lever C of the same page).  Both LDS arrays are XOR-swizzled (Lever B):
// K for the 32-row column reads of the A operand, V for the transposed reads.
// Software pipeline inside each wavefront: the MFMAs of S(j+1) are issued in
// the same basic block as the exp/convert/sum work of tile j, so the matrix
// core and the vector ALU run concurrently, then P(j) V(j) follows.
// Causal: key tiles wholly above the diagonal of the workgroup are never
// loaded, wavefronts skip tiles above their own rows, and only tiles that
// cross the diagonal evaluate the mask (Lever A).  Query tiles are issued
// heaviest first so the triangular work packs well onto the CUs.
#pragma once

#include <type_traits>

#include "fa_device.hpp"

namespace fa {

template <int D, int BN, int NW>
struct FwdCfg {
  static constexpr int NWAVES = NW;
  static constexpr int THREADS = 64 * NWAVES;
  static constexpr int BM = 32 * NWAVES;
  static constexpr int KCH = D / 8;    // 16-byte chunks per K / V row
  static constexpr int NKB = BN / 32;  // 32-key blocks per tile
  static constexpr int NDB = D / 32;   // 32-wide d blocks of the output
  static constexpr int KS = D / 16;    // k-steps of S = K Q^T
  static constexpr int TILE_BYTES = BN * D * 2;
  static constexpr int LPW = TILE_BYTES / 1024 / NWAVES;  // 1 KiB LDS loads per wavefront per tile
  static constexpr int V_BASE = 2 * TILE_BYTES;           // LDS: K0 K1 V0 V1
  static constexpr int EPI_BYTES = NWAVES * 32 * D * 2;
  static constexpr int LDS_BYTES = (4 * TILE_BYTES > EPI_BYTES) ? 4 * TILE_BYTES : EPI_BYTES;
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert(TILE_BYTES % (1024 * NWAVES) == 0, "tile must split into 1 KiB loads per wavefront");
  static_assert(LDS_BYTES <= 65536, "static LDS budget");
};


// Workgroups per CU the register budget is sized for.  Two wavefronts per
// SIMD let one wavefront's softmax overlap the other's MFMAs: at D <= 128
// that is one 8-wavefront workgroup (every K/V tile in LDS then serves 256
// query rows) or two 4-wavefront ones (twice the workgroups, for small
// grids).  At D = 256 the 32 x 256 fp32 accumulator of a wavefront needs the
// whole register file: one 4-wavefront workgroup.
template <int D, int NW>
constexpr int fwd_wg_per_cu() { return (D <= 128 && NW == 4) ? 2 : 1; }

// Resident key tiles (fwd_kernel RES > 0): LDS for RES K and RES V tiles,
// or the epilogue's transpose if larger; and the largest RES whose tiles fit
// the 64 KiB of static LDS.
template <int D, int BN, int NW, int RES>
constexpr int fwd_resident_lds() {
  return (2 * RES * BN * D * 2 > NW * 32 * D * 2) ? 2 * RES * BN * D * 2 : NW * 32 * D * 2;
}
template <int D, int BN>
constexpr int fwd_resident_tiles() { return 65536 / (2 * BN * D * 2); }

// Packed variable-length batches ("Adaptive High-Performance Attention
// Kernels in CUDA", Advanced Production Features, 3. Ragged / Variable-Length
// Sequences): tokens of all sequences in one stream [total, H, D], sequence
// b owning tokens cu[b] .. cu[b+1]-1.  Each workgroup reads its sequence's
// bounds from the cumulative-length arrays and exits if its query tile lies
// past the sequence's end.
struct VarlenArgs {
  const int* cu_q;  // [B + 1]
  const int* cu_k;  // [B + 1]
  int H, total_q, total_k, max_q, max_k;
};

// Key-range split of small grids, for grids too small to keep every CU
// busy until the end (the split-KV idea of the decode, "Adaptive
// High-Performance Attention Kernels in CUDA", Split-K / Flash-Decoding,
// applied to the query tiles of a prefill).  Two schemes:
//
// Parts (D <= 128, two 4-wavefront workgroups per CU): query tiles ts ..
// nqt-1 are each processed as ns workgroups over consecutive parts of their
// key range.  Each part writes its normalised fp32 partial O and its
// log-sum-exp to rows of [rows, ns, D] / [rows, ns] (row = (slice, tile - ts,
// row in tile)); fwd_merge_kernel combines them.  Tiles below ts run whole.
// Work items are issued heaviest first: the split parts and the whole tiles
// are two lists of falling weight, merged by weight.
//
// Runs (D = 256, one workgroup per CU, so a workgroup's start-up is never
// hidden behind another's work; "stream-K"): the work of every slice is a
// row of key tiles (its query tiles in split_order, each with the key tiles
// it visits); the rows of all slices are laid end to end and cut into runs,
// one per workgroup: run g starts at key-tile position split_start(g), i.e.
// even runs get total / runs + bias key tiles and odd runs that - bias (the bias
// leaves room for the second segment that an odd run of a causal grid
// usually holds).  A run is a few segments (a query tile over a range of its
// key tiles).  A segment that holds all of its tile's key tiles writes O and
// LSE as usual.  A tile cut between runs writes its normalised fp32 partial O
// and its log2-sum-exp, and fwd_split_merge_kernel combines the parts of
// every cut tile in part order.
struct KeySplit {
  int ts, ns;    // parts: first split query tile, parts per split tile
  int runs;      // runs: number of runs (workgroups doing work)
  int bias;      // runs: 0 <= bias < total / runs
  int units;     // runs: key tiles of one slice
  int total;     // runs: key tiles of all slices
  float* ws_o;   // parts: [BH * (nqt - ts) * BM, ns, D]; runs: [grid, 2, BM, D]
  float* ws_lse; // parts: [BH * (nqt - ts) * BM, ns]; runs: [grid, 2, BM] (log2 units)
};

// Whether the split of the D-wide kernel is by runs (else by parts).
template <int D>
constexpr bool split_by_runs() { return D == 256; }

// First key-tile position of run g of `runs` over `total` key tiles (odd
// runs start `bias` later), and the run that holds position x.  Runs are
// floor(total / runs) or one more key tiles long before the bias, so two
// consecutive runs cover exactly one (heavy, light) pair whenever the pairs
// hold 2 * total / runs key tiles.  The planner takes runs only when
// (runs + 8) * total < 2^32 (g <= runs + 7 for the workgroups of a grid
// rounded up to a multiple of 8), so these products fit 32-bit unsigned
// arithmetic (a 64-bit division costs ~140 instructions on the GPU).
__host__ __device__ inline long long split_start(int g, int runs, int total, int bias) {
  return (long long)((uint32_t)g * (uint32_t)total / (uint32_t)runs) + ((g & 1) ? bias : 0);
}
__host__ __device__ inline int split_run(int x, int runs, int total, int bias) {
  int g = (int)(((uint32_t)(x + 1) * (uint32_t)runs - 1u) / (uint32_t)total);
  if ((g & 1) && split_start(g, runs, total, bias) > x) --g;
  return g;
}

// Workspace slot of run g's segment of a tile that starts at key-tile
// position tile_lin: a tile that began in an earlier run is its run's first
// segment, else its last.
__host__ __device__ inline size_t split_slot(int g, int tile_lin, int runs, int total, int bias) {
  return (size_t)g * 2 + (tile_lin < split_start(g, runs, total, bias) ? 0 : 1);
}

// Key tiles of BN keys that query tile t (BM rows) visits.
__host__ __device__ inline int fwd_tile_units(int t, int BM, int BN, int Sq, int Sk, bool causal) {
  const int all = (Sk + BN - 1) / BN;
  if (!causal) return all;
  const int hi = min(min((t + 1) * BM, Sq), Sk);
  return min(all, (hi + BN - 1) / BN);
}

// Order of the query tiles of a slice in an even split: heaviest, lightest,
// second heaviest, second lightest, ... (tile ranks: rank 0 is the heaviest
// causal tile), so that consecutive pairs carry about the same work and a
// run boundary cuts few tiles.
__host__ __device__ inline int split_order(int i, int nqt) { return (i & 1) ? nqt - 1 - (i >> 1) : (i >> 1); }
__host__ __device__ inline int split_position(int rank, int nqt) {
  return (2 * rank < nqt) ? 2 * rank : 2 * (nqt - 1 - rank) + 1;
}

template <int D, int BN, int NW, bool CAUSAL, bool VARLEN = false, bool KSPLIT = false, int RES = 0>
__global__ void __launch_bounds__(64 * NW, (fwd_wg_per_cu<D, NW>()))
fwd_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
           const _Float16* __restrict__ V, _Float16* __restrict__ O, float* __restrict__ LSE,
           int Sq, int Sk, int BH, int nqt, float c2, VarlenArgs va = {}, KeySplit ksp = {}) {
  using C = FwdCfg<D, BN, NW>;
  // RES > 0: every key tile of the slice (at most RES) is copied to LDS
  // in the prologue and stays, so the loop waits for no copy (short key
  // ranges, where each streamed tile would cost a memory round trip)
  constexpr bool RESIDENT = RES > 0;
  static_assert(!RESIDENT || (!VARLEN && !KSPLIT), "resident tiles: dense, unsplit grids");
  constexpr int LDS_BYTES = RESIDENT ? fwd_resident_lds<D, BN, NW, RES>() : C::LDS_BYTES;
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so per-wave branches stay scalar
  const int r32 = lane & 31;
  const int hh = lane >> 5;

  // Work item: consecutive workgroup ids walk all (batch, head) slices of
  // one query-tile rank before the next rank, so the dispatcher sees the
  // heaviest causal tiles first and, with B*H a multiple of 8, every tile
  // of a slice runs on the same XCD (workgroups are dealt to XCDs round
  // robin by id) and shares its L2.
  // Packed batches: workgroup id = (g * nqt + rank) * 8 + x for the slice
  // bh = 8 g + x, so all query tiles of a slice run back to back on one XCD
  // (ids are dealt to the 8 XCDs round robin) and share its L2 copy of the
  // slice's K / V, whatever the number of slices.
  int rank = VARLEN ? (int)((blockIdx.x >> 3) % (unsigned)nqt) : (int)(blockIdx.x / BH);
  int bh = VARLEN ? (int)((blockIdx.x >> 3) / (unsigned)nqt) * 8 + (int)(blockIdx.x & 7)
                  : (int)(blockIdx.x - rank * BH);
  // Parts: walk the two weight-ordered lists (parts of tiles ts..nqt-1,
  // whole tiles 0..ts-1, each from the top) to this workgroup's item.  Within
  // a tile the items are part-major, slice-minor, so a slice keeps its XCD.
  constexpr bool RUNS = KSPLIT && split_by_runs<D>();
  int part = 0, nparts = 1;
  if constexpr (KSPLIT && !RUNS) {
    int idx = (int)blockIdx.x, th = nqt - 1, tl = ksp.ts - 1;
    for (;;) {
      const int wh = th >= ksp.ts ? (fwd_tile_units(th, C::BM, BN, Sq, Sk, CAUSAL) + ksp.ns - 1) / ksp.ns : -1;
      const int wl = tl >= 0 ? fwd_tile_units(tl, C::BM, BN, Sq, Sk, CAUSAL) : -1;
      if (wh < 0 && wl < 0) return;  // past the last item
      if (wh >= wl) {
        if (idx < ksp.ns * BH) {
          part = idx / BH;
          bh = idx - part * BH;
          nparts = ksp.ns;
          rank = CAUSAL ? nqt - 1 - th : th;
          break;
        }
        idx -= ksp.ns * BH;
        --th;
      } else {
        if (idx < BH) {
          bh = idx;
          rank = CAUSAL ? nqt - 1 - tl : tl;
          break;
        }
        idx -= BH;
        --tl;
      }
    }
  }
  // Runs: workgroup ids are dealt to the 8 XCDs round robin; run = (id % 8) *
  // (grid / 8) + id / 8 gives each XCD a block of consecutive runs, so the
  // runs of a slice share one L2 copy of its K / V (the grid is a multiple of
  // 8; runs past the last exit at once).  Other grids make one pass of the
  // segment loop below.
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
        seg_units = fwd_tile_units(CAUSAL ? nqt - 1 - rank : rank, C::BM, BN, Sq, Sk, CAUSAL);
        if (off < base + seg_units || i == nqt - 1) break;
        base += seg_units;
      }
      seg_kb = off - base;
      seg_ke = min(seg_units, seg_kb + (lin_end - lin));
      tile_lin = lin - seg_kb;
      lin += seg_ke - seg_kb;
    }
    if (VARLEN && bh >= BH) return;  // the grid rounds the slice count up to a multiple of 8
    // Slice of this work item: base pointers, lengths and the row stride (in
    // elements) of q, k, v, o.  Dense [B, H, S, D]: rows D apart.  Packed
    // [total, H, D]: rows H*D apart, lengths from the cumulative arrays
    // (clamped into the tensors and to the maximum lengths the grid covers).
    const _Float16 *qs, *ks_, *vs;
    _Float16* os;
    float* ls;
    int RS;
    if constexpr (VARLEN) {
      const int b = bh / va.H;
      const int h = bh - b * va.H;
      const int sq0 = min(max(va.cu_q[b], 0), va.total_q);
      const int sk0 = min(max(va.cu_k[b], 0), va.total_k);
      Sq = min(min(max(va.cu_q[b + 1] - sq0, 0), va.total_q - sq0), va.max_q);
      Sk = min(min(max(va.cu_k[b + 1] - sk0, 0), va.total_k - sk0), va.max_k);
      nqt = (Sq + C::BM - 1) / C::BM;  // this sequence's tiles (the grid covers the longest)
      if (rank >= nqt) return;  // the sequence has no query tile of this rank
      RS = va.H * D;
      qs = Q + ((size_t)sq0 * va.H + h) * D;
      os = O + ((size_t)sq0 * va.H + h) * D;
      ks_ = K + ((size_t)sk0 * va.H + h) * D;
      vs = V + ((size_t)sk0 * va.H + h) * D;
      ls = LSE + (size_t)h * va.total_q + sq0;
    } else {
      RS = D;
      qs = Q + (size_t)bh * Sq * D;
      os = O + (size_t)bh * Sq * D;
      ks_ = K + (size_t)bh * Sk * D;
      vs = V + (size_t)bh * Sk * D;
      ls = LSE + (size_t)bh * Sq;
    }
    const int qt = CAUSAL ? (nqt - 1 - rank) : rank;
    const int q0 = qt * C::BM;
    const int qw = q0 + 32 * w;  // first query row of this wavefront
    const int qi = qw + r32;     // query row held by this lane

    // Per-slice buffer resources: rows past Sq / Sk read as zero and stores
    // past Sq are dropped (the extent ends with the last row's D elements).
    auto extent = [&](int rows) { return rows > 0 ? (uint32_t)((rows - 1) * RS + D) * 2u : 0u; };
    const auto rq = make_rsrc(qs, extent(Sq));
    const auto ro = make_rsrc(os, extent(Sq));

    // Q fragment: B operand of S^T = K Q^T, 8 consecutive d per lane and step.
    h8 qreg[C::KS];
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) qreg[ks] = as_h8(buf_load16(rq, ((uint32_t)qi * RS + 16 * ks + 8 * hh) * 2u));
    if constexpr (D == 256) {
      // one wavefront per SIMD: Q (64 registers), only ever an MFMA operand,
      // stays in the accumulation registers and the VGPRs hold O, S and P
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) asm volatile("" : "+a"(qreg[ks]));
    }

    const int nkt_all = (Sk + BN - 1) / BN;
    const int nkt = CAUSAL ? min(nkt_all, (min(q0 + C::BM, Sk) + BN - 1) / BN) : nkt_all;
    // key tiles [kb, ke) of this work item (a part or a segment of the range
    // when split)
    int kb = 0, ke = nkt;
    if constexpr (RUNS) {
      kb = seg_kb;
      ke = seg_ke;
    } else if (KSPLIT && nparts > 1) {
      const int c = (nkt + nparts - 1) / nparts;
      kb = min(part * c, nkt);
      ke = min(kb + c, nkt);
    }
    const bool cut = RUNS && (seg_kb > 0 || seg_ke < seg_units);  // a segment of a tile cut between runs
    // last key tile this wavefront needs (below kb: none, e.g. rows past Sq)
    const int jlast = (qw >= Sq) ? -1 : (CAUSAL ? min(ke - 1, (qw + 31) / BN) : ke - 1);

    // Global byte offsets (inside one tile) of the 16-byte chunks this lane
    // moves into LDS: wavefront w fills 1 KiB blocks w*LPW .. w*LPW+LPW-1 of
    // each stage, lane l the 16 bytes at 16*l, and the chunk that belongs
    // there is found through the inverse swizzle.
    uint32_t kgo[C::LPW], vgo[C::LPW];
#pragma unroll
    for (int u = 0; u < C::LPW; ++u) {
      const int p = (w * C::LPW + u) * 1024 + lane * 16;
      int r, c;
      swz_inv<C::KCH>(p >> 8, (p >> 4) & 15, r, c);
      kgo[u] = (uint32_t)(r * RS + c * 8) * 2;
      vswz_inv<C::KCH>(p >> 8, (p >> 4) & 15, r, c);
      vgo[u] = (uint32_t)(r * RS + c * 8) * 2;
    }
    const uint32_t tile_stride = (uint32_t)BN * RS * 2;  // bytes between key tiles
    const u32x4 rkw = rsrc_words(ks_, extent(Sk));
    const u32x4 rvw = rsrc_words(vs, extent(Sk));
    const uint32_t lds0 = lds_addr_of(smem);
  // LDS slot of key tile kt: two-stage rings (K0 K1 V0 V1), or one slot per
  // tile (K0..K(RES-1) V0..V(RES-1)) for resident tiles
  constexpr int V_BASE = RESIDENT ? RES * C::TILE_BYTES : C::V_BASE;
  auto kst = [](int kt) { return RESIDENT ? kt : (kt & 1); };
    auto load_k = [&](int kt, int stage) {
      const uint32_t tb = (uint32_t)kt * tile_stride;
#pragma unroll
      for (int u = 0; u < C::LPW; ++u)
        dma16(rkw, lds0 + stage * C::TILE_BYTES + (w * C::LPW + u) * 1024, tb + kgo[u]);
    };
    auto load_v = [&](int kt, int stage) {
      const uint32_t tb = (uint32_t)kt * tile_stride;
#pragma unroll
      for (int u = 0; u < C::LPW; ++u)
        dma16(rvw, lds0 + V_BASE + stage * C::TILE_BYTES + (w * C::LPW + u) * 1024, tb + vgo[u]);
    };

    // S^T = K Q^T for the tile in K stage `stage`.
    auto qk = [&](int stage, f32x16 (&s)[C::NKB]) {
      const char* Ks = smem + stage * C::TILE_BYTES;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
        for (int j = 0; j < 16; ++j) s[kb][j] = 0.f;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          const h8 a = *reinterpret_cast<const h8*>(Ks + swz<C::KCH>(32 * kb + r32, 2 * ks + hh));
          s[kb] = mfma_32x32x16(a, qreg[ks], s[kb]);
        }
      }
    };

    // Lane constants of the transposed V reads: key offset i/4 inside the
    // 4-key group, 16-byte chunk and 8-byte half of column 16*(g%2) + 4*(i%4).
    const int ti = lane & 15;
    const int tg = (lane >> 4) & 1;
    const int v_key = 4 * hh + (ti >> 2);
    const int v_chunk = 2 * tg + ((ti & 3) >> 1);
    const int v_half = (ti & 1) * 8;

    f32x16 oacc[C::NDB];
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) oacc[db][j] = 0.f;
    // Reference max of s*c (log2 units) of this lane's row: the first tile's
    // row max, or far below any score for a row without a visible key there
    // (a later tile with one then moves it, and a masked score still gives
    // exp2(-inf) = 0); it moves only when the P of a tile could leave fp16's
    // range (see refit).
    float m_run = kMRunInit;
    float l_run = 0.f;  // this lane's share of the row sum
    f32x16 s_cur[C::NKB];

    // Masks S^T of key tile kt: keys past Sk, and keys after the row when
    // causal (only instantiated for tiles that need it).
    auto mask_tile = [&](f32x16 (&s)[C::NKB], int kt) {
      const int kbase = kt * BN;
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = kbase + 32 * kb + 8 * (j >> 2) + 4 * hh + (j & 3);
          if (key >= Sk || (CAUSAL && key > qi)) s[kb][j] = kNegInf;
        }
    };
    // p = 2^(s*c - m_run) rounded to fp16 into the B operand of P V; returns
    // this lane's share of the tile's row sum (of the fp16 P that feeds P V).
    auto softmax_tile = [&](f32x16 (&s)[C::NKB], h8 (&pop)[C::NKB][2]) {
      float t = 0.f;
      const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
      for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
          h2 pr;
          pr[0] = (_Float16)exp2_fast(__builtin_fmaf(s[kb][j], c2, -m_run));
          pr[1] = (_Float16)exp2_fast(__builtin_fmaf(s[kb][j + 1], c2, -m_run));
          t = dot2(pr, ones, t);
          pop[kb][j >> 3][j & 7] = pr[0];
          pop[kb][j >> 3][(j & 7) + 1] = pr[1];
        }
      return t;
    };
    // Every p is at most a lane's share t of the row sum, so t <= kPSumMax
    // keeps P inside fp16's range at full relative precision.  Otherwise
    // (rare: the first tile of a row, or a row max that grew by more than
    // ~2^15 over the reference) the reference moves to the tile's row max
    // (the online-softmax rescale of O and l by 2^(m_old - m_new)) and P is
    // formed again.
    auto refit = [&](f32x16 (&s)[C::NKB], h8 (&pop)[C::NKB][2], float& t) {
      if (__builtin_expect(wave_any(!(t <= kPSumMax)), 0)) {
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int j = 0; j < 16; j += 2) mx = fmaxf(fmaxf(mx, s[kb][j]), s[kb][j + 1]);
        const float m_new = fmaxf(m_run, xhalf_max(mx) * c2);
        const float alpha = exp2_fast(m_run - m_new);  // 0 before the row's first visible key
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
          for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha;
        m_run = m_new;
        t = softmax_tile(s, pop);
      }
    };

    // One pipelined step on tile kt: exp/convert/sum of S(kt) issued together
    // with the MFMAs of S(kt+1) (when NEXT, into s_n), then O += P(kt) V(kt),
    // and the mask of S(kt+1) when the next tile needs one.
    auto step = [&](int kt, f32x16 (&s_c)[C::NKB], f32x16 (&s_n)[C::NKB], auto mask_next, auto next_tag) {
      constexpr bool NEXT = decltype(next_tag)::value;
      h8 pop[C::NKB][2];
      // 8 wavefronts: the next tile's K fragments are all read before the
      // softmax, so its MFMAs wait once instead of once per fragment (held
      // there by a scheduling barrier; left to the compiler, each read sat
      // just ahead of its MFMA; 0.7% on the 4096-token causal prefill, and
      // slower on the 4-wavefront shapes, which keep the plain order)
      constexpr bool EARLY_K = NEXT && NW == 8;
      h8 kfr[C::NKB][C::KS];
      if constexpr (EARLY_K) {
        const char* Ks = smem + kst(kt + 1) * C::TILE_BYTES;
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int ks = 0; ks < C::KS; ++ks)
            kfr[kb][ks] = *reinterpret_cast<const h8*>(Ks + swz<C::KCH>(32 * kb + r32, 2 * ks + hh));
        __builtin_amdgcn_sched_barrier(0);
      }
      float t = softmax_tile(s_c, pop);
      if constexpr (EARLY_K) {
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
          for (int j = 0; j < 16; ++j) s_n[kb][j] = 0.f;
#pragma unroll
          for (int ks = 0; ks < C::KS; ++ks) s_n[kb] = mfma_32x32x16(kfr[kb][ks], qreg[ks], s_n[kb]);
        }
      } else if constexpr (NEXT) {
        qk(kst(kt + 1), s_n);
      }
      refit(s_c, pop, t);
      l_run += t;

      const char* Vs = smem + V_BASE + kst(kt) * C::TILE_BYTES;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
          for (int k2 = 0; k2 < 2; ++k2) {
            const int key = 32 * kb + 16 * k2 + v_key;
            const int chunk = 4 * db + v_chunk;
            const h4v lo = lds_read_tr16(Vs + vswz<C::KCH>(key, chunk) + v_half);
            const h4v hi = lds_read_tr16(Vs + vswz<C::KCH>(key + 8, chunk) + v_half);
            const h8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            oacc[db] = mfma_32x32x16(a, pop[kb][k2], oacc[db]);
          }
      if constexpr (NEXT && decltype(mask_next)::value) mask_tile(s_n, kt + 1);
    };
    auto tile_needs_mask = [&](int kt) { return (kt * BN + BN > Sk) || (CAUSAL && kt * BN + BN - 1 > qw); };

    // Prologue: K(kb), V(kb), K(kb+1) resident, S(kb) computed, masked and maxed.
    if (!KSPLIT || kb < ke) {
      load_k(kb, kst(kb));
      load_v(kb, kst(kb));
    }
    if constexpr (RESIDENT) {
      for (int t = kb + 1; t < ke; ++t) {
        load_k(t, t);
        load_v(t, t);
      }
    } else if (kb + 1 < ke) {
      load_k(kb + 1, kst(kb + 1));
    }
    wait_vmem_all();
    __syncthreads();
    if (jlast >= kb) {
      qk(kst(kb), s_cur);
      if (tile_needs_mask(kb)) mask_tile(s_cur, kb);
      // the reference starts at the first tile's row max (a row without a
      // visible key there keeps kMRunInit), so its P needs no refit
      float mx = kNegInf;
#pragma unroll
      for (int kb2 = 0; kb2 < C::NKB; ++kb2)
#pragma unroll
        for (int j = 0; j < 16; j += 2) mx = fmaxf(fmaxf(mx, s_cur[kb2][j]), s_cur[kb2][j + 1]);
      m_run = fmaxf(xhalf_max(mx) * c2, kMRunInit);
    }
    if constexpr (!RESIDENT) __syncthreads();  // K stage 0 is refilled with K(2) below

    auto begin_tile = [&](int kt) {
      if constexpr (!RESIDENT) {
        if (kt + 2 < ke) load_k(kt + 2, kst(kt + 2));
        if (kt + 1 < ke) load_v(kt + 1, kst(kt + 1));
      }
    };
    auto end_tile = [&]() {
      if constexpr (!RESIDENT) {
        wait_vmem_all();
        __syncthreads();
      }
    };

    // Hot loop, unrolled by two so the current / next S^T register sets swap
    // roles without copies: every step kt < kclean has a next tile that this
    // wavefront needs and that needs no mask.
    const int kmask = min(CAUSAL ? (qw + 1) / BN : nkt_all, (Sk % BN) ? nkt_all - 1 : nkt_all);
    const int kclean = min(kmask - 1, jlast);
    f32x16 s_alt[C::NKB];
    int kt = kb;
    for (; kt + 2 <= kclean; kt += 2) {
      begin_tile(kt);
      step(kt, s_cur, s_alt, std::false_type{}, std::true_type{});
      end_tile();
      begin_tile(kt + 1);
      step(kt + 1, s_alt, s_cur, std::false_type{}, std::true_type{});
      end_tile();
    }
    // The last few tiles (diagonal, ragged tail, past this wavefront's rows):
    // the next tile's scores are always masked here (the mask leaves a tile
    // that needs none unchanged), and the final tile has no next one.
    for (; kt + 1 < ke; ++kt) {
      begin_tile(kt);
      if (kt <= jlast) {
        step(kt, s_cur, s_alt, std::true_type{}, std::true_type{});
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) s_cur[kb] = s_alt[kb];
      }
      end_tile();
    }
    if (kt < ke) {
      begin_tile(kt);
      if (kt <= jlast) step(kt, s_cur, s_alt, std::false_type{}, std::false_type{});
      end_tile();
    }

    // Epilogue: O = acc / l, LSE = (m + log2 l) * ln 2.  The O^T fragment is
    // transposed through LDS so each row leaves as coalesced 16-byte stores.
    const float l_tot = xhalf_sum(l_run);
    // a row with no key at all (an empty key range of a packed sequence):
    // O = 0, LSE = -inf
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    const float lse2 = (l_tot > 0.f) ? m_run + __builtin_log2f(l_tot) : kNegInf;  // log2-sum-exp of the row
    if (KSPLIT && !RUNS && nparts > 1) {
      // one part of a split tile: normalised fp32 partial O and its log-sum-
      // exp, in the merge kernel's [row, part, D] / [row, part] order
      if (qi < Sq) {
        const size_t row = ((size_t)bh * (nqt - ksp.ts) + (qt - ksp.ts)) * C::BM + (qi - q0);
        float* po = ksp.ws_o + (row * nparts + part) * D;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
          for (int jg = 0; jg < 4; ++jg) {
            f32x4 val;
#pragma unroll
            for (int e = 0; e < 4; ++e) val[e] = oacc[db][4 * jg + e] * inv;
            *reinterpret_cast<f32x4*>(po + 32 * db + 8 * jg + 4 * hh) = val;
          }
        if (hh == 0) ksp.ws_lse[row * nparts + part] = lse2 * kLn2;
      }
      return;
    }
    if (cut) {
      // a segment of a tile cut between runs: normalised fp32 partial O and
      // its log2-sum-exp for the merge kernel
      if (qi < Sq) {
        const size_t slot = split_slot(run, tile_lin, ksp.runs, ksp.total, ksp.bias);
        float* po = ksp.ws_o + (slot * C::BM + (qi - q0)) * D;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
          for (int jg = 0; jg < 4; ++jg) {
            f32x4 val;
#pragma unroll
            for (int e = 0; e < 4; ++e) val[e] = oacc[db][4 * jg + e] * inv;
            *reinterpret_cast<f32x4*>(po + 32 * db + 8 * jg + 4 * hh) = val;
          }
        if (hh == 0) ksp.ws_lse[slot * C::BM + (qi - q0)] = lse2;
      }
      continue;  // the last step's barrier already ended every LDS read
    }
    if constexpr (RESIDENT) __syncthreads();  // every wavefront is done reading K / V
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
    if (qw < Sq) {
#pragma unroll
      for (int u = 0; u < (32 * D / 8) / 64; ++u) {
        const int ci = lane + 64 * u;
        const int row = ci / C::KCH, c = ci % C::KCH;
        buf_store16(ro, ((uint32_t)(qw + row) * RS + c * 8) * 2u,
                    *reinterpret_cast<const u32x4*>(Os + swz<C::KCH>(row, c)));
      }
    }
    if (hh == 0 && qi < Sq) ls[qi] = lse2 * kLn2;
    if constexpr (!RUNS) return;
    __syncthreads();  // the next segment refills LDS
  }
}

// Merge of an even split (KeySplit): one workgroup per 4 * 1024 / D rows of
// a query tile; tiles that no run boundary cuts exit at once.  For each row of a
// cut tile, over its parts p (the runs g0 .. g1 that hold its key tiles, in
// that order): lse2 = M + log2 sum_p 2^(lse2_p - M), O = sum_p 2^(lse2_p -
// lse2) O_p, the log-sum-exp combination of "Adaptive High-Performance
// Attention Kernels in CUDA", Split-K / Flash-Decoding, phase two.  D/4
// threads per row, 4 consecutive d each (16-byte loads); the loads of all
// of a thread's rows and of up to NPARTS parts (an instantiation per bound,
// so short lists keep few registers) are issued before any is used.
template <int D, int BM, int NPARTS>
struct SplitMergeCfg {
  static constexpr int THREADS = 256;
  static constexpr int TPR = D / 4;               // threads per row
  static constexpr int RPP = THREADS / TPR;       // rows per pass
  static constexpr int PASSES = 4;                // rows per thread
  static constexpr int ROWS = RPP * PASSES;       // rows per workgroup
  static constexpr int BLOCKS = BM / ROWS;        // workgroups per query tile
  static constexpr int NP = NPARTS;               // parts loaded together (at least the most parts of any tile)
  static_assert(THREADS % TPR == 0 && ROWS % RPP == 0 && BM % ROWS == 0, "merge geometry");
};

template <int D, int BM, int BN, bool CAUSAL, int NPARTS>
__global__ void __launch_bounds__(256)
fwd_split_merge_kernel(KeySplit ksp, _Float16* __restrict__ O, float* __restrict__ LSE, int Sq, int Sk, int nqt) {
  using M = SplitMergeCfg<D, BM, NPARTS>;
  const int tile = (int)blockIdx.x / M::BLOCKS;
  const int rb = ((int)blockIdx.x - tile * M::BLOCKS) * M::ROWS;  // first row of this workgroup
  const int bh = tile / nqt;
  const int rank = tile - bh * nqt;
  const int qt = CAUSAL ? nqt - 1 - rank : rank;
  const int u = fwd_tile_units(qt, BM, BN, Sq, Sk, CAUSAL);
  // key tiles of the slice's tiles ahead of this one in the run order, one
  // tile per lane and summed across the wavefront
  const int pos = split_position(rank, nqt);
  const int lane = (int)threadIdx.x & 63;
  int before = 0;
  for (int i0 = 0; i0 < pos; i0 += 64) {
    int ui = 0;
    if (i0 + lane < pos) {
      const int r = split_order(i0 + lane, nqt);
      ui = fwd_tile_units(CAUSAL ? nqt - 1 - r : r, BM, BN, Sq, Sk, CAUSAL);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ui += __shfl_xor(ui, off);
    before += ui;
  }
  const int tile_lin = bh * ksp.units + before;
  const int g0 = split_run(tile_lin, ksp.runs, ksp.total, ksp.bias);
  const int g1 = split_run(tile_lin + u - 1, ksp.runs, ksp.total, ksp.bias);
  if (g0 == g1) return;  // written whole by its run
  const int d0 = 4 * ((int)threadIdx.x % M::TPR);
  const int r0 = rb + (int)threadIdx.x / M::TPR;
  const int np = g1 - g0 + 1;
  // one output row: O and LSE from the weights' denominator and numerator
  auto store = [&](int rrow, float mx, float den, const f32x4& num) {
    const int q = qt * BM + rrow;
    if (q >= Sq) return;
    // no key in any part (rows of an empty key range): O = 0, LSE = -inf
    const float inv = (den > 0.f) ? 1.f / den : 0.f;
    h4 res;
#pragma unroll
    for (int e = 0; e < 4; ++e) res[e] = (_Float16)(num[e] * inv);
    const size_t out = (size_t)bh * Sq + q;
    *reinterpret_cast<h4*>(O + out * D + d0) = res;
    if (d0 == 0) LSE[out] = (den > 0.f) ? (mx + __builtin_log2f(den)) * kLn2 : kNegInf;
  };
  if (np <= M::NP) {
    size_t slot[M::NP];
    float lp[M::PASSES][M::NP];
    f32x4 xp[M::PASSES][M::NP];
#pragma unroll
    for (int i = 0; i < M::NP; ++i) slot[i] = split_slot(min(g0 + i, g1), tile_lin, ksp.runs, ksp.total, ksp.bias);
#pragma unroll
    for (int k = 0; k < M::PASSES; ++k)
#pragma unroll
      for (int i = 0; i < M::NP; ++i)
        if (i < np) {
          const size_t row = slot[i] * BM + r0 + k * M::RPP;
          lp[k][i] = ksp.ws_lse[row];
          xp[k][i] = *reinterpret_cast<const f32x4*>(ksp.ws_o + row * D + d0);
        }
#pragma unroll
    for (int k = 0; k < M::PASSES; ++k) {
      float mx = kNegInf;
#pragma unroll
      for (int i = 0; i < M::NP; ++i)
        if (i < np) mx = fmaxf(mx, lp[k][i]);
      float den = 0.f;
      f32x4 num = {0.f, 0.f, 0.f, 0.f};
      if (mx != kNegInf) {
#pragma unroll
        for (int i = 0; i < M::NP; ++i)
          if (i < np) {
            const float wgt = exp2_fast(lp[k][i] - mx);
            den += wgt;
#pragma unroll
            for (int e = 0; e < 4; ++e) num[e] += wgt * xp[k][i][e];
          }
      }
      store(r0 + k * M::RPP, mx, den, num);
    }
    return;
  }
  // A tile cut into more than NP parts (not planned, kept for any KeySplit):
  // the same arithmetic, one part at a time.
  for (int k = 0; k < M::PASSES; ++k) {
    const int rrow = r0 + k * M::RPP;
    float mx = kNegInf;
    for (int p = g0; p <= g1; ++p) mx = fmaxf(mx, ksp.ws_lse[split_slot(p, tile_lin, ksp.runs, ksp.total, ksp.bias) * BM + rrow]);
    float den = 0.f;
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    if (mx != kNegInf) {
      for (int p = g0; p <= g1; ++p) {
        const size_t row = split_slot(p, tile_lin, ksp.runs, ksp.total, ksp.bias) * BM + rrow;
        const float wgt = exp2_fast(ksp.ws_lse[row] - mx);
        const f32x4 x = *reinterpret_cast<const f32x4*>(ksp.ws_o + row * D + d0);
        den += wgt;
#pragma unroll
        for (int e = 0; e < 4; ++e) num[e] += wgt * x[e];
      }
    }
    store(rrow, mx, den, num);
  }
}

// Merge of the key parts of a split forward (the parts of the D <= 128
// key split and of the Split-D forward): for each query row, lse = ln sum_p
// e^(lse_p) and O = sum_p e^(lse_p - lse) O_p, the log-sum-exp combination
// of partial softmax results ("Adaptive High-Performance Attention Kernels
// in CUDA", Split-K / Flash-Decoding, phase two).  D/4 threads per row, 4
// consecutive d each (16-byte loads), 256 / (D/4) rows per workgroup; all
// loads of a thread's parts (up to NP, an instantiation per bound) are
// issued before any is used, so a row waits for one memory round trip.
// Row = (slice, tile - ts, row in tile), written to O[slice, (ts + tile) *
// BM + row] and LSE at the same position.
template <int D, int NP>
struct MergeCfg {
  static constexpr int TPR = D / 4;         // threads per row
  static constexpr int ROWS = 256 / TPR;    // rows per workgroup
  static_assert(D % 4 == 0 && TPR <= 256 && 256 % TPR == 0 && NP >= 1 && NP <= 16, "merge geometry");
};

template <int D, int NP>
__global__ void __launch_bounds__(256)
fwd_merge_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_lse, _Float16* __restrict__ O,
                 float* __restrict__ LSE, int Sq, int BM, int ts, int nsplit, int ns, int rows) {
  using M = MergeCfg<D, NP>;
  const int row = (int)blockIdx.x * M::ROWS + (int)threadIdx.x / M::TPR;
  const int d0 = 4 * ((int)threadIdx.x % M::TPR);
  if (row >= rows) return;
  const int r = row % BM;
  const int tl = (row / BM) % nsplit;
  const int bh = row / (BM * nsplit);
  const int q = (ts + tl) * BM + r;
  if (q >= Sq) return;
  const size_t out = (size_t)bh * Sq + q;
  float lp[NP];
  f32x4 xp[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    lp[j] = kNegInf;
    xp[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (j < ns) {
      lp[j] = ws_lse[(size_t)row * ns + j];
      xp[j] = *reinterpret_cast<const f32x4*>(ws_o + ((size_t)row * ns + j) * D + d0);
    }
  }
  float mx = kNegInf;
#pragma unroll
  for (int j = 0; j < NP; ++j)
    if (j < ns) mx = fmaxf(mx, lp[j]);
  h4 res;
  if (mx == kNegInf) {  // no key in any part: O = 0, LSE = -inf
    res = h4{0, 0, 0, 0};
  } else {
    float den = 0.f;
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      if (j < ns) {
        const float wgt = exp2_fast((lp[j] - mx) * kLog2e);
        den += wgt;
#pragma unroll
        for (int e = 0; e < 4; ++e) num[e] += wgt * xp[j][e];
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) res[e] = (_Float16)(num[e] / den);
    mx += __builtin_logf(den);
  }
  *reinterpret_cast<h4*>(O + out * D + d0) = res;
  if (d0 == 0) LSE[out] = mx;
}

}  // namespace fa
