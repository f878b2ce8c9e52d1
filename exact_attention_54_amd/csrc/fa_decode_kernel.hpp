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
// contiguous bytes (4 key rows at D = 128).  Every lane keeps an independent
// online softmax over the keys of its slot; the NWAVES x SLOTS slot states of
// a workgroup are merged through LDS at the end into one normalised partial
// output O_s and lse_s -- the same split-and-merge one level down.
//
// Phase two (decode_merge_kernel): per slice, lse = ln sum_s exp(lse_s) and
// O = sum_s exp(lse_s - lse) O_s, rounded to fp16.
//
// With a single partition per slice the workgroup has 1024 threads (16
// wavefronts, as many as four 256-thread partitions) and its in-LDS merge
// writes the final fp16 O and LSE: no workspace and no second kernel.
#pragma once

#include <type_traits>

#include "fa_device.hpp"

namespace fa {

template <int D, int T = 256>
struct DecCfg {
  static constexpr int THREADS = T;
  static constexpr int NWAVES = THREADS / 64;
  static constexpr int LPK = (D / 8 < 16) ? D / 8 : 16;  // lanes per key row
  static constexpr int CPL = (D / 8) / LPK;              // 16-byte chunks per lane
  static constexpr int SLOTS = 64 / LPK;                 // key rows per wavefront load
  static constexpr int U = 4;                            // loads in flight per lane and tensor
  static constexpr int KEYS_PER_WAVE_ITER = SLOTS * U;
  static constexpr int KEYS_PER_WG_ITER = NWAVES * KEYS_PER_WAVE_ITER;
  static constexpr int NSTATE = NWAVES * SLOTS;          // independent softmax states per workgroup
};

// Where the K and V rows of a group of keys live.  decode_accumulate walks
// groups of KEYS_PER_WAVE_ITER consecutive keys (one per wavefront and
// step, starting at a wave-uniform key `base`); a loader fills kr / vr with
// the 16-byte chunks of this lane's keys base + u * SLOTS + slot whose
// present[u] is set, clears present[u] for keys it finds absent, and leaves
// zeros elsewhere.  start(base) is called once with the wavefront's first
// base, before the first group.

// Contiguous rows: key j of the slice is row j of k / v.
template <int D, int T>
struct ContigRows {
  using C = DecCfg<D, T>;
  const _Float16* __restrict__ k;
  const _Float16* __restrict__ v;
  int slot, dl;
  __device__ __forceinline__ void start(int) {}
  __device__ __forceinline__ void operator()(int base, bool (&present)[C::U], u32x4 (&kr)[C::U][C::CPL],
                                             u32x4 (&vr)[C::U][C::CPL]) const {
#pragma unroll
    for (int u = 0; u < C::U; ++u)
#pragma unroll
      for (int c = 0; c < C::CPL; ++c) {
        u32x4 tk = {0u, 0u, 0u, 0u}, tv = {0u, 0u, 0u, 0u};
        if (present[u]) {
          // read once: non-temporal loads keep the stream from evicting
          // useful cache lines (measured ~13% more HBM bandwidth)
          const size_t off = (size_t)(base + u * C::SLOTS + slot) * D + (dl + c * C::LPK) * 8;
          tk = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k + off));
          tv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v + off));
        }
        kr[u][c] = tk;
        vr[u][c] = tv;
      }
  }
};

// Paged rows, one page per lane's key: the general case (pages shorter
// than a group).  tbl holds the physical pages of logical blocks blk0 ...;
// an entry outside [0, num_blocks) marks its keys absent.
template <int D, int T>
struct PagedLaneRows {
  using C = DecCfg<D, T>;
  const _Float16* __restrict__ k;
  const _Float16* __restrict__ v;
  const int* tbl;
  int blk0, end, num_blocks, H, h, lbs, slot, dl;  // end: unused (the paged forms share one initializer)
  __device__ __forceinline__ void start(int) {}
  __device__ __forceinline__ void operator()(int base, bool (&present)[C::U], u32x4 (&kr)[C::U][C::CPL],
                                             u32x4 (&vr)[C::U][C::CPL]) const {
    const int bmask = (1 << lbs) - 1;
#pragma unroll
    for (int u = 0; u < C::U; ++u) {
      const int key = base + u * C::SLOTS + slot;
      int64_t row = -1;
      if (present[u]) {
        const int pb = tbl[(key >> lbs) - blk0];
        if ((unsigned)pb < (unsigned)num_blocks) row = (((int64_t)pb * H + h) << lbs) + (key & bmask);
      }
      present[u] = row >= 0;
#pragma unroll
      for (int c = 0; c < C::CPL; ++c) {
        u32x4 tk = {0u, 0u, 0u, 0u}, tv = {0u, 0u, 0u, 0u};
        if (present[u]) {
          const size_t off = (size_t)row * D + (dl + c * C::LPK) * 8;
          tk = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k + off));
          tv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v + off));
        }
        kr[u][c] = tk;
        vr[u][c] = tv;
      }
    }
  }
};

// Paged rows when a page holds at least one whole group (block size >=
// KEYS_PER_WAVE_ITER, groups aligned to their size): the group's page is
// one table entry, looked up once per wavefront, and its address is
// wave-uniform, so the lane addresses are 32-bit offsets from it (fewer
// registers than a 64-bit row per key: the kernel keeps the contiguous
// kernel's occupancy).  The entry of the wavefront's next group is read
// from LDS one step ahead, so that read does not delay the group's loads.
template <int D, int T>
struct PagedGroupRows {
  using C = DecCfg<D, T>;
  const _Float16* __restrict__ k;
  const _Float16* __restrict__ v;
  const int* tbl;
  int blk0, end, num_blocks, H, h, lbs, slot, dl;
  int next = -1;  // table entry of the group at the next call's base (lane copy)

  __device__ __forceinline__ int entry(int base) const {
    return base < end ? tbl[(base >> lbs) - blk0] : -1;
  }
  __device__ __forceinline__ void start(int base) { next = entry(base); }
  __device__ __forceinline__ void operator()(int base, bool (&present)[C::U], u32x4 (&kr)[C::U][C::CPL],
                                             u32x4 (&vr)[C::U][C::CPL]) {
    const int pb = __builtin_amdgcn_readfirstlane(next);
    next = entry(base + C::KEYS_PER_WG_ITER);
    const bool ok = (unsigned)pb < (unsigned)num_blocks;
    const size_t page = ((((size_t)pb * H + h) << lbs) + (base & ((1 << lbs) - 1))) * D;
    const _Float16* kq = k + (ok ? page : 0);
    const _Float16* vq = v + (ok ? page : 0);
#pragma unroll
    for (int u = 0; u < C::U; ++u) {
      present[u] = present[u] && ok;
#pragma unroll
      for (int c = 0; c < C::CPL; ++c) {
        u32x4 tk = {0u, 0u, 0u, 0u}, tv = {0u, 0u, 0u, 0u};
        if (present[u]) {
          const int off = (u * C::SLOTS + slot) * D + (dl + c * C::LPK) * 8;
          tk = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kq + off));
          tv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vq + off));
        }
        kr[u][c] = tk;
        vr[u][c] = tv;
      }
    }
  }
};

// Online softmax of one lane slot over the keys [kb, ke).  The wavefront
// visits groups of KEYS_PER_WAVE_ITER keys starting at a0 + w * that size
// (a0 <= kb, aligned by the caller), stepping by the workgroup's stride;
// lane slot takes keys base + u * SLOTS + slot, and keys outside [kb, ke)
// or absent in the loader's view score -inf.  Contiguous and paged rows
// walk the keys in the same order, so their results agree bit for bit.
template <int D, int T, class Load>
__device__ __forceinline__ void decode_accumulate(const h8 (&qh)[DecCfg<D>::CPL], int a0, int kb, int ke,
                                                  Load& load, int w, int slot, float c2, float& m_run,
                                                  float& l_run, float (&acc)[DecCfg<D>::CPL][8]) {
  using C = DecCfg<D, T>;
  load.start(a0 + w * C::KEYS_PER_WAVE_ITER);
  for (int base = a0 + w * C::KEYS_PER_WAVE_ITER; base < ke; base += C::KEYS_PER_WG_ITER) {
    u32x4 kr[C::U][C::CPL], vr[C::U][C::CPL];
    bool present[C::U];
#pragma unroll
    for (int u = 0; u < C::U; ++u) {
      const int key = base + u * C::SLOTS + slot;
      present[u] = key >= kb && key < ke;
    }
    load(base, present, kr, vr);
    float sc[C::U];
#pragma unroll
    for (int u = 0; u < C::U; ++u) {
      float part = 0.f;
#pragma unroll
      for (int c = 0; c < C::CPL; ++c) {
        const h8 kh = as_h8(kr[u][c]);
#pragma unroll
        for (int e = 0; e < 8; e += 2) part = dot2(h2{kh[e], kh[e + 1]}, h2{qh[c][e], qh[c][e + 1]}, part);
      }
#pragma unroll
      for (int off = 1; off < C::LPK; off <<= 1) part += __shfl_xor(part, off);
      sc[u] = present[u] ? part : kNegInf;
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
}

// Merges the NSTATE slot states of a workgroup through LDS.  Partial
// (FINAL false): the normalised partial output out_o[0..D) (fp32) and its
// natural-log lse; a partition whose slots saw no present key gets O_s = 0,
// lse_s = -inf.  FINAL: the slice's fp16 output out_h[0..D) and its LSE
// (O = 0, LSE = -inf when no key is present).
template <int D, int T, bool FINAL>
__device__ __forceinline__ void decode_merge_slots(float m_run, float l_run, const float (&acc)[DecCfg<D>::CPL][8],
                                                   int tid, int w, int slot, int dl, float* __restrict__ out_o,
                                                   _Float16* __restrict__ out_h, float* __restrict__ out_lse) {
  using C = DecCfg<D, T>;
  __shared__ float s_m[C::NSTATE];
  __shared__ float s_l[C::NSTATE];
  __shared__ __attribute__((aligned(16))) float s_acc[C::NSTATE][D];
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
#pragma unroll 8
  for (int i = 0; i < C::NSTATE; ++i) M = fmaxf(M, s_m[i]);
  for (int d = tid; d < D; d += C::THREADS) {
    if (M == kNegInf) {  // no present key
      if constexpr (FINAL)
        out_h[d] = (_Float16)0.f;
      else
        out_o[d] = 0.f;
      if (d == 0) *out_lse = kNegInf;
      continue;
    }
    float den = 0.f, num = 0.f;
#pragma unroll 8
    for (int i = 0; i < C::NSTATE; ++i) {
      const float wgt = exp2_fast(s_m[i] - M);  // 0 for a slot that saw no key
      den += wgt * s_l[i];
      num += wgt * s_acc[i][d];
    }
    if constexpr (FINAL)
      out_h[d] = (_Float16)(num / den);
    else
      out_o[d] = num / den;
    if (d == 0) *out_lse = (M + __builtin_log2f(den)) * kLn2;
  }
}

// Partial (FINAL false): ws_o [BH, ns, D] fp32, ws_lse [BH, ns] fp32
// (natural log).  FINAL (ns = 1): O [BH, D] fp16 and LSE [BH] directly.
// Occupancy target of the contiguous kernel: 8 wavefronts per SIMD (two
// 1024-thread or eight 256-thread workgroups per CU) at D <= 128, 4 at
// D = 256.
template <int D>
constexpr int dec_waves_per_eu() { return D <= 128 ? 8 : 4; }

template <int D, int T, bool FINAL>
__global__ void __launch_bounds__(T, dec_waves_per_eu<D>())
decode_partial_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
                      const _Float16* __restrict__ V, float* __restrict__ ws_o,
                      float* __restrict__ ws_lse, _Float16* __restrict__ O, float* __restrict__ LSE, int Sk,
                      int ns, int chunk, float c2) {
  using C = DecCfg<D, T>;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int slot = lane / C::LPK;
  const int dl = lane % C::LPK;
  const int bh = blockIdx.x / ns;
  const int s = blockIdx.x - bh * ns;
  const int k0 = s * chunk;
  const int k1 = min(Sk, k0 + chunk);
  float* out_o = FINAL ? nullptr : ws_o + ((size_t)bh * ns + s) * D;
  _Float16* out_h = FINAL ? O + (size_t)bh * D : nullptr;
  float* out_lse = FINAL ? LSE + bh : ws_lse + (size_t)bh * ns + s;

  if (k0 >= k1) {  // empty partition: weight zero in the merge
    for (int d = tid; d < D; d += C::THREADS) {
      if constexpr (FINAL)
        out_h[d] = (_Float16)0.f;
      else
        out_o[d] = 0.f;
    }
    if (tid == 0) *out_lse = kNegInf;
    return;
  }

  const _Float16* qp = Q + (size_t)bh * D;
  // q stays fp16: the scores are fp32 sums of fp16 products (v_dot2), so no
  // conversion waits for q before the first K / V loads are issued
  h8 qh[C::CPL];
#pragma unroll
  for (int c = 0; c < C::CPL; ++c) qh[c] = as_h8(*reinterpret_cast<const u32x4*>(qp + (dl + c * C::LPK) * 8));

  float m_run = kNegInf, l_run = 0.f;
  float acc[C::CPL][8];
#pragma unroll
  for (int c = 0; c < C::CPL; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[c][e] = 0.f;

  ContigRows<D, T> rows{K + (size_t)bh * Sk * D, V + (size_t)bh * Sk * D, slot, dl};
  decode_accumulate<D, T>(qh, k0 & ~(C::KEYS_PER_WAVE_ITER - 1), k0, k1, rows, w, slot, c2, m_run, l_run, acc);
  decode_merge_slots<D, T, FINAL>(m_run, l_run, acc, tid, w, slot, dl, out_o, out_h, out_lse);
}

// Paged KV cache ("Adaptive High-Performance Attention Kernels in CUDA",
// Advanced Production Features, 4. PagedAttention): K and V live in
// fixed-size physical blocks [num_blocks, H, block_size, D], and row b of
// the block table [B, max_blocks] names the physical block that holds
// logical block j (keys j*block_size .. +block_size-1) of sequence b.  The
// workgroup of (b, h, partition) copies the table entries of its key range
// to LDS (in segments of at most kPagedTbl blocks), then streams keys as the
// contiguous kernel does, translating keys to physical rows.  Table entries
// outside [0, num_blocks) mark absent keys: they are never read.
//
// GROUP (block_size >= KEYS_PER_WAVE_ITER): a wavefront's group of keys
// lies in one page, translated once per group into a wave-uniform address
// (PagedGroupRows); this form needs the registers of the contiguous kernel
// and keeps its occupancy.  Otherwise every lane translates its own keys
// (PagedLaneRows; held to the contiguous kernel's 64 registers, that
// translation spills).
constexpr int kPagedTbl = 2048;

template <int D, bool GROUP>
constexpr int paged_waves_per_eu() { return GROUP ? dec_waves_per_eu<D>() : 1; }

template <int D, int T, bool FINAL, bool GROUP>
__global__ void __launch_bounds__(T, (paged_waves_per_eu<D, GROUP>()))
decode_paged_partial_kernel(const _Float16* __restrict__ Q, const _Float16* __restrict__ Kc,
                            const _Float16* __restrict__ Vc, const int* __restrict__ tables,
                            const int* __restrict__ seq_lens, float* __restrict__ ws_o,
                            float* __restrict__ ws_lse, _Float16* __restrict__ O, float* __restrict__ LSE, int H,
                            int ns, int num_blocks, int lbs, int max_blocks, float c2) {
  using C = DecCfg<D, T>;
  __shared__ int s_tbl[kPagedTbl];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int slot = lane / C::LPK;
  const int dl = lane % C::LPK;
  const int bh = blockIdx.x / ns;
  const int s = blockIdx.x - bh * ns;
  const int b = bh / H;
  const int h = bh - b * H;
  // context length, clamped to what the table row can address
  const int L = min(max(seq_lens[b], 0), max_blocks << lbs);
  const int chunk = (L + ns - 1) / ns;
  const int k0 = s * chunk;
  const int k1 = min(L, k0 + chunk);
  float* out_o = FINAL ? nullptr : ws_o + ((size_t)bh * ns + s) * D;
  _Float16* out_h = FINAL ? O + (size_t)bh * D : nullptr;
  float* out_lse = FINAL ? LSE + bh : ws_lse + (size_t)bh * ns + s;

  if (k0 >= k1) {  // empty partition (or empty context): weight zero in the merge
    for (int d = tid; d < D; d += C::THREADS) {
      if constexpr (FINAL)
        out_h[d] = (_Float16)0.f;
      else
        out_o[d] = 0.f;
    }
    if (tid == 0) *out_lse = kNegInf;
    return;
  }

  const _Float16* qp = Q + (size_t)bh * D;
  // q stays fp16: the scores are fp32 sums of fp16 products (v_dot2), so no
  // conversion waits for q before the first K / V loads are issued
  h8 qh[C::CPL];
#pragma unroll
  for (int c = 0; c < C::CPL; ++c) qh[c] = as_h8(*reinterpret_cast<const u32x4*>(qp + (dl + c * C::LPK) * 8));

  float m_run = kNegInf, l_run = 0.f;
  float acc[C::CPL][8];
#pragma unroll
  for (int c = 0; c < C::CPL; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[c][e] = 0.f;

  const int* trow = tables + (size_t)b * max_blocks;
  // Segments are whole workgroup steps from the group-aligned start, so the
  // keys meet the lanes in the contiguous kernel's order; a segment spans at
  // most seg_keys / block_size + 1 <= kPagedTbl blocks.
  static_assert(kPagedTbl - 1 >= C::KEYS_PER_WG_ITER, "a segment holds at least one workgroup step");
  const int a0 = k0 & ~(C::KEYS_PER_WAVE_ITER - 1);
  const int seg_keys = ((kPagedTbl - 1) << lbs) / C::KEYS_PER_WG_ITER * C::KEYS_PER_WG_ITER;
  for (int seg = a0; seg < k1; seg += seg_keys) {
    const int seg_end = min(k1, seg + seg_keys);
    const int blk0 = seg >> lbs;
    const int nblk = ((seg_end - 1) >> lbs) - blk0 + 1;
    __syncthreads();  // the previous segment's table reads are done
    for (int i = tid; i < nblk; i += C::THREADS) s_tbl[i] = trow[blk0 + i];
    __syncthreads();
    using Rows = std::conditional_t<GROUP, PagedGroupRows<D, T>, PagedLaneRows<D, T>>;
    Rows rows{Kc, Vc, s_tbl, blk0, seg_end, num_blocks, H, h, lbs, slot, dl};
    decode_accumulate<D, T>(qh, seg, max(seg, k0), seg_end, rows, w, slot, c2, m_run, l_run, acc);
  }
  decode_merge_slots<D, T, FINAL>(m_run, l_run, acc, tid, w, slot, dl, out_o, out_h, out_lse);
}

// Phase two: one workgroup of T threads per slice.  D/4 threads cover a row
// (4 consecutive d each, 16-byte loads), so the workgroup holds G = 4T/D
// such groups; group g takes partitions g, g + G, g + 2G, ..., and the G
// group sums are added through LDS in group order (deterministic for a
// given ns and T).  Spreading the partitions over the workgroup keeps a
// slice's merge short when a small batch is split into many partitions:
// 256 threads, or 1024 when that leaves a group more than 4 partitions.
template <int D, int T = 256>
struct DecMergeCfg {
  static constexpr int TPR = D / 4;     // threads per row
  static constexpr int G = T / TPR;     // partition groups
  static_assert(D % 4 == 0 && T % TPR == 0 && G >= 1, "merge geometry");
};

template <int D, int T>
__global__ void __launch_bounds__(T)
decode_merge_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_lse,
                    _Float16* __restrict__ O, float* __restrict__ LSE, int ns) {
  using M = DecMergeCfg<D, T>;
  __shared__ __attribute__((aligned(16))) float s_num[M::G][D];
  __shared__ float s_den[M::G];
  __shared__ float s_max[M::G];
  const int bh = blockIdx.x;
  const int g = (int)threadIdx.x / M::TPR;
  const int d0 = 4 * ((int)threadIdx.x % M::TPR);
  const float* lp = ws_lse + (size_t)bh * ns;
  const float* op = ws_o + (size_t)bh * ns * D + d0;
  // the lse and partial O of the group's first NPG partitions are loaded
  // together, before the maximum is known (one memory round trip); any
  // further partitions are read in a loop below
  constexpr int NPG = 4;
  float lv[NPG];
  f32x4 xv[NPG];
#pragma unroll
  for (int i = 0; i < NPG; ++i) {
    const int s = g + i * M::G;
    lv[i] = kNegInf;
    xv[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (s < ns) {
      lv[i] = lp[s];
      xv[i] = *reinterpret_cast<const f32x4*>(op + (size_t)s * D);
    }
  }
  // lse max over the partitions: per group, then across the groups
  float mx = kNegInf;
#pragma unroll
  for (int i = 0; i < NPG; ++i)
    if (g + i * M::G < ns) mx = fmaxf(mx, lv[i]);
  for (int s = g + NPG * M::G; s < ns; s += M::G) mx = fmaxf(mx, lp[s]);
  if (d0 == 0) s_max[g] = mx;
  __syncthreads();
  mx = s_max[0];
#pragma unroll
  for (int j = 1; j < M::G; ++j) mx = fmaxf(mx, s_max[j]);
  if (mx == kNegInf) {  // no key at all (empty paged context): O = 0, LSE = -inf
    if (g == 0) {
      *reinterpret_cast<h4*>(O + (size_t)bh * D + d0) = h4{0, 0, 0, 0};
      if (d0 == 0) LSE[bh] = kNegInf;
    }
    return;
  }
  float den = 0.f;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NPG; ++i) {
    if (g + i * M::G < ns) {
      const float wgt = exp2_fast((lv[i] - mx) * kLog2e);
      den += wgt;
#pragma unroll
      for (int e = 0; e < 4; ++e) num[e] += wgt * xv[i][e];
    }
  }
  for (int s = g + NPG * M::G; s < ns; s += M::G) {
    const float wgt = exp2_fast((lp[s] - mx) * kLog2e);
    const f32x4 x = *reinterpret_cast<const f32x4*>(op + (size_t)s * D);
    den += wgt;
#pragma unroll
    for (int e = 0; e < 4; ++e) num[e] += wgt * x[e];
  }
  *reinterpret_cast<f32x4*>(&s_num[g][d0]) = num;
  if (d0 == 0) s_den[g] = den;
  __syncthreads();
  if (g == 0) {
#pragma unroll
    for (int j = 1; j < M::G; ++j) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(&s_num[j][d0]);
      den += s_den[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) num[e] += x[e];
    }
    h4 res;
#pragma unroll
    for (int e = 0; e < 4; ++e) res[e] = (_Float16)(num[e] / den);
    *reinterpret_cast<h4*>(O + (size_t)bh * D + d0) = res;
    if (d0 == 0) LSE[bh] = mx + __builtin_logf(den);
  }
}

}  // namespace fa
