// Host side of the C ABI declared in include/fa.h: argument validation,
// kernel selection, launch geometry and error reporting.  Every entry point
// validates all arguments before its first HIP call.
#include "fa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <functional>
#include <mutex>
#include <type_traits>
#include <vector>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "fa_bwd_kernel.hpp"
#include "fa_decode_kernel.hpp"
#include "fa_fwd_kernel.hpp"
#include "fa_splitd_kernel.hpp"

namespace fa {
// The D = 256 prefill kernels are compiled in fa_fwd256.hip (with MFMA
// results in VGPRs); here they are only launched.
#define FA_FWD256_EXTERN(CAUSAL, VARLEN, KSPLIT)                                                                 \
  extern template __global__ void fwd_kernel<256, 32, 4, CAUSAL, VARLEN, KSPLIT>(                                \
      const _Float16* __restrict__, const _Float16* __restrict__, const _Float16* __restrict__,                  \
      _Float16* __restrict__, float* __restrict__, int, int, int, int, float, VarlenArgs, KeySplit);
FA_FWD256_EXTERN(false, false, false)
FA_FWD256_EXTERN(true, false, false)
FA_FWD256_EXTERN(false, false, true)
FA_FWD256_EXTERN(true, false, true)
FA_FWD256_EXTERN(false, true, false)
FA_FWD256_EXTERN(true, true, false)
#undef FA_FWD256_EXTERN
}  // namespace fa

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// a*b*c*d <= limit without overflow (all >= 1).
bool product_le(int64_t a, int64_t b, int64_t c, int64_t d, int64_t limit) {
  if (a > limit) return false;
  int64_t p = a;
  for (int64_t x : {b, c, d}) {
    if (p > limit / x) return false;
    p *= x;
  }
  return p <= limit;
}

constexpr int64_t kMaxElems = int64_t(1) << 40;  // per tensor, far above any HBM size
constexpr int64_t kMaxGrid = 0x7fffffff;
constexpr int64_t kMaxSliceBytes = int64_t(1) << 31;

int validate(const void* q, const void* k, const void* v, const void* o, const void* lse, int B, int H,
             int Sq, int Sk, int D, int causal, float scale) {
  if (!q || !k || !v || !o || !lse) return fail(FA_ERR_INVALID_ARG, "null tensor pointer");
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1 || D < 1)
    return fail(FA_ERR_INVALID_ARG, "sizes must be >= 1 (B=%d H=%d Sq=%d Sk=%d D=%d)", B, H, Sq, Sk, D);
  if (D != 32 && D != 64 && D != 128 && D != 256 && D != 512 && D != 1024)
    return fail(FA_ERR_UNSUPPORTED, "head dim %d not in {32, 64, 128, 256, 512, 1024}", D);
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", causal);
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(FA_ERR_INVALID_ARG, "q, k, v, o must be 16-byte aligned");
  if (!aligned(lse, 4)) return fail(FA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (!product_le(B, H, Sq, D, kMaxElems) || !product_le(B, H, Sk, D, kMaxElems))
    return fail(FA_ERR_INVALID_ARG, "tensor too large");
  // one (batch, head) slice is addressed with 32-bit byte offsets
  if ((int64_t)Sq * D * 2 >= kMaxSliceBytes || (int64_t)Sk * D * 2 >= kMaxSliceBytes)
    return fail(FA_ERR_INVALID_ARG, "sequence too long: one [S, D] slice must stay below 2 GiB");
  return FA_OK;
}

int hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(FA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return FA_OK;
}

int launched(const char* what) { return hip_check(hipGetLastError(), what); }

int device_cu_count(int* out);
int workspace_pool(hipMemPool_t* out);
size_t ws_bytes(int64_t BH, int D, int ns);

// Key-tile width of the D <= 128 prefill kernels: 32 keys at D = 128, 64
// below (every D = 128 kernel uses the same width, so a sequence gives the
// same bits through the dense, packed and split paths' tile loops).
template <int D>
constexpr int fa_bn() { return D == 128 ? 32 : 64; }

// Key-range split of a small prefill grid (fa::KeySplit).  Parts (D <=
// 128): query tiles ts .. nqt-1 in ns parts each.  Runs (D = 256): the key
// tiles of all query tiles cut into `grid` runs (split_start).
struct SplitPlan {
  int ts = 0, ns = 1;     // parts
  int runs = 0, bias = 0;  // runs: run count and bias (split_start)
  int units = 0;          // runs: key tiles of one slice
  int64_t total = 0;      // runs: key tiles of all slices
  int64_t grid = 0;       // workgroups of the split kernel (0: no split)
  int max_parts = 1;      // most parts any query tile is cut into
};

// Cost model of a parts plan (D <= 128, the 4-wavefront kernel), fitted to
// 34 timed plans over five shapes (kernels and merge, rocprofv3 kernel
// trace): with these constants every shape gets its fastest measured plan
// or one within 1% of it (and the shapes where no split paid stay whole).
// A work item costs its key tiles at unit_us each plus item_us of fixed
// work (Q load, pipeline fill, epilogue); items go, heaviest first, to the
// CU that frees first; and the whole job takes at least full_load times its
// mean time per CU (the clock of a fully loaded chip is lower than that of
// one whose last heavy tiles run alone).
struct PartsModel {
  double unit_us, item_us, full_load, min_gain;
  bool causal_only;
};

PartsModel fwd_parts_model(int D) {
  // a lone 4-wavefront workgroup of 128 rows runs a 64-key tile of D = 128
  // in ~1.2 us; non-causal grids measured no gain from splitting
  return {1.2 * D / 128.0, 3.0, 1.0, 0.7, true};
}

double fwd_parts_time(int nqt, int BH, int BM, int BN, int Sq, int Sk, bool causal, int ts, int ns, int slots,
                      const PartsModel& m) {
  std::vector<double> finish((size_t)slots, 0.0);  // min-heap of slot finishing times
  double total = 0.0;
  auto push = [&](int units) {
    const double w = units * m.unit_us + m.item_us;
    std::pop_heap(finish.begin(), finish.end(), std::greater<double>());
    finish.back() += w;
    std::push_heap(finish.begin(), finish.end(), std::greater<double>());
    total += w;
  };
  int th = nqt - 1, tl = ts - 1;
  for (;;) {
    const int wh = th >= ts ? (fa::fwd_tile_units(th, BM, BN, Sq, Sk, causal) + ns - 1) / ns : -1;
    const int wl = tl >= 0 ? fa::fwd_tile_units(tl, BM, BN, Sq, Sk, causal) : -1;
    if (wh < 0 && wl < 0) break;
    if (wh >= wl) {
      for (int i = 0; i < ns * BH; ++i) push(wh);
      --th;
    } else {
      for (int i = 0; i < BH; ++i) push(wl);
      --tl;
    }
  }
  const double makespan = *std::max_element(finish.begin(), finish.end());
  return std::max(makespan, m.full_load * total / slots);
}

// Split only grids of at most two work items per CU, and only when the
// modelled time plus the merge (its HBM bytes at ~4.5 TB/s, and a launch)
// beats the unsplit grid by the model's margin.
SplitPlan plan_fwd_parts(int nqt, int BH, int BM, int BN, int D, int Sq, int Sk, bool causal, int cus) {
  SplitPlan best;
  const PartsModel m = fwd_parts_model(D);
  if (cus < 1 || (int64_t)nqt * BH > 2 * (int64_t)cus || (m.causal_only && !causal)) return best;
  double best_cost = m.min_gain * fwd_parts_time(nqt, BH, BM, BN, Sq, Sk, causal, nqt, 1, cus, m);
  const int starts[4] = {0, nqt / 4, nqt / 2, 3 * nqt / 4};
  const int parts[5] = {2, 3, 4, 6, 8};
  for (int ts : starts) {
    if (ts >= nqt || (!causal && ts > 0)) continue;
    for (int ns : parts) {
      if (ns > fa::fwd_tile_units(ts, BM, BN, Sq, Sk, causal)) continue;
      const int64_t grid = (int64_t)BH * ((int64_t)(nqt - ts) * ns + ts);
      if (grid > kMaxGrid) continue;
      const double rows = (double)BH * (nqt - ts) * BM;
      // partials read back, O and LSE written
      const double bytes = rows * (ns * (D + 1) * 4.0 + D * 2.0 + 4.0);
      const double cost = fwd_parts_time(nqt, BH, BM, BN, Sq, Sk, causal, ts, ns, cus, m) + bytes / 4.5e6 + 2.0;
      if (cost < best_cost) {
        best_cost = cost;
        best.ts = ts;
        best.ns = ns;
        best.grid = grid;
        best.max_parts = ns;
      }
    }
  }
  return best;
}

// Cost model of a runs plan (D = 256), from per-workgroup start / end
// times read inside the kernel (s_memrealtime) on the (1, 16, 2048, 2048,
// 256) causal grid.  Unsplit: a workgroup takes lone_unit_us per key tile
// plus lone_first_us (Q and the first K / V tiles, every workgroup loading
// at once), and the last heavy tiles run at that rate while the light ones
// have finished.  Runs (every CU busy to the end): unit_us per key tile,
// first_us for a run's first segment and seg_us for each further one; the
// merge reads the partials at merge_bw bytes per us after merge_us.
struct RunsModel {
  double lone_unit_us, lone_first_us, unit_us, first_us, seg_us, merge_us, merge_bw;
};

constexpr RunsModel kRunsModel = {0.82, 6.0, 0.92, 7.9, 3.9, 3.0, 4.0e6};

// The same model for the Split-D kernel at D = 512 (32-row tiles, 32-key
// tiles): unsplit, 50.6 us for the heaviest causal tile (32 key tiles) run
// while the others finish; split into runs of 16.5 key tiles, 35.9 us plus
// an 8.6 us merge of 16 MiB of partials (kernel trace, (1, 8, 1024, 1024,
// 512) causal).  At D = 1024 the grids of the pages' shapes are too short
// for runs (544 key tiles on 256 CUs): runs measured slower than equal key
// parts there, so D = 1024 keeps the parts.
constexpr RunsModel kSplitDRunsModel = {1.46, 4.0, 1.69, 5.0, 3.0, 4.5, 4.0e6};

// Makespan of the unsplit grid: query tiles heaviest first, each to the CU
// that frees first.
double fwd_unsplit_time(int nqt, int BH, int BM, int BN, int Sq, int Sk, bool causal, int cus, const RunsModel& m) {
  std::vector<double> finish((size_t)cus, 0.0);  // min-heap of CU finishing times
  for (int r = 0; r < nqt; ++r) {
    const int t = causal ? nqt - 1 - r : r;
    const double w = fa::fwd_tile_units(t, BM, BN, Sq, Sk, causal) * m.lone_unit_us + m.lone_first_us;
    for (int i = 0; i < BH; ++i) {
      std::pop_heap(finish.begin(), finish.end(), std::greater<double>());
      finish.back() += w;
      std::push_heap(finish.begin(), finish.end(), std::greater<double>());
    }
  }
  return *std::max_element(finish.begin(), finish.end());
}

// Modelled time of these runs: the slowest run, plus the merge of the cut
// tiles.  Also reports the most parts of any tile.
double fwd_runs_time(int nqt, int BH, int BM, int BN, int D, int Sq, int Sk, bool causal, int runs, int total,
                     int bias, const RunsModel& m, int* max_parts) {
  std::vector<double> cost((size_t)runs, 0.0);
  std::vector<char> started((size_t)runs, 0);
  int64_t cut_parts = 0;
  *max_parts = 1;
  int64_t lin = 0;
  for (int b = 0; b < BH; ++b)
    for (int i = 0; i < nqt; ++i) {
      const int r = fa::split_order(i, nqt);
      const int u = fa::fwd_tile_units(causal ? nqt - 1 - r : r, BM, BN, Sq, Sk, causal);
      const int g0 = fa::split_run((int)lin, runs, total, bias);
      const int g1 = fa::split_run((int)(lin + u - 1), runs, total, bias);
      for (int g = g0; g <= g1; ++g) {
        const int64_t lo = std::max<int64_t>(lin, fa::split_start(g, runs, total, bias));
        const int64_t hi = std::min<int64_t>(lin + u, fa::split_start(g + 1, runs, total, bias));
        cost[(size_t)g] += (hi - lo) * m.unit_us + (started[(size_t)g] ? m.seg_us : m.first_us);
        started[(size_t)g] = 1;
      }
      if (g1 > g0) cut_parts += g1 - g0 + 1;
      *max_parts = std::max(*max_parts, g1 - g0 + 1);
      lin += u;
    }
  const double merge = cut_parts ? m.merge_us + (double)cut_parts * BM * (D + 1) * 4.0 / m.merge_bw : 0.0;
  return *std::max_element(cost.begin(), cost.end()) + merge;
}

// Split only grids of at most two query tiles per CU, and only when the
// best modelled runs (one per CU, biases 0 .. a quarter of a run) beat the
// unsplit grid by 10%.
SplitPlan plan_fwd_runs(int nqt, int BH, int BM, int BN, int D, int Sq, int Sk, bool causal, int cus,
                        const RunsModel& m) {
  SplitPlan best;
  if (cus < 1 || (int64_t)nqt * BH > 2 * (int64_t)cus) return best;
  int64_t units = 0;
  int umax = 0;
  for (int t = 0; t < nqt; ++t) {
    const int u = fa::fwd_tile_units(t, BM, BN, Sq, Sk, causal);
    units += u;
    umax = std::max(umax, u);
  }
  const int64_t total = units * BH;
  if (total > (int64_t)1 << 28) return best;
  double best_time = 0.9 * fwd_unsplit_time(nqt, BH, BM, BN, Sq, Sk, causal, cus, m);
  // one run per CU, but at least 4 key tiles per run, and no tile in more
  // than 8 parts (what the merge loads at once): a run holds at least a
  // seventh of the longest tile
  int64_t runs = std::min<int64_t>(cus, total / 4);
  runs = std::min<int64_t>(runs, 7 * total / umax);
  // the run boundaries are computed in 32-bit unsigned arithmetic
  if (runs < 2 || (runs + 8) * total >= ((int64_t)1 << 32)) return best;
  const int len = (int)(total / runs);  // shortest run before the bias
  const int step = std::max(1, (len / 4) / 8);
  for (int bias = 0; bias <= len / 4; bias += step) {
    int max_parts = 1;
    const double t =
        fwd_runs_time(nqt, BH, BM, BN, D, Sq, Sk, causal, (int)runs, (int)total, bias, m, &max_parts);
    if (t < best_time) {
      best_time = t;
      best.runs = (int)runs;
      best.bias = bias;
      best.units = (int)units;
      best.total = total;
      best.grid = runs;
      best.max_parts = max_parts;
    }
  }
  return best;
}

size_t round256(size_t n) { return (n + 255) / 256 * 256; }

// Workspace of a runs split: the partial O [grid, 2, BM, D] and
// log2-sum-exp [grid, 2, BM] of every run.
size_t runs_ws_bytes(int BM, int D, const SplitPlan& pl) {
  return round256((size_t)pl.grid * 2 * BM * D * 4) + round256((size_t)pl.grid * 2 * BM * 4);
}

// Launches an instantiation of fa::fwd_kernel (its LDS is static).
template <int D, int BN, int NW, bool CAUSAL, bool VARLEN, bool KSPLIT, int RES = 0, class... Args>
int launch_fwd_kernel(unsigned grid, hipStream_t stream, const char* what, Args... args) {
  using Cfg = fa::FwdCfg<D, BN, NW>;
  hipLaunchKernelGGL((fa::fwd_kernel<D, BN, NW, CAUSAL, VARLEN, KSPLIT, RES>), dim3(grid), dim3(Cfg::THREADS), 0,
                     stream, args...);
  return launched(what);
}

// The parts merge (fwd_merge_kernel) instantiated for the smallest bound
// on the parts that holds ns (the parts planner cuts at most 8, Split-D at
// most 16).
template <int D>
int launch_fwd_merge(const float* ws_o, const float* ws_lse, void* o, float* lse, int Sq, int BM, int ts,
                     int nsplit, int ns, int64_t rows, hipStream_t stream, const char* what) {
  if (ns < 1 || ns > 16) return fail(FA_ERR_INVALID_ARG, "%s: %d key parts (at most 16)", what, ns);
  auto go = [&](auto bound) {
    constexpr int NP = decltype(bound)::value;
    constexpr int R = fa::MergeCfg<D, NP>::ROWS;
    hipLaunchKernelGGL((fa::fwd_merge_kernel<D, NP>), dim3((unsigned)((rows + R - 1) / R)), dim3(256), 0, stream,
                       ws_o, ws_lse, static_cast<_Float16*>(o), lse, Sq, BM, ts, nsplit, ns, (int)rows);
    return launched(what);
  };
  if (ns <= 2) return go(std::integral_constant<int, 2>{});
  if (ns <= 4) return go(std::integral_constant<int, 4>{});
  if (ns <= 8) return go(std::integral_constant<int, 8>{});
  return go(std::integral_constant<int, 16>{});
}

template <int D, int BN, int NW, bool CAUSAL>
int launch_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int Sq, int Sk,
                     float scale, hipStream_t stream, const SplitPlan& pl, void* ws) {
  using Cfg = fa::FwdCfg<D, BN, NW>;
  const int nqt = (Sq + Cfg::BM - 1) / Cfg::BM;
  fa::KeySplit ksp = {};
  if constexpr (fa::split_by_runs<D>()) {
    ksp.runs = pl.runs;
    ksp.bias = pl.bias;
    ksp.units = pl.units;
    ksp.total = (int)pl.total;
    ksp.ws_o = static_cast<float*>(ws);
    ksp.ws_lse = reinterpret_cast<float*>(static_cast<char*>(ws) + round256((size_t)pl.grid * 2 * Cfg::BM * D * 4));
    int rc = launch_fwd_kernel<D, BN, NW, CAUSAL, false, true>(
        (unsigned)((pl.grid + 7) / 8 * 8), stream, "fa_fwd split kernel launch", static_cast<const _Float16*>(q),
        static_cast<const _Float16*>(k), static_cast<const _Float16*>(v), static_cast<_Float16*>(o), lse, Sq, Sk,
        BH, nqt, scale * fa::kLog2e, fa::VarlenArgs{}, ksp);
    if (rc != FA_OK) return rc;
    auto merge = [&](auto nparts) {
      constexpr int NP = decltype(nparts)::value;
      using M = fa::SplitMergeCfg<D, Cfg::BM, NP>;
      hipLaunchKernelGGL((fa::fwd_split_merge_kernel<D, Cfg::BM, BN, CAUSAL, NP>), dim3((unsigned)(BH * nqt * M::BLOCKS)),
                         dim3(M::THREADS), 0, stream, ksp, static_cast<_Float16*>(o), lse, Sq, Sk, nqt);
      return launched("fa_fwd split merge launch");
    };
    if (pl.max_parts <= 2) return merge(std::integral_constant<int, 2>{});
    if (pl.max_parts <= 4) return merge(std::integral_constant<int, 4>{});
    return merge(std::integral_constant<int, 8>{});
  } else {
    const int nsplit = nqt - pl.ts;
    const int64_t rows = (int64_t)BH * nsplit * Cfg::BM;
    ksp.ts = pl.ts;
    ksp.ns = pl.ns;
    ksp.ws_o = static_cast<float*>(ws);
    ksp.ws_lse = ksp.ws_o + (size_t)rows * pl.ns * D;
    int rc = launch_fwd_kernel<D, BN, NW, CAUSAL, false, true>(
        (unsigned)pl.grid, stream, "fa_fwd key-split kernel launch", static_cast<const _Float16*>(q),
        static_cast<const _Float16*>(k), static_cast<const _Float16*>(v), static_cast<_Float16*>(o), lse, Sq, Sk,
        BH, nqt, scale * fa::kLog2e, fa::VarlenArgs{}, ksp);
    if (rc != FA_OK) return rc;
    return launch_fwd_merge<D>(ksp.ws_o, ksp.ws_lse, o, lse, Sq, Cfg::BM, pl.ts, nsplit, pl.ns, rows, stream,
                               "fa_fwd key-split merge launch");
  }
}

template <int D, int BN, int NW, bool CAUSAL>
int launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int Sq, int Sk,
               float scale, hipStream_t stream, const SplitPlan& pl, void* ws) {
  using Cfg = fa::FwdCfg<D, BN, NW>;
  if (pl.grid > 0) return launch_fwd_split<D, BN, NW, CAUSAL>(q, k, v, o, lse, BH, Sq, Sk, scale, stream, pl, ws);
  const int nqt = (Sq + Cfg::BM - 1) / Cfg::BM;
  auto run = [&](auto res) {
    return launch_fwd_kernel<D, BN, NW, CAUSAL, false, false, decltype(res)::value>(
        (unsigned)(nqt * BH), stream, "fa_fwd kernel launch", static_cast<const _Float16*>(q),
        static_cast<const _Float16*>(k), static_cast<const _Float16*>(v), static_cast<_Float16*>(o), lse, Sq, Sk, BH,
        nqt, scale * fa::kLog2e, fa::VarlenArgs{}, fa::KeySplit{});
  };
  // short key ranges on the two-workgroups-per-CU kernel: every key tile
  // copied to LDS once, in the prologue
  if constexpr (NW == 4 && D <= 128) {
    constexpr int RES = fa::fwd_resident_tiles<D, BN>();
    if ((Sk + BN - 1) / BN <= RES) return run(std::integral_constant<int, RES>{});
  }
  return run(std::integral_constant<int, 0>{});
}

// The tile kernel of head dim D with the geometry the plan chose: D = 256
// 32-key tiles; D = 32 always 128-row workgroups (a 64-key tile of D = 32
// is 4 KiB: one 1 KiB copy for each of 4 wavefronts); D = 64, 128 256-row
// workgroups when the plan says so (with 32-key tiles at D = 128).
template <int D, bool CAUSAL>
int launch_fwd_d(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int Sq, int Sk,
                 float scale, hipStream_t stream, int nw, const SplitPlan& pl, void* ws) {
  if constexpr (D == 256) {
    return launch_fwd<256, 32, 4, CAUSAL>(q, k, v, o, lse, BH, Sq, Sk, scale, stream, pl, ws);
  } else if constexpr (D == 32) {
    return launch_fwd<32, 64, 4, CAUSAL>(q, k, v, o, lse, BH, Sq, Sk, scale, stream, pl, ws);
  } else {
    // D = 128: 32-key tiles in every kernel (the scores take 16 registers
    // instead of 32; the 8-wavefront kernel 192 VGPRs against 240, measured
    // 0-1.4% faster on the 4096-token causal prefill, about 1% on average)
    constexpr int BN = fa_bn<D>();
    if (nw == 8) return launch_fwd<D, BN, 8, CAUSAL>(q, k, v, o, lse, BH, Sq, Sk, scale, stream, pl, ws);
    return launch_fwd<D, BN, 4, CAUSAL>(q, k, v, o, lse, BH, Sq, Sk, scale, stream, pl, ws);
  }
}

template <int D, int BN, int NW, bool CAUSAL>
int launch_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, fa::VarlenArgs va, int B,
                      float scale, hipStream_t stream) {
  using Cfg = fa::FwdCfg<D, BN, NW>;
  const int nqt = (va.max_q + Cfg::BM - 1) / Cfg::BM;
  const int64_t BH = (int64_t)B * va.H;
  const int64_t grid = (BH + 7) / 8 * 8 * nqt;  // slice count rounded up to a multiple of 8 (one per XCD)
  if (grid > kMaxGrid) return fail(FA_ERR_INVALID_ARG, "grid too large");
  return launch_fwd_kernel<D, BN, NW, CAUSAL, true, false>(
      (unsigned)grid, stream, "fa_fwd_varlen kernel launch", static_cast<const _Float16*>(q),
      static_cast<const _Float16*>(k), static_cast<const _Float16*>(v), static_cast<_Float16*>(o), lse, 0, 0,
      (int)BH, nqt, scale * fa::kLog2e, va, fa::KeySplit{});
}

template <int D, bool CAUSAL>
int launch_fwd_varlen_d(const void* q, const void* k, const void* v, void* o, float* lse, fa::VarlenArgs va, int B,
                        float scale, hipStream_t stream) {
  if constexpr (D == 256) {
    return launch_fwd_varlen<256, 32, 4, CAUSAL>(q, k, v, o, lse, va, B, scale, stream);
  } else if constexpr (D == 32) {
    return launch_fwd_varlen<32, 64, 4, CAUSAL>(q, k, v, o, lse, va, B, scale, stream);
  } else {
    int cus = 0;
    int rc = device_cu_count(&cus);
    if (rc != FA_OK) return rc;
    // 256-row workgroups only for long sequences: each sequence's last
    // query tile is partly empty, and a half-idle 8-wavefront workgroup holds
    // its whole CU (the ragged 256..4096-token batch, 2156 tokens on average,
    // ran 9% faster with 128-row workgroups; dense 4096-token prefill 7%
    // slower)
    const int64_t wg8 = (int64_t)B * va.H * ((va.max_q + 255) / 256);
    if (wg8 >= cus && va.total_q >= (int64_t)3072 * B)
      return launch_fwd_varlen<D, fa_bn<D>(), 8, CAUSAL>(q, k, v, o, lse, va, B, scale, stream);
    return launch_fwd_varlen<D, fa_bn<D>(), 4, CAUSAL>(q, k, v, o, lse, va, B, scale, stream);
  }
}

// Head dims above 256: Split-D, one workgroup of D/128 wavefronts per 32
// query rows.
template <int D, bool CAUSAL>
int launch_fwd_splitd(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int Sq, int Sk,
                      float scale, hipStream_t stream, int ns, float* ws_o, float* ws_lse) {
  const int nqt = (Sq + 31) / 32;
  hipLaunchKernelGGL((fa::fwd_splitd_kernel<D, CAUSAL>), dim3(nqt * BH * ns), dim3(fa::SplitDCfg<D>::THREADS), 0,
                     stream, static_cast<const _Float16*>(q), static_cast<const _Float16*>(k),
                     static_cast<const _Float16*>(v), static_cast<_Float16*>(o), lse, Sq, Sk, BH, nqt, ns,
                     scale * fa::kLog2e, ws_o, ws_lse);
  int rc = launched("fa_fwd Split-D kernel launch");
  if (rc != FA_OK || ns == 1) return rc;
  // combine the key parts of every query row: rows of [BH * Sq, ns, D], one
  // tile of Sq rows per slice in the merge kernel's terms
  const int64_t rows = (int64_t)BH * Sq;
  if (rows > kMaxGrid) return fail(FA_ERR_INVALID_ARG, "grid too large");
  return launch_fwd_merge<D>(ws_o, ws_lse, o, lse, Sq, Sq, 0, 1, ns, rows, stream, "fa_fwd Split-D merge launch");
}

// Workgroup size of the single-partition decode (its in-LDS merge writes
// the final output; no workspace, no merge kernel).
constexpr int kDecFusedThreads = 1024;

// Phase two of the split decode: 1024-thread merge workgroups when 256
// threads would leave each partition group more than 4 partitions.
template <int D>
void launch_decode_merge(int BH, int ns, hipStream_t stream, const float* ws_o, const float* ws_lse, _Float16* o,
                         float* lse) {
  if (ns > 4 * fa::DecMergeCfg<D, 256>::G)
    hipLaunchKernelGGL((fa::decode_merge_kernel<D, 1024>), dim3(BH), dim3(1024), 0, stream, ws_o, ws_lse, o, lse, ns);
  else
    hipLaunchKernelGGL((fa::decode_merge_kernel<D, 256>), dim3(BH), dim3(256), 0, stream, ws_o, ws_lse, o, lse, ns);
}

template <int D>
int launch_decode(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int Sk,
                  float scale, hipStream_t stream, int ns, float* ws_o, float* ws_lse) {
  const int chunk = (Sk + ns - 1) / ns;
  const float c2 = scale * fa::kLog2e;
  if (ns == 1) {
    hipLaunchKernelGGL((fa::decode_partial_kernel<D, kDecFusedThreads, true>), dim3(BH), dim3(kDecFusedThreads), 0,
                       stream, static_cast<const _Float16*>(q), static_cast<const _Float16*>(k),
                       static_cast<const _Float16*>(v), nullptr, nullptr, static_cast<_Float16*>(o), lse, Sk, 1,
                       Sk, c2);
    return launched("decode launch");
  }
  hipLaunchKernelGGL((fa::decode_partial_kernel<D, 256, false>), dim3(BH * ns), dim3(256), 0, stream,
                     static_cast<const _Float16*>(q), static_cast<const _Float16*>(k),
                     static_cast<const _Float16*>(v), ws_o, ws_lse, nullptr, nullptr, Sk, ns, chunk, c2);
  int rc = launched("decode phase-one launch");
  if (rc != FA_OK) return rc;
  launch_decode_merge<D>(BH, ns, stream, ws_o, ws_lse, static_cast<_Float16*>(o), lse);
  return launched("decode merge launch");
}

template <int D, int T, bool FINAL, bool GROUP>
void launch_paged_partial(const void* q, const void* kc, const void* vc, const int* tables, const int* seq_lens,
                          float* ws_o, float* ws_lse, void* o, float* lse, int BH, int H, int ns, int num_blocks,
                          int lbs, int max_blocks, float c2, hipStream_t stream) {
  hipLaunchKernelGGL((fa::decode_paged_partial_kernel<D, T, FINAL, GROUP>), dim3(BH * ns), dim3(T), 0, stream,
                     static_cast<const _Float16*>(q), static_cast<const _Float16*>(kc),
                     static_cast<const _Float16*>(vc), tables, seq_lens, ws_o, ws_lse, static_cast<_Float16*>(o),
                     lse, H, ns, num_blocks, lbs, max_blocks, c2);
}

template <int D>
int launch_decode_paged(const void* q, const void* kc, const void* vc, const int* tables, const int* seq_lens,
                        void* o, float* lse, int B, int H, int num_blocks, int lbs, int max_blocks, float scale,
                        hipStream_t stream, int ns, float* ws_o, float* ws_lse) {
  const float c2 = scale * fa::kLog2e;
  const int BH = B * H;
  // a wavefront's group of keys lies in one page: translated once per group
  const bool group = (1 << lbs) >= fa::DecCfg<D>::KEYS_PER_WAVE_ITER;
  if (ns == 1) {
    if (group)
      launch_paged_partial<D, kDecFusedThreads, true, true>(q, kc, vc, tables, seq_lens, nullptr, nullptr, o, lse,
                                                            BH, H, 1, num_blocks, lbs, max_blocks, c2, stream);
    else
      launch_paged_partial<D, kDecFusedThreads, true, false>(q, kc, vc, tables, seq_lens, nullptr, nullptr, o, lse,
                                                             BH, H, 1, num_blocks, lbs, max_blocks, c2, stream);
    return launched("paged decode launch");
  }
  if (group)
    launch_paged_partial<D, 256, false, true>(q, kc, vc, tables, seq_lens, ws_o, ws_lse, nullptr, nullptr, BH, H, ns,
                                              num_blocks, lbs, max_blocks, c2, stream);
  else
    launch_paged_partial<D, 256, false, false>(q, kc, vc, tables, seq_lens, ws_o, ws_lse, nullptr, nullptr, BH, H,
                                               ns, num_blocks, lbs, max_blocks, c2, stream);
  int rc = launched("paged decode phase-one launch");
  if (rc != FA_OK) return rc;
  launch_decode_merge<D>(BH, ns, stream, ws_o, ws_lse, static_cast<_Float16*>(o), lse);
  return launched("paged decode merge launch");
}

template <int D, bool CAUSAL>
int launch_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
               void* dq, void* dk, void* dv, int BH, int Sq, int Sk, float scale, hipStream_t stream, float* dvec) {
  constexpr int NW = 4;
  const int64_t rows = (int64_t)BH * Sq;
  const int64_t kv_grid = (int64_t)((Sk + 32 * NW - 1) / (32 * NW)) * BH;
  const int nqt = (Sq + 32 * NW - 1) / (32 * NW);
  const int64_t q_grid = (int64_t)nqt * BH;
  if (kv_grid > kMaxGrid || q_grid > kMaxGrid) return fail(FA_ERR_INVALID_ARG, "grid too large");
  const auto* Q = static_cast<const _Float16*>(q);
  const auto* K = static_cast<const _Float16*>(k);
  const auto* V = static_cast<const _Float16*>(v);
  const auto* dO = static_cast<const _Float16*>(dout);
  float* l2 = dvec + rows;  // LSE in log2 units
  int rc = FA_OK;
  // dynamic LDS; above 64 KiB (D = 256) the kernels must be allowed it first
  constexpr int kv_dyn = fa::dkdv_lds_bytes<D, NW>();
  constexpr int q_dyn = fa::dq_lds_bytes<D, NW>();
  static_assert(kv_dyn <= 160 * 1024 && q_dyn <= 160 * 1024, "LDS budget per CU");
  auto* kv_kern = &fa::bwd_dkdv_kernel<D, NW, CAUSAL>;
  auto* q_kern = &fa::bwd_dq_kernel<D, NW, CAUSAL>;
  if constexpr (kv_dyn > 65536) {
    rc = hip_check(hipFuncSetAttribute(reinterpret_cast<const void*>(kv_kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kv_dyn),
                   "fa_bwd LDS size attribute");
    if (rc != FA_OK) return rc;
  }
  if constexpr (q_dyn > 65536) {
    rc = hip_check(hipFuncSetAttribute(reinterpret_cast<const void*>(q_kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, q_dyn),
                   "fa_bwd LDS size attribute");
    if (rc != FA_OK) return rc;
  }
  // dQ first: it also writes D and the log2 LSE of every query row, which
  // the dK/dV kernel reads
  hipLaunchKernelGGL(q_kern, dim3((unsigned)q_grid), dim3(64 * NW), q_dyn, stream, Q, K, V,
                     static_cast<const _Float16*>(o), dO, lse, l2, dvec, static_cast<_Float16*>(dq), Sq, Sk, BH, nqt,
                     scale);
  rc = launched("fa_bwd dQ launch");
  if (rc != FA_OK) return rc;
  hipLaunchKernelGGL(kv_kern, dim3((unsigned)kv_grid), dim3(64 * NW), kv_dyn, stream, Q, K, V, dO, l2, dvec,
                     static_cast<_Float16*>(dk), static_cast<_Float16*>(dv), Sq, Sk, BH, (int)(kv_grid / BH), scale);
  return launched("fa_bwd dK/dV launch");
}

std::atomic<int> g_cu_count[64];

int device_cu_count(int* out) {
  int dev = 0;
  int rc = hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (rc != FA_OK) return rc;
  if (dev >= 0 && dev < 64) {
    const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0) {
      *out = cached;
      return FA_OK;
    }
  }
  int n = 0;
  rc = hip_check(hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev), "CU count query");
  if (rc != FA_OK) return rc;
  if (dev >= 0 && dev < 64) g_cu_count[dev].store(n, std::memory_order_relaxed);
  *out = n;
  return FA_OK;
}

// One stream-ordered memory pool per device for decode workspaces.  Its
// release threshold is unlimited, so memory freed with hipFreeAsync stays in
// the pool and the next call reuses it without a new device allocation.
constexpr int kMaxDevices = 64;
std::mutex g_pool_mu;
hipMemPool_t g_pool[kMaxDevices] = {};

int workspace_pool(hipMemPool_t* out) {
  int dev = 0;
  int rc = hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (rc != FA_OK) return rc;
  if (dev < 0 || dev >= kMaxDevices) return fail(FA_ERR_HIP, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_pool_mu);
  if (!g_pool[dev]) {
    hipMemPoolProps props = {};
    props.allocType = hipMemAllocationTypePinned;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool = nullptr;
    rc = hip_check(hipMemPoolCreate(&pool, &props), "hipMemPoolCreate");
    if (rc != FA_OK) return rc;
    uint64_t keep = UINT64_MAX;
    rc = hip_check(hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep), "pool release threshold");
    if (rc != FA_OK) {
      (void)hipMemPoolDestroy(pool);
      return rc;
    }
    g_pool[dev] = pool;
  }
  *out = g_pool[dev];
  return FA_OK;
}

size_t ws_bytes(int64_t BH, int D, int ns) {
  const size_t floats = (size_t)BH * ns * (D + 1);
  return (floats * 4 + 255) / 256 * 256;
}

// Key parts for the Split-D forward: 1 when the (query tile, slice) work
// items give every CU one, else enough parts to do so, each of at least two
// key tiles, at most 16.  (A second co-resident workgroup per CU, which the
// D = 512 kernel's LDS would allow, measured slower once the merge is paid:
// the CU's LDS and copy bandwidth is already the limit.)
int splitd_parts(int64_t work_items, int nkt_all, int cus) {
  if (work_items >= cus) return 1;
  int64_t ns = (cus + work_items - 1) / work_items;
  ns = std::min<int64_t>(ns, std::max(1, nkt_all / 2));
  ns = std::min<int64_t>(ns, 16);
  return (int)std::max<int64_t>(ns, 1);
}

// Split-D split into runs (fwd_splitd_kernel<D, CAUSAL, true>) and the
// merge of its cut tiles.
template <int D, bool CAUSAL>
int launch_fwd_splitd_runs(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int Sq, int Sk,
                           float scale, hipStream_t stream, const SplitPlan& pl, void* ws) {
  const int nqt = (Sq + 31) / 32;
  fa::KeySplit ksp = {};
  ksp.runs = pl.runs;
  ksp.bias = pl.bias;
  ksp.units = pl.units;
  ksp.total = (int)pl.total;
  ksp.ws_o = static_cast<float*>(ws);
  ksp.ws_lse = reinterpret_cast<float*>(static_cast<char*>(ws) + round256((size_t)pl.grid * 2 * 32 * D * 4));
  hipLaunchKernelGGL((fa::fwd_splitd_kernel<D, CAUSAL, true>), dim3((unsigned)((pl.grid + 7) / 8 * 8)),
                     dim3(fa::SplitDCfg<D>::THREADS), 0, stream, static_cast<const _Float16*>(q),
                     static_cast<const _Float16*>(k), static_cast<const _Float16*>(v), static_cast<_Float16*>(o), lse,
                     Sq, Sk, BH, nqt, 1, scale * fa::kLog2e, nullptr, nullptr, ksp);
  int rc = launched("fa_fwd Split-D split kernel launch");
  if (rc != FA_OK) return rc;
  auto merge = [&](auto nparts) {
    constexpr int NP = decltype(nparts)::value;
    using M = fa::SplitMergeCfg<D, 32, NP>;
    hipLaunchKernelGGL((fa::fwd_split_merge_kernel<D, 32, 32, CAUSAL, NP>), dim3((unsigned)(BH * nqt * M::BLOCKS)),
                       dim3(M::THREADS), 0, stream, ksp, static_cast<_Float16*>(o), lse, Sq, Sk, nqt);
    return launched("fa_fwd Split-D split merge launch");
  };
  if (pl.max_parts <= 2) return merge(std::integral_constant<int, 2>{});
  if (pl.max_parts <= 4) return merge(std::integral_constant<int, 4>{});
  return merge(std::integral_constant<int, 8>{});
}

template <int D>
int run_fwd_splitd(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int Sq, int Sk,
                   int causal, float scale, hipStream_t s, int ns, void* ws, const SplitPlan& pl) {
  if (pl.grid > 0)
    return causal ? launch_fwd_splitd_runs<D, true>(q, k, v, o, lse, BH, Sq, Sk, scale, s, pl, ws)
                  : launch_fwd_splitd_runs<D, false>(q, k, v, o, lse, BH, Sq, Sk, scale, s, pl, ws);
  float* ws_o = static_cast<float*>(ws);  // unused (may be null) without a key split
  float* ws_lse = ns > 1 ? ws_o + (size_t)BH * Sq * ns * D : nullptr;
  return causal ? launch_fwd_splitd<D, true>(q, k, v, o, lse, BH, Sq, Sk, scale, s, ns, ws_o, ws_lse)
                : launch_fwd_splitd<D, false>(q, k, v, o, lse, BH, Sq, Sk, scale, s, ns, ws_o, ws_lse);
}

int validate_decode(const void* q, const void* k, const void* v, const void* o, const void* lse, int B, int H,
                    int Sq, int Sk, int D, int causal, float scale, int num_splits) {
  int rc = validate(q, k, v, o, lse, B, H, Sq, Sk, D, causal, scale);
  if (rc != FA_OK) return rc;
  if (D > 256) return fail(FA_ERR_UNSUPPORTED, "split-KV decoding supports head dims 32, 64, 128, 256");
  if (Sq != 1) return fail(FA_ERR_INVALID_ARG, "split-KV decoding needs Sq == 1 (got %d)", Sq);
  if (causal != 0) return fail(FA_ERR_INVALID_ARG, "split-KV decoding is non-causal");
  if (num_splits > Sk) return fail(FA_ERR_INVALID_ARG, "num_splits %d exceeds Sk %d", num_splits, Sk);
  if ((int64_t)B * H * (num_splits > 0 ? num_splits : 1) > kMaxGrid) return fail(FA_ERR_INVALID_ARG, "grid too large");
  return FA_OK;
}

int run_decode(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int Sk, int D,
               float scale, hipStream_t stream, int ns, void* ws) {
  float* ws_o = static_cast<float*>(ws);  // unused (may be null) with a single partition
  float* ws_lse = ws ? ws_o + (size_t)BH * ns * D : nullptr;
  switch (D) {
    case 32: return launch_decode<32>(q, k, v, o, lse, BH, Sk, scale, stream, ns, ws_o, ws_lse);
    case 64: return launch_decode<64>(q, k, v, o, lse, BH, Sk, scale, stream, ns, ws_o, ws_lse);
    case 128: return launch_decode<128>(q, k, v, o, lse, BH, Sk, scale, stream, ns, ws_o, ws_lse);
    default: return launch_decode<256>(q, k, v, o, lse, BH, Sk, scale, stream, ns, ws_o, ws_lse);
  }
}

int validate_varlen(const void* q, const void* k, const void* v, const void* o, const void* lse, const int* cu_q,
                    const int* cu_k, int B, int H, int total_q, int total_k, int max_q, int max_k, int D,
                    int causal, float scale) {
  if (!q || !k || !v || !o || !lse || !cu_q || !cu_k) return fail(FA_ERR_INVALID_ARG, "null pointer");
  if (B < 1 || H < 1 || total_q < 1 || total_k < 1 || max_q < 1 || max_k < 1 || D < 1)
    return fail(FA_ERR_INVALID_ARG, "sizes must be >= 1 (B=%d H=%d total_q=%d total_k=%d max_q=%d max_k=%d D=%d)",
                B, H, total_q, total_k, max_q, max_k, D);
  if (D != 32 && D != 64 && D != 128 && D != 256)
    return fail(FA_ERR_UNSUPPORTED, "head dim %d not in {32, 64, 128, 256}", D);
  if (causal != 0 && causal != 1) return fail(FA_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", causal);
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return fail(FA_ERR_INVALID_ARG, "q, k, v, o must be 16-byte aligned");
  if (!aligned(lse, 4) || !aligned(cu_q, 4) || !aligned(cu_k, 4))
    return fail(FA_ERR_INVALID_ARG, "lse and the cumulative lengths must be 4-byte aligned");
  if (!product_le(total_q, H, D, 1, kMaxElems) || !product_le(total_k, H, D, 1, kMaxElems))
    return fail(FA_ERR_INVALID_ARG, "tensor too large");
  // one sequence of one head is addressed with 32-bit byte offsets, which
  // also reach up to one query tile (256 rows) past its end
  if ((int64_t)(max_q + 256) * H * D * 2 >= kMaxSliceBytes || (int64_t)(max_k + 256) * H * D * 2 >= kMaxSliceBytes)
    return fail(FA_ERR_INVALID_ARG, "sequence too long: (max_seqlen + 256) * H * D * 2 must stay below 2 GiB");
  if ((int64_t)B * H > kMaxGrid) return fail(FA_ERR_INVALID_ARG, "grid too large");
  return FA_OK;
}

int validate_paged(const void* q, const void* kc, const void* vc, const int* tables, const int* seq_lens,
                   const void* o, const void* lse, int B, int H, int D, int num_blocks, int block_size,
                   int max_blocks, float scale, int num_splits, int* lbs) {
  if (!q || !kc || !vc || !tables || !seq_lens || !o || !lse) return fail(FA_ERR_INVALID_ARG, "null pointer");
  if (B < 1 || H < 1 || D < 1 || num_blocks < 1 || max_blocks < 1)
    return fail(FA_ERR_INVALID_ARG, "sizes must be >= 1 (B=%d H=%d D=%d num_blocks=%d max_blocks=%d)", B, H, D,
                num_blocks, max_blocks);
  if (D != 32 && D != 64 && D != 128 && D != 256)
    return fail(FA_ERR_UNSUPPORTED, "head dim %d not in {32, 64, 128, 256}", D);
  if (block_size < 1 || block_size > 1024 || (block_size & (block_size - 1)))
    return fail(FA_ERR_INVALID_ARG, "block_size %d is not a power of two in [1, 1024]", block_size);
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(FA_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (!aligned(q, 16) || !aligned(kc, 16) || !aligned(vc, 16) || !aligned(o, 16))
    return fail(FA_ERR_INVALID_ARG, "q, caches and o must be 16-byte aligned");
  if (!aligned(lse, 4) || !aligned(tables, 4) || !aligned(seq_lens, 4))
    return fail(FA_ERR_INVALID_ARG, "lse, block_tables and seq_lens must be 4-byte aligned");
  const int64_t max_ctx = (int64_t)max_blocks * block_size;
  if (max_ctx >= (int64_t(1) << 30)) return fail(FA_ERR_INVALID_ARG, "max_blocks * block_size too large");
  if (!product_le(num_blocks, H, block_size, D, kMaxElems)) return fail(FA_ERR_INVALID_ARG, "cache too large");
  if (!product_le(B, max_blocks, 1, 1, kMaxElems)) return fail(FA_ERR_INVALID_ARG, "block table too large");
  if (num_splits > max_ctx) return fail(FA_ERR_INVALID_ARG, "num_splits %d exceeds max context %lld", num_splits,
                                        (long long)max_ctx);
  if ((int64_t)B * H * (num_splits > 0 ? num_splits : 1) > kMaxGrid) return fail(FA_ERR_INVALID_ARG, "grid too large");
  int l = 0;
  while ((1 << l) < block_size) ++l;
  *lbs = l;
  return FA_OK;
}

int resolve_splits(int B, int H, int Sk, int num_splits, int* ns) {
  if (num_splits > 0) {
    *ns = num_splits;
    return FA_OK;
  }
  int cus = 0;
  int rc = device_cu_count(&cus);
  if (rc != FA_OK) return rc;
  *ns = fa_decode_auto_splits(B, H, Sk, cus);
  if (*ns < 1) return fail(FA_ERR_INVALID_ARG, "could not choose a split count");
  if ((int64_t)B * H * *ns > kMaxGrid) return fail(FA_ERR_INVALID_ARG, "grid too large");
  return FA_OK;
}

// How fa_fwd runs a call of these sizes on a device with `cus` CUs: the
// kernel, its geometry, its key split and the workspace bytes it needs.  A
// pure function of its arguments, so fa_fwd, fa_fwd_ws and the two query
// functions always agree.
enum FwdKind { kFwdTile = 0, kFwdSplitD = 1, kFwdDecode = 2 };
struct FwdPlan {
  int kind = kFwdTile;
  int nw = 4;     // wavefronts per workgroup of the tile kernel
  SplitPlan sp;   // even split of the tile kernel (sp.grid > 0: split)
  int ns = 1;     // key parts of Split-D, or decode partitions
  size_t ws = 0;  // workspace bytes (0: none)
};

int compute_plan_fwd(int B, int H, int Sq, int Sk, int D, bool causal, int cus, FwdPlan* out) {
  FwdPlan p;
  const int64_t BH = (int64_t)B * H;
  if (BH > kMaxGrid) return fail(FA_ERR_INVALID_ARG, "grid too large");
  if (Sq == 1 && !causal && D <= 256) {
    // a single query row attending to every key is a decode step: the
    // split-KV path ("FlashAttention-2 MMA", Architecture & Dispatch Flow,
    // seq_q == 1).  Causal single rows see key 0 only (top-left mask) and
    // stay on the tile kernel.
    p.kind = kFwdDecode;
    p.ns = fa_decode_auto_splits(B, H, Sk, cus);
    if (p.ns < 1) return fail(FA_ERR_INVALID_ARG, "could not choose a split count");
    if (BH * p.ns > kMaxGrid) return fail(FA_ERR_INVALID_ARG, "grid too large");
    p.ws = p.ns > 1 ? ws_bytes(BH, D, p.ns) : 0;
  } else if (D >= 512) {
    p.kind = kFwdSplitD;
    const int64_t nqt = (Sq + 31) / 32;
    if (nqt * BH > kMaxGrid) return fail(FA_ERR_INVALID_ARG, "grid too large");
    // runs of key tiles when the model says they pay (small or causal
    // grids), else equal key parts when the grid is too small
    if (D == 512) p.sp = plan_fwd_runs((int)nqt, (int)BH, 32, 32, D, Sq, Sk, causal, cus, kSplitDRunsModel);
    if (p.sp.grid > 0) {
      p.ns = 1;
      p.ws = runs_ws_bytes(32, D, p.sp);
    } else {
      p.ns = splitd_parts(nqt * BH, (Sk + 31) / 32, cus);
      p.ws = p.ns > 1 ? ws_bytes(BH * Sq, D, p.ns) : 0;
    }
  } else {
    // BN here is the planners' unit, 64 keys below D = 256 (their cost
    // models were fitted per 64-key tile), whatever width the kernel walks
    int BM = 128, BN = 64;
    if (D == 256) {
      BN = 32;
    } else if (D != 32 && BH * ((Sq + 255) / 256) >= cus) {
      // D = 64, 128: 256-row workgroups (one per CU) when that still gives
      // every CU one, else 128-row ones (two per CU) so small problems
      // spread over more CUs
      p.nw = 8;
      BM = 256;
    }
    const int64_t nqt = (Sq + BM - 1) / BM;
    if (nqt * BH > kMaxGrid) return fail(FA_ERR_INVALID_ARG, "grid too large");
    // small grids: the heaviest causal tiles, or too few tiles, leave CUs idle
    if (p.nw == 4)
      p.sp = D == 256 ? plan_fwd_runs((int)nqt, (int)BH, BM, BN, D, Sq, Sk, causal, cus, kRunsModel)
                      : plan_fwd_parts((int)nqt, (int)BH, BM, BN, D, Sq, Sk, causal, cus);
    if (p.sp.grid > 0)
      p.ws = D == 256 ? runs_ws_bytes(BM, D, p.sp) : ws_bytes(BH * (nqt - p.sp.ts) * BM, D, p.sp.ns);
  }
  *out = p;
  return FA_OK;
}

// Plans depend only on the sizes and the CU count, and the key-split
// planner simulates every candidate dispatch (hundreds of microseconds on
// the host for a 256-workgroup grid), so plans are cached: a direct-mapped
// table of recent sizes, shared by all threads under one mutex.
struct PlanKey {
  int B, H, Sq, Sk, D, causal, cus;
  bool operator==(const PlanKey& o) const {
    return B == o.B && H == o.H && Sq == o.Sq && Sk == o.Sk && D == o.D && causal == o.causal && cus == o.cus;
  }
};
struct PlanSlot {
  bool used = false;
  PlanKey key{};
  FwdPlan plan;
};
constexpr int kPlanSlots = 256;
std::mutex g_plan_mu;
PlanSlot g_plans[kPlanSlots];

int plan_fwd(int B, int H, int Sq, int Sk, int D, bool causal, int cus, FwdPlan* out) {
  const PlanKey key{B, H, Sq, Sk, D, causal ? 1 : 0, cus};
  uint64_t h = 1469598103934665603ull;  // FNV-1a over the seven sizes
  for (int x : {B, H, Sq, Sk, D, key.causal, cus}) {
    h ^= (uint32_t)x;
    h *= 1099511628211ull;
  }
  PlanSlot& slot = g_plans[h % kPlanSlots];
  {
    std::lock_guard<std::mutex> lock(g_plan_mu);
    if (slot.used && slot.key == key) {
      *out = slot.plan;
      return FA_OK;
    }
  }
  FwdPlan p;
  const int rc = compute_plan_fwd(B, H, Sq, Sk, D, causal, cus, &p);
  if (rc != FA_OK) return rc;  // invalid sizes are not cached: the error message is set again each call
  std::lock_guard<std::mutex> lock(g_plan_mu);
  slot.used = true;
  slot.key = key;
  slot.plan = p;
  *out = p;
  return FA_OK;
}

int run_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Sq, int Sk, int D,
            int causal, float scale, hipStream_t s, const FwdPlan& p, void* ws) {
  const int BH = B * H;
  if (p.kind == kFwdDecode) return run_decode(q, k, v, o, lse, BH, Sk, D, scale, s, p.ns, ws);
  switch (D) {
    case 32:
      return causal ? launch_fwd_d<32, true>(q, k, v, o, lse, BH, Sq, Sk, scale, s, p.nw, p.sp, ws)
                    : launch_fwd_d<32, false>(q, k, v, o, lse, BH, Sq, Sk, scale, s, p.nw, p.sp, ws);
    case 64:
      return causal ? launch_fwd_d<64, true>(q, k, v, o, lse, BH, Sq, Sk, scale, s, p.nw, p.sp, ws)
                    : launch_fwd_d<64, false>(q, k, v, o, lse, BH, Sq, Sk, scale, s, p.nw, p.sp, ws);
    case 128:
      return causal ? launch_fwd_d<128, true>(q, k, v, o, lse, BH, Sq, Sk, scale, s, p.nw, p.sp, ws)
                    : launch_fwd_d<128, false>(q, k, v, o, lse, BH, Sq, Sk, scale, s, p.nw, p.sp, ws);
    case 256:
      return causal ? launch_fwd_d<256, true>(q, k, v, o, lse, BH, Sq, Sk, scale, s, p.nw, p.sp, ws)
                    : launch_fwd_d<256, false>(q, k, v, o, lse, BH, Sq, Sk, scale, s, p.nw, p.sp, ws);
    case 512:
      return run_fwd_splitd<512>(q, k, v, o, lse, BH, Sq, Sk, causal, scale, s, p.ns, ws, p.sp);
    default:
      return run_fwd_splitd<1024>(q, k, v, o, lse, BH, Sq, Sk, causal, scale, s, p.ns, ws, p.sp);
  }
}

// Static scratch of fa_decode_splitkv_noalloc: the phase-one partials of a
// split decode, in a file-scope device array that every GPU the library
// runs on holds (its own copy) until the process ends.  Host code never
// passes the array's name to a kernel or a copy (on the host it is only a
// stand-in symbol): the device address of each GPU's copy is looked up once
// per device with hipGetSymbolAddress and kept in g_scratch.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's address of `scratch`, resolved on the first call on
// that device (with that device current).
int scratch_address(void** out) {
  int dev = 0;
  int rc = hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (rc != FA_OK) return rc;
  if (dev < 0 || dev >= kMaxDevices) return fail(FA_ERR_HIP, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    rc = hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "scratch symbol address");
    if (rc != FA_OK) return rc;
    if (!p) return fail(FA_ERR_HIP, "scratch symbol address is null");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return FA_OK;
}

// A workspace of `bytes` from the device's stream-ordered pool, usable by
// work queued on `s` from now on; release with hipFreeAsync on `s`.
int pool_alloc(size_t bytes, hipStream_t s, void** out) {
  hipMemPool_t pool = nullptr;
  int rc = workspace_pool(&pool);
  if (rc != FA_OK) return rc;
  return hip_check(hipMallocFromPoolAsync(out, bytes, pool, s), "workspace allocation");
}

// Row workspace of the backward: D and the LSE in log2 units, one fp32 each
// per query row.
size_t bwd_row_bytes(int64_t BH, int Sq) { return ((size_t)BH * Sq * 8 + 255) / 256 * 256; }

int validate_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                 void* dq, void* dk, void* dv, int B, int H, int Sq, int Sk, int D, int causal, float scale) {
  int rc = validate(q, k, v, o, lse, B, H, Sq, Sk, D, causal, scale);
  if (rc != FA_OK) return rc;
  if (!dout || !dq || !dk || !dv) return fail(FA_ERR_INVALID_ARG, "null gradient pointer");
  if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return fail(FA_ERR_INVALID_ARG, "dout, dq, dk, dv must be 16-byte aligned");
  if (D > 256) return fail(FA_ERR_UNSUPPORTED, "the backward pass supports head dims 32, 64, 128 and 256");
  if ((int64_t)B * H > kMaxGrid) return fail(FA_ERR_INVALID_ARG, "grid too large");
  return FA_OK;
}

// The backward's kernels on the per-row workspace `ws`.
int run_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
            void* dk, void* dv, int B, int H, int Sq, int Sk, int D, int causal, float scale, hipStream_t s, void* ws) {
  const int BH = B * H;
  float* dvec = static_cast<float*>(ws);
  switch (D) {
    case 32:
      return causal ? launch_bwd<32, true>(q, k, v, o, lse, dout, dq, dk, dv, BH, Sq, Sk, scale, s, dvec)
                    : launch_bwd<32, false>(q, k, v, o, lse, dout, dq, dk, dv, BH, Sq, Sk, scale, s, dvec);
    case 64:
      return causal ? launch_bwd<64, true>(q, k, v, o, lse, dout, dq, dk, dv, BH, Sq, Sk, scale, s, dvec)
                    : launch_bwd<64, false>(q, k, v, o, lse, dout, dq, dk, dv, BH, Sq, Sk, scale, s, dvec);
    case 128:
      return causal ? launch_bwd<128, true>(q, k, v, o, lse, dout, dq, dk, dv, BH, Sq, Sk, scale, s, dvec)
                    : launch_bwd<128, false>(q, k, v, o, lse, dout, dq, dk, dv, BH, Sq, Sk, scale, s, dvec);
    default:
      return causal ? launch_bwd<256, true>(q, k, v, o, lse, dout, dq, dk, dv, BH, Sq, Sk, scale, s, dvec)
                    : launch_bwd<256, false>(q, k, v, o, lse, dout, dq, dk, dv, BH, Sq, Sk, scale, s, dvec);
  }
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Sq, int Sk, int D,
           int causal, float scale, void* stream) {
  int rc = validate(q, k, v, o, lse, B, H, Sq, Sk, D, causal, scale);
  if (rc != FA_OK) return rc;
  int cus = 0;
  rc = device_cu_count(&cus);
  if (rc != FA_OK) return rc;
  FwdPlan p;
  rc = plan_fwd(B, H, Sq, Sk, D, causal != 0, cus, &p);
  if (rc != FA_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.ws == 0) return run_fwd(q, k, v, o, lse, B, H, Sq, Sk, D, causal, scale, s, p, nullptr);
  void* ws = nullptr;
  rc = pool_alloc(p.ws, s, &ws);
  if (rc != FA_OK) return rc;
  rc = run_fwd(q, k, v, o, lse, B, H, Sq, Sk, D, causal, scale, s, p, ws);
  const int frc = hip_check(hipFreeAsync(ws, s), "hipFreeAsync workspace");
  return rc != FA_OK ? rc : frc;
}

int fa_fwd_ws(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Sq, int Sk, int D,
              int causal, float scale, void* stream, void* workspace, size_t workspace_bytes) {
  int rc = validate(q, k, v, o, lse, B, H, Sq, Sk, D, causal, scale);
  if (rc != FA_OK) return rc;
  if (workspace && !aligned(workspace, 16)) return fail(FA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  int cus = 0;
  rc = device_cu_count(&cus);
  if (rc != FA_OK) return rc;
  FwdPlan p;
  rc = plan_fwd(B, H, Sq, Sk, D, causal != 0, cus, &p);
  if (rc != FA_OK) return rc;
  if (p.ws > 0 && (!workspace || workspace_bytes < p.ws))
    return fail(FA_ERR_INVALID_ARG, "workspace holds %zu bytes, %zu needed", workspace ? workspace_bytes : 0, p.ws);
  return run_fwd(q, k, v, o, lse, B, H, Sq, Sk, D, causal, scale, static_cast<hipStream_t>(stream), p,
                 p.ws ? workspace : nullptr);
}

size_t fa_fwd_workspace_bytes(int B, int H, int Sq, int Sk, int D, int causal, int num_cus) {
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1 || num_cus < 1 || (causal != 0 && causal != 1)) return 0;
  if (D != 32 && D != 64 && D != 128 && D != 256 && D != 512 && D != 1024) return 0;
  FwdPlan p;
  if (plan_fwd(B, H, Sq, Sk, D, causal != 0, num_cus, &p) != FA_OK) return 0;
  return p.ws;
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_seqlens_q,
                  const int* cu_seqlens_k, int B, int H, int total_q, int total_k, int max_seqlen_q,
                  int max_seqlen_k, int D, int causal, float scale, void* stream) {
  int rc = validate_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, H, total_q, total_k, max_seqlen_q,
                           max_seqlen_k, D, causal, scale);
  if (rc != FA_OK) return rc;
  fa::VarlenArgs va = {cu_seqlens_q, cu_seqlens_k, H, total_q, total_k, max_seqlen_q, max_seqlen_k};
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (D) {
    case 32:
      return causal ? launch_fwd_varlen_d<32, true>(q, k, v, o, lse, va, B, scale, s)
                    : launch_fwd_varlen_d<32, false>(q, k, v, o, lse, va, B, scale, s);
    case 64:
      return causal ? launch_fwd_varlen_d<64, true>(q, k, v, o, lse, va, B, scale, s)
                    : launch_fwd_varlen_d<64, false>(q, k, v, o, lse, va, B, scale, s);
    case 128:
      return causal ? launch_fwd_varlen_d<128, true>(q, k, v, o, lse, va, B, scale, s)
                    : launch_fwd_varlen_d<128, false>(q, k, v, o, lse, va, B, scale, s);
    default:
      return causal ? launch_fwd_varlen_d<256, true>(q, k, v, o, lse, va, B, scale, s)
                    : launch_fwd_varlen_d<256, false>(q, k, v, o, lse, va, B, scale, s);
  }
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
           void* dq, void* dk, void* dv, int B, int H, int Sq, int Sk, int D, int causal, float scale,
           void* stream) {
  int rc = validate_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, Sq, Sk, D, causal, scale);
  if (rc != FA_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipMemPool_t pool = nullptr;
  rc = workspace_pool(&pool);
  if (rc != FA_OK) return rc;
  void* ws = nullptr;
  rc = hip_check(hipMallocFromPoolAsync(&ws, bwd_row_bytes((int64_t)B * H, Sq), pool, s), "workspace allocation");
  if (rc != FA_OK) return rc;
  rc = run_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, Sq, Sk, D, causal, scale, s, ws);
  const int frc = hip_check(hipFreeAsync(ws, s), "hipFreeAsync workspace");
  return rc != FA_OK ? rc : frc;
}

size_t fa_bwd_workspace_bytes(int B, int H, int Sq, int D) {
  if (B < 1 || H < 1 || Sq < 1) return 0;
  if (D != 32 && D != 64 && D != 128 && D != 256) return 0;
  return bwd_row_bytes((int64_t)B * H, Sq);
}

int fa_bwd_ws(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
              void* dq, void* dk, void* dv, int B, int H, int Sq, int Sk, int D, int causal, float scale,
              void* stream, void* workspace, size_t workspace_bytes) {
  int rc = validate_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, Sq, Sk, D, causal, scale);
  if (rc != FA_OK) return rc;
  if (!workspace || !aligned(workspace, 16)) return fail(FA_ERR_INVALID_ARG, "workspace must be non-null and 16-byte aligned");
  const size_t need = bwd_row_bytes((int64_t)B * H, Sq);
  if (workspace_bytes < need)
    return fail(FA_ERR_INVALID_ARG, "workspace holds %zu bytes, %zu needed", workspace_bytes, need);
  return run_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, Sq, Sk, D, causal, scale, static_cast<hipStream_t>(stream),
                 workspace);
}

int fa_fwd_key_splits(int B, int H, int Sq, int Sk, int D, int causal, int num_cus) {
  if (B < 1 || H < 1 || Sq < 1 || Sk < 1 || num_cus < 1 || (causal != 0 && causal != 1)) return 0;
  if (D != 32 && D != 64 && D != 128 && D != 256 && D != 512 && D != 1024) return 0;
  FwdPlan p;
  if (plan_fwd(B, H, Sq, Sk, D, causal != 0, num_cus, &p) != FA_OK) return 0;
  return (p.kind == kFwdTile || p.sp.grid > 0) ? p.sp.max_parts : p.ns;
}

int fa_decode_auto_splits(int B, int H, int Sk, int num_cus) {
  if (B < 1 || H < 1 || Sk < 1 || num_cus < 1) return 0;
  const int64_t bh = (int64_t)B * H;
  // one 1024-thread workgroup per slice already gives every CU two of them
  // (32 wavefronts): a single partition, merged in LDS, with no workspace
  if (bh >= (int64_t)2 * num_cus) return 1;
  const int64_t target = (int64_t)8 * num_cus;
  int64_t ns = 1;
  while (bh * ns < target && ns < Sk) ns *= 2;
  while (ns > 1 && (Sk + ns - 1) / ns < 256) ns /= 2;
  if (ns > Sk) ns = Sk;
  return (int)ns;
}

size_t fa_decode_workspace_bytes(int B, int H, int D, int num_splits) {
  if (B < 1 || H < 1 || D < 1 || num_splits < 1) return 0;
  return ws_bytes((int64_t)B * H, D, num_splits);
}

int fa_decode_splitkv_ws(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Sq,
                         int Sk, int D, int causal, float scale, void* stream, int num_splits, void* workspace,
                         size_t workspace_bytes) {
  int rc = validate_decode(q, k, v, o, lse, B, H, Sq, Sk, D, causal, scale, num_splits);
  if (rc != FA_OK) return rc;
  if (!workspace) return fail(FA_ERR_INVALID_ARG, "null workspace");
  if (!aligned(workspace, 16)) return fail(FA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  int ns = 0;
  rc = resolve_splits(B, H, Sk, num_splits, &ns);
  if (rc != FA_OK) return rc;
  const size_t need = ws_bytes((int64_t)B * H, D, ns);
  if (workspace_bytes < need)
    return fail(FA_ERR_INVALID_ARG, "workspace holds %zu bytes, %zu needed", workspace_bytes, need);
  return run_decode(q, k, v, o, lse, B * H, Sk, D, scale, static_cast<hipStream_t>(stream), ns, workspace);
}

int fa_decode_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Sq,
                      int Sk, int D, int causal, float scale, void* stream, int num_splits) {
  int rc = validate_decode(q, k, v, o, lse, B, H, Sq, Sk, D, causal, scale, num_splits);
  if (rc != FA_OK) return rc;
  int ns = 0;
  rc = resolve_splits(B, H, Sk, num_splits, &ns);
  if (rc != FA_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (ns == 1) return run_decode(q, k, v, o, lse, B * H, Sk, D, scale, s, 1, nullptr);  // no workspace
  hipMemPool_t pool = nullptr;
  rc = workspace_pool(&pool);
  if (rc != FA_OK) return rc;
  void* ws = nullptr;
  rc = hip_check(hipMallocFromPoolAsync(&ws, ws_bytes((int64_t)B * H, D, ns), pool, s), "workspace allocation");
  if (rc != FA_OK) return rc;
  rc = run_decode(q, k, v, o, lse, B * H, Sk, D, scale, s, ns, ws);
  const int frc = hip_check(hipFreeAsync(ws, s), "hipFreeAsync workspace");
  return rc != FA_OK ? rc : frc;
}

int fa_decode_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Sq,
                              int Sk, int D, int causal, float scale, void* stream, int num_splits) {
  int rc = validate_decode(q, k, v, o, lse, B, H, Sq, Sk, D, causal, scale, num_splits);
  if (rc != FA_OK) return rc;
  int ns = 0;
  rc = resolve_splits(B, H, Sk, num_splits, &ns);
  if (rc != FA_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (ns == 1) return run_decode(q, k, v, o, lse, B * H, Sk, D, scale, s, 1, nullptr);  // no scratch
  const size_t need = ws_bytes((int64_t)B * H, D, ns);
  if (need > kScratchBytes)
    return fail(FA_ERR_INVALID_ARG, "%zu bytes of partials exceed the %zu-byte static scratch (B*H*ns*(D+1)*4)",
                need, kScratchBytes);
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc != FA_OK) return rc;
  return run_decode(q, k, v, o, lse, B * H, Sk, D, scale, s, ns, ws);
}

int fa_decode_paged(const void* q, const void* k_cache, const void* v_cache, const int* block_tables,
                    const int* seq_lens, void* o, float* lse, int B, int H, int D, int num_blocks, int block_size,
                    int max_blocks, float scale, void* stream, int num_splits) {
  int lbs = 0;
  int rc = validate_paged(q, k_cache, v_cache, block_tables, seq_lens, o, lse, B, H, D, num_blocks, block_size,
                          max_blocks, scale, num_splits, &lbs);
  if (rc != FA_OK) return rc;
  int ns = 0;
  rc = resolve_splits(B, H, max_blocks * block_size, num_splits, &ns);
  if (rc != FA_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (ns > 1) {  // a single partition needs no workspace
    hipMemPool_t pool = nullptr;
    rc = workspace_pool(&pool);
    if (rc != FA_OK) return rc;
    rc = hip_check(hipMallocFromPoolAsync(&ws, ws_bytes((int64_t)B * H, D, ns), pool, s), "workspace allocation");
    if (rc != FA_OK) return rc;
  }
  float* ws_o = static_cast<float*>(ws);
  float* ws_lse = ws ? ws_o + (size_t)B * H * ns * D : nullptr;
  switch (D) {
    case 32:
      rc = launch_decode_paged<32>(q, k_cache, v_cache, block_tables, seq_lens, o, lse, B, H, num_blocks, lbs,
                                   max_blocks, scale, s, ns, ws_o, ws_lse);
      break;
    case 64:
      rc = launch_decode_paged<64>(q, k_cache, v_cache, block_tables, seq_lens, o, lse, B, H, num_blocks, lbs,
                                   max_blocks, scale, s, ns, ws_o, ws_lse);
      break;
    case 128:
      rc = launch_decode_paged<128>(q, k_cache, v_cache, block_tables, seq_lens, o, lse, B, H, num_blocks, lbs,
                                    max_blocks, scale, s, ns, ws_o, ws_lse);
      break;
    default:
      rc = launch_decode_paged<256>(q, k_cache, v_cache, block_tables, seq_lens, o, lse, B, H, num_blocks, lbs,
                                    max_blocks, scale, s, ns, ws_o, ws_lse);
      break;
  }
  if (!ws) return rc;
  const int frc = hip_check(hipFreeAsync(ws, s), "hipFreeAsync workspace");
  return rc != FA_OK ? rc : frc;
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported head dimension";
    case FA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* fa_last_error(void) { return g_err; }

}  // extern "C"
