// Host-side check of the LDS layouts the attention kernels use (built for the
// CPU tests; no GPU code runs).  For each layout and row width C (16-byte
// chunks per row) it enumerates a tile and checks:
//   * the map (row, chunk) -> byte offset is a bijection onto the tile and
//     its inverse (used to place the direct HBM -> LDS copies) undoes it;
//   * the access groups the kernels issue land on 16 distinct 16-byte slots
//     of a 256-byte line (the 64 four-byte banks): 16 consecutive rows of one
//     chunk column (ds_read_b128 of an MFMA operand), and, for the layouts
//     read transposed, 4 consecutive rows x 4 consecutive chunks
//     (ds_read_b64_tr_b16, 8 bytes per lane over 32 lanes).
// swizzle_check returns the number of failures and describes the first.
#include <cstdio>
#include <cstring>

#include "fa_bwd_kernel.hpp"
#include "fa_device.hpp"

namespace {

char g_msg[256];
int g_fail = 0;

void fail(const char* what, int C, int r, int c) {
  if (g_fail++ == 0) snprintf(g_msg, sizeof(g_msg), "%s C=%d at row %d chunk %d", what, C, r, c);
}

template <int C, class F, class Finv>
void check_layout(const char* name, int rows, F fwd, Finv inv, bool row_reads, bool tr_reads) {
  const int slots = rows * C;
  static int seen[1 << 16];
  if (slots > (1 << 16)) return fail(name, C, -1, -1);
  memset(seen, 0, sizeof(int) * slots);
  for (int r = 0; r < rows; ++r)
    for (int c = 0; c < C; ++c) {
      const unsigned off = fwd(r, c);
      if (off % 16 || off / 16 >= (unsigned)slots || seen[off / 16]++) return fail(name, C, r, c);
      int r2 = -1, c2 = -1;
      inv((int)(off / 256), (int)((off / 16) % 16), r2, c2);
      if (r2 != r || c2 != c) return fail(name, C, r, c);
    }
  if (row_reads)
    for (int r0 = 0; r0 + 16 <= rows; r0 += 16)
      for (int c = 0; c < C; ++c) {
        int mask = 0;
        for (int i = 0; i < 16; ++i) mask |= 1 << ((fwd(r0 + i, c) / 16) % 16);
        if (mask != 0xffff) return fail(name, C, r0, c);
      }
  if (tr_reads && C >= 4)
    for (int r0 = 0; r0 + 4 <= rows; r0 += 4)
      for (int c0 = 0; c0 + 4 <= C; c0 += 4) {
        int mask = 0;
        for (int i = 0; i < 4; ++i)
          for (int j = 0; j < 4; ++j) mask |= 1 << ((fwd(r0 + i, c0 + j) / 16) % 16);
        if (mask != 0xffff) return fail(name, C, r0, c0);
      }
}

template <int C>
void check_width(int rows) {
  // K tiles (row reads) and output staging: swz
  check_layout<C>("swz", rows, [](int r, int c) { return fa::swz<C>(r, c); },
                  [](int l, int s, int& r, int& c) { fa::swz_inv<C>(l, s, r, c); }, true, false);
  // V tiles (transposed reads): vswz
  check_layout<C>("vswz", rows, [](int r, int c) { return fa::vswz<C>(r, c); },
                  [](int l, int s, int& r, int& c) { fa::vswz_inv<C>(l, s, r, c); }, false, true);
}

template <int C>
void check_bwd(int rows) {
  // backward tiles read both ways: bswz
  check_layout<C>("bswz", rows, [](int r, int c) { return fa::bswz<C>(r, c); },
                  [](int l, int s, int& r, int& c) { fa::bswz_inv<C>(l, s, r, c); }, true, true);
}

}  // namespace

extern "C" int swizzle_check(char* msg, int n) {
  g_fail = 0;
  g_msg[0] = 0;
  check_width<4>(64);
  check_width<8>(64);
  check_width<16>(64);
  check_width<32>(64);
  check_width<64>(32);
  check_width<128>(32);
  check_bwd<4>(64);
  check_bwd<8>(64);
  check_bwd<16>(64);
  check_bwd<32>(64);
  if (msg && n > 0) snprintf(msg, (size_t)n, "%s", g_msg);
  return g_fail;
}
