// Host enumeration of the SGEMM kernel's LDS accesses and block order, from
// the kernel's own geometry (lds_tiled_matrix_amd/csrc/sgemm_lanes.h).
// Prints one line per LDS instruction of each built (k step, As layout):
//   lds <kernel> <phase> <width bytes> <is_write> <addr lane 0> ... <lane 63>
// and one line per self-check:
//   check <what> ok|FAIL <detail>
// The bank analysis of the addresses is done by the caller.
#include <stdio.h>

#include <set>
#include <string>
#include <vector>

#include "../../lds_tiled_matrix_amd/csrc/sgemm_lanes.h"

using namespace xpose;

static std::set<std::string> seen;

static void emit(const std::string &kernel, const char *phase, int width,
                 int wr, const int *addr) {
  std::string line = "lds " + kernel + " " + phase + " " +
                     std::to_string(width) + " " + std::to_string(wr);
  for (int l = 0; l < 64; ++l) line += " " + std::to_string(addr[l]);
  if (seen.insert(line).second) printf("%s\n", line.c_str());
}

static void check(const std::string &what, bool ok, const char *detail = "") {
  printf("check %s %s %s\n", what.c_str(), ok ? "ok" : "FAIL", detail);
}

template <int BK, int L, int BM = 128>
static void kernel() {
  using T = SgemmTile<BK, L, BM>;
  const char *lname = L == kAsUnpadded ? "unpadded"
                      : L == kAsPadded ? "padded" : "swizzle";
  const std::string name = "sgemm/bk" + std::to_string(BK) + "/" + lname +
                           (BM == 128 ? "" : "/m" + std::to_string(BM));
  int a[64];
  // Every (l, i) of As written exactly once, inside the array.
  std::vector<int> hits(T::AS_FLOATS, 0);
  bool in_bounds = true;
  for (int w = 0; w < T::NT / 64; ++w)
    for (int p = 0; p < T::A_PASSES; ++p)
      for (int e = 0; e < 4; ++e) {
        for (int q = 0; q < 64; ++q) {
          const int t = 64 * w + q;
          const int idx = T::as_index(T::a_col(t, p) + e, T::a_row(t, p));
          in_bounds &= idx >= 0 && idx < T::AS_FLOATS;
          if (idx >= 0 && idx < T::AS_FLOATS) ++hits[idx];
          a[q] = 4 * idx;
        }
        emit(name, "a_store", 4, 1, a);
      }
  int once = 0, twice = 0;
  for (int h : hits) once += h == 1, twice += h > 1;
  check(name + "/a_store_covers", in_bounds && once == BK * T::BM && !twice);
  std::vector<int> bhits(T::BS_FLOATS, 0);
  in_bounds = true;
  for (int w = 0; w < T::NT / 64; ++w)
    for (int p = 0; p < T::B_PASSES; ++p) {
      for (int q = 0; q < 64; ++q) {
        const int t = 64 * w + q;
        const int idx = T::bs_index(T::b_row(t, p), T::b_col(t));
        in_bounds &= idx >= 0 && idx + 3 < T::BS_FLOATS && idx % 4 == 0;
        for (int e = 0; e < 4 && idx + e < T::BS_FLOATS; ++e) ++bhits[idx + e];
        a[q] = 4 * idx;
      }
      emit(name, "b_store", 16, 1, a);
    }
  once = twice = 0;
  for (int h : bhits) once += h == 1, twice += h > 1;
  check(name + "/b_store_covers", in_bounds && once == T::BS_FLOATS && !twice);
  // Matrix-core operand reads: every (l, i) the product needs is where the
  // store put it, and reads stay inside the arrays.
  in_bounds = true;
  for (int w = 0; w < T::NT / 64; ++w)
    for (int kk = 0; kk < BK; kk += 2)
      for (int x = 0; x < 2; ++x) {
        for (int q = 0; q < 64; ++q) {
          const int idx =
              T::as_index(kk + q / 32, T::wave_row(w) + 32 * x + q % 32);
          in_bounds &= idx >= 0 && idx < T::AS_FLOATS;
          a[q] = 4 * idx;
        }
        emit(name, "a_read", 4, 0, a);
        for (int q = 0; q < 64; ++q) {
          const int idx =
              T::bs_index(kk + q / 32, T::wave_col(w) + 32 * x + q % 32);
          in_bounds &= idx >= 0 && idx < T::BS_FLOATS;
          a[q] = 4 * idx;
        }
        emit(name, "b_read", 4, 0, a);
      }
  check(name + "/reads_in_bounds", in_bounds);
  check(name + "/lds_bytes", T::LDS_BYTES == 4 * BK * (T::AS_STRIDE + 128));
  // The whole-block epilogue addresses C element (row, col) of the block as
  // one per-lane offset (row acc_row(q, 0) of the wave's block) plus a
  // per-register row offset (acc_row(0, r)): the sum must be the lane's own
  // accumulator row, and every element must fall inside the descriptor's
  // extent, (BM - 1) * ldc + BN floats, for the largest pitch it takes.
  bool sum_ok = true, extent_ok = true;
  const int64_t ldc = ((int64_t)1 << 29) / T::BM;
  const int64_t records = ((T::BM - 1) * ldc + T::BN) * 4;
  for (int w = 0; w < T::NT / 64; ++w)
    for (int q = 0; q < 64; ++q)
      for (int x = 0; x < 2; ++x)
        for (int y = 0; y < 2; ++y)
          for (int r = 0; r < 16; ++r) {
            sum_ok &= T::acc_row(q, r) == T::acc_row(q, 0) + T::acc_row(0, r);
            const int64_t lane_off =
                ((T::wave_row(w) + T::acc_row(q, 0)) * ldc + T::wave_col(w) +
                 q % 32) * 4;
            const int64_t off = lane_off + 128 * y +
                                (32 * x + T::acc_row(0, r)) * ldc * 4;
            extent_ok &= lane_off < INT32_MAX && off >= 0 && off + 4 <= records &&
                         records <= INT32_MAX;
          }
  check(name + "/epilogue_rows", sum_ok);
  check(name + "/epilogue_extent", extent_ok);
}

// The block order must be a bijection onto the tiles_m x tiles_n blocks.
static void block_order(uint32_t tm, uint32_t tn, uint32_t g, int remap) {
  std::vector<int> hit(tm * tn, 0);
  bool ok = true;
  for (uint32_t b = 0; b < tm * tn; ++b) {
    uint32_t bm, bn;
    sgemm_block(b, tm, tn, g, remap, bm, bn);
    if (bm >= tm || bn >= tn) {
      ok = false;
      continue;
    }
    ++hit[bm * tn + bn];
  }
  for (int h : hit) ok &= h == 1;
  char what[96];
  snprintf(what, sizeof what, "block_order/%ux%u/g%u/r%d", tm, tn, g, remap);
  check(what, ok);
}

// uniform_bits with an identity broadcast of the builtin's int(int) shape
// must give back every address, low halves with bit 31 set included.
static void uniform_addresses() {
  const uint64_t vals[] = {0x00007f12c0001000ull, 0x00007f1240001000ull,
                           0x0000000080000000ull, 0x00007fffffffffffull,
                           0xffffffff00000000ull, 0x0000000000000010ull};
  bool ok = true;
  for (uint64_t v : vals)
    ok &= uniform_bits(v, [](int x) { return x; }) == v;
  check("uniform_bits/identity", ok);
}

int main() {
  uniform_addresses();
  kernel<8, kAsUnpadded>(); kernel<8, kAsPadded>(); kernel<8, kAsSwizzle>();
  kernel<16, kAsUnpadded>(); kernel<16, kAsPadded>(); kernel<16, kAsSwizzle>();
  kernel<32, kAsUnpadded>(); kernel<32, kAsPadded>(); kernel<32, kAsSwizzle>();
  kernel<64, kAsUnpadded>(); kernel<64, kAsPadded>(); kernel<64, kAsSwizzle>();
  kernel<16, kAsUnpadded, 256>(); kernel<16, kAsPadded, 256>();
  kernel<16, kAsSwizzle, 256>(); kernel<32, kAsUnpadded, 256>();
  kernel<32, kAsPadded, 256>(); kernel<32, kAsSwizzle, 256>();
  kernel<16, kAsUnpadded, 64>(); kernel<16, kAsPadded, 64>();
  kernel<16, kAsSwizzle, 64>();
  const uint32_t dims[] = {1, 2, 3, 7, 8, 9, 32, 33};
  for (uint32_t tm : dims)
    for (uint32_t tn : dims)
      for (uint32_t g : {1u, 2u, 8u})
        for (int r = 0; r < 2; ++r)
          if (g <= tm) block_order(tm, tn, g, r);
  return 0;
}
