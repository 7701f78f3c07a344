// Host enumeration of the LDS byte addresses every lane of every wave
// touches in each LDS instruction of the transpose kernels, for each built
// tile shape.  One line per instruction:
//   <kernel> <phase> <width bytes> <is_write> <addr lane 0> ... <addr lane 63>
// The lane maps and layouts are the kernels' own (xpose_lanes.h); the bank
// analysis of these addresses is done by the caller.
#include <stdio.h>

#include <set>
#include <string>

#include "../../lds_tiled_matrix_amd/csrc/xpose_lanes.h"

using namespace xpose;

static const char *layout_name(int l) {
  return l == kUnpadded ? "unpadded" : l == kPad1 ? "pad1" : "swizzle";
}

// Identical instructions (same kernel, phase and addresses) print once.
static std::set<std::string> seen;

static void emit(const char *kernel, const char *phase, int width, int wr,
                 const int *addr) {
  std::string line = std::string(kernel) + " " + phase + " " +
                     std::to_string(width) + " " + std::to_string(wr);
  for (int l = 0; l < 64; ++l) line += " " + std::to_string(addr[l]);
  if (seen.insert(line).second) printf("%s\n", line.c_str());
}

// Packed-register tiles (xpose_tile_kernel): vector_to_lds and
// lds_to_global of every wave.
template <int S, int TR, int TC, int NT, int L>
static void tile() {
  using T = Tile<S, TR, TC, NT, L, kCacheDefault>;
  char name[96];
  snprintf(name, sizeof name, "tile/s%d/%dx%d/%d/%s", S, TR, TC, NT,
           layout_name(L));
  constexpr bool LSPLIT = !T::WIDE_WRITE;
  int a[64];
  for (int wave = 0; wave < T::NW; ++wave) {
    for (int it = 0; it < T::LIT; ++it) {
      if (T::WIDE_WRITE) {
        for (int g = 0; g < T::V / T::UPV; ++g) {
          for (int lane = 0; lane < 64; ++lane) {
            int p, ch;
            lane_map<T::NCI, LSPLIT>(it * T::NW + wave, lane, p, ch);
            a[lane] = T::lds_index(p, ch * T::V + g * T::UPV) * T::UB;
          }
          emit(name, "write", 16, 1, a);
        }
      } else {
        for (int e = 0; e < T::V; ++e) {
          for (int lane = 0; lane < 64; ++lane) {
            int p, ch;
            lane_map<T::NCI, LSPLIT>(it * T::NW + wave, lane, p, ch);
            a[lane] = T::lds_index(p, ch * T::V + e) * T::UB;
          }
          emit(name, "write", T::UB, 1, a);
        }
      }
    }
    for (int it = 0; it < T::SIT; ++it)
      for (int k = 0; k < T::UPV; ++k) {
        for (int lane = 0; lane < 64; ++lane) {
          int c, q;
          lane_map<T::NCO, true>(it * T::NW + wave, lane, c, q);
          a[lane] = T::lds_index(q * T::UPV + k, c) * T::UB;
        }
        emit(name, "read", T::UB, 0, a);
      }
  }
}

template <int S, int TR, int TC, int NT>
static void tiles() {
  tile<S, TR, TC, NT, kUnpadded>();
  tile<S, TR, TC, NT, kPad1>();
  tile<S, TR, TC, NT, kSwizzle>();
}

// Line-aligned output tiles: the phase-1 writes of the underlying swizzled
// tile of TR + 128 / S rows, and the shifted gathers for the segment starts
// of every output pitch (mod one line) at three base addresses: output row
// j starts d_j = ((base + j * ld_out * S) mod 128) / S elements past a line.
template <int S, int TR, int TC, int NT>
static void shift() {
  using T = ShiftTile<S, TR, TC, NT, kCacheDefault>;
  using B = typename T::Base;
  char name[96];
  snprintf(name, sizeof name, "shift/s%d/%dx%d/%d/swizzle", S, TR, TC, NT);
  constexpr int UB = (int)sizeof(typename B::U);
  int a[64];
  for (int wave = 0; wave < B::NW; ++wave)
    for (int it = 0; it < B::LIT; ++it)
      for (int g = 0; g < B::V / B::UPV; ++g) {
        for (int lane = 0; lane < 64; ++lane) {
          int p, ch;
          lane_map<B::NCI, false>(it * B::NW + wave, lane, p, ch);
          a[lane] = B::lds_index(p, ch * B::V + g * B::UPV) * UB;
        }
        emit(name, "write", 16, 1, a);
      }
  for (int wave = 0; wave < T::NW; ++wave)
    for (int ld = 0; ld < 128 / S; ++ld)
      for (int base : {0, (5 * S) % 128, 128 - S})
        for (int it = 0; it < T::SIT; ++it)
          for (int k = 0; k < T::GATHER_UNITS; ++k) {
            for (int lane = 0; lane < 64; ++lane) {
              int c, q;
              lane_map<T::NCO, true>(it * T::NW + wave, lane, c, q);
              const int d = ((base + c * ld * S) & 127) / S;
              int ur, shift;
              T::gather_rows(T::HALO - d + T::V * q, ur, shift);
              a[lane] = T::unit_index(ur + k, c) * UB;
            }
            emit(name, "read", UB, 0, a);
          }
}

// Transpose-read tiles: chunk writes and the transpose reads.
template <int S, int TR, int TC, int NT, bool D>
static void tr() {
  using T = TrTile<S, TR, TC, NT, kCacheDefault, D>;
  char name[96];
  snprintf(name, sizeof name, "tr/s%d/%dx%d/%d/%s", S, TR, TC, NT,
           D ? "direct" : "swizzle");
  constexpr int RPT = 64 / T::NCL;
  int a[64];
  for (int wave = 0; wave < T::NW; ++wave) {
    if (!D)
      for (int it = 0; it < T::LIT; ++it) {
        for (int lane = 0; lane < 64; ++lane) {
          const int row = (it * T::NW + wave) * RPT + lane / T::NCL;
          int off;
          bool swap;
          T::chunk_at(row, lane % T::NCL, off, swap);
          a[lane] = off;
        }
        emit(name, "write", 16, 1, a);
      }
    for (int it = 0; it < T::SIT; ++it)
      for (int k = 0; k < 2; ++k) {
        for (int lane = 0; lane < 64; ++lane) {
          const int q = lane >> 4, i = lane & 15;
          const int gt = (it * T::NW + wave) * 4 + q;
          const int rb = gt % T::NRB, cu = gt / T::NRB;
          const int row = rb * 32 + (i % T::NQ) * T::V + k * T::HR + i / T::NQ;
          a[lane] = T::unit_at(row, cu);
        }
        emit(name, "read", 8, 0, a);
      }
  }
}

int main() {
  // 4-byte elements
  tiles<4, 32, 32, 256>(); tiles<4, 32, 32, 128>(); tiles<4, 32, 32, 64>();
  tiles<4, 32, 64, 128>(); tiles<4, 64, 32, 128>(); tiles<4, 64, 64, 256>();
  tiles<4, 64, 128, 256>(); tiles<4, 128, 64, 256>();
  tiles<4, 128, 128, 256>(); tiles<4, 32, 128, 256>();
  tiles<4, 128, 32, 256>(); tiles<4, 256, 128, 256>();
  shift<4, 64, 64, 256>(); shift<4, 128, 64, 256>(); shift<4, 256, 64, 256>();
  shift<4, 128, 32, 256>(); shift<4, 64, 32, 128>();
  shift<4, 64, 128, 256>(); shift<4, 128, 128, 256>(); shift<4, 256, 128, 256>();
  // 2-byte elements
  tiles<2, 32, 32, 64>(); tiles<2, 32, 64, 128>(); tiles<2, 64, 32, 128>();
  tiles<2, 64, 64, 128>(); tiles<2, 64, 64, 256>(); tiles<2, 128, 128, 256>();
  tiles<2, 256, 256, 256>(); tiles<2, 256, 256, 512>();
  tiles<2, 64, 128, 256>(); tiles<2, 128, 64, 256>();
  shift<2, 64, 64, 256>(); shift<2, 128, 64, 256>(); shift<2, 256, 64, 256>();
  tr<2, 64, 64, 256, false>(); tr<2, 128, 64, 256, false>();
  tr<2, 64, 128, 256, false>(); tr<2, 128, 128, 256, false>();
  tr<2, 64, 32, 128, false>(); tr<2, 64, 64, 256, true>();
  tr<2, 128, 64, 256, true>(); tr<2, 128, 128, 256, true>();
  // 1-byte elements
  tiles<1, 64, 64, 64>(); tiles<1, 64, 128, 128>(); tiles<1, 128, 64, 128>();
  tiles<1, 128, 128, 256>();
  tr<1, 128, 128, 256, false>(); tr<1, 64, 128, 128, false>();
  tr<1, 128, 64, 128, false>(); tr<1, 128, 256, 256, false>();
  tr<1, 128, 128, 256, true>();
  // 8-byte elements
  tiles<8, 32, 32, 128>(); tiles<8, 32, 32, 256>();
  tiles<8, 64, 64, 256>(); tiles<8, 128, 128, 256>();
  shift<8, 32, 32, 256>(); shift<8, 64, 32, 256>(); shift<8, 64, 64, 256>();
  return 0;
}
