// LDS tile geometry and lane maps of the transpose kernels: where each lane
// puts and finds each 16-byte chunk, unit or element in LDS.  Host and
// device code: the kernels use it, and a host program enumerates the LDS
// addresses every instruction touches so the bank behaviour of each built
// tile shape can be checked without a GPU.  Internal, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "xpose_kernels.h"

#define XPOSE_HD __host__ __device__

namespace xpose {

// Partial 16-byte vectors at a matrix edge: the first n bytes (0 <= n < 16)
// of a vector move with at most four accesses of 8, 4, 2 and 1 bytes,
// largest first, so each piece sits at a multiple of its own size and none
// straddles the vector's two 8-byte halves (lo = bytes 0-7, hi = 8-15).
// Bytes past n are neither read nor written; loaded ones come back zero.
// Addresses need no alignment (gfx950 serves unaligned global accesses).
typedef uint64_t u64_any __attribute__((aligned(1)));
typedef uint32_t u32_any __attribute__((aligned(1)));
typedef uint16_t u16_any __attribute__((aligned(1)));

XPOSE_HD inline void put_piece(uint64_t &lo, uint64_t &hi, int off,
                               uint64_t v) {
  if (off >= 8) hi |= v << (8 * (off - 8));
  else lo |= v << (8 * off);
}
XPOSE_HD inline uint64_t get_piece(uint64_t lo, uint64_t hi, int off) {
  return off >= 8 ? hi >> (8 * (off - 8)) : lo >> (8 * off);
}

XPOSE_HD inline void load_head(const char *p, int n, uint64_t &lo,
                               uint64_t &hi) {
  lo = hi = 0;
  int off = 0;
  if (n & 8) {
    lo = *reinterpret_cast<const u64_any *>(p);
    off = 8;
  }
  if (n & 4) {
    put_piece(lo, hi, off, *reinterpret_cast<const u32_any *>(p + off));
    off += 4;
  }
  if (n & 2) {
    put_piece(lo, hi, off, *reinterpret_cast<const u16_any *>(p + off));
    off += 2;
  }
  if (n & 1) put_piece(lo, hi, off, (uint8_t)p[off]);
}

XPOSE_HD inline void store_head(char *p, int n, uint64_t lo, uint64_t hi) {
  int off = 0;
  if (n & 8) {
    *reinterpret_cast<u64_any *>(p) = lo;
    off = 8;
  }
  if (n & 4) {
    *reinterpret_cast<u32_any *>(p + off) = (uint32_t)get_piece(lo, hi, off);
    off += 4;
  }
  if (n & 2) {
    *reinterpret_cast<u16_any *>(p + off) = (uint16_t)get_piece(lo, hi, off);
    off += 2;
  }
  if (n & 1) p[off] = (char)get_piece(lo, hi, off);
}

// Edge tiles on the 16-byte path load every chunk with one unconditional
// 16-byte access (no branch, so all of a lane's loads go out before the
// first wait), which needs an in-bounds address for every chunk.  The tile
// holds at least one whole chunk of each of its rows (16 bytes from the
// tile's first element on), and `have` is the number of row elements from
// the chunk's first to the row's end (<= 0 past the end).
//  * have >= V (whole chunk): the chunk itself;
//  * 0 < have < V (the chunk crosses the row's end): the 16 bytes that end
//    at the row's last element, which lie in the row;
//  * have <= 0 or a row past the matrix: the tile's first chunk (whole).
XPOSE_HD inline const char *edge_chunk_src(const char *tile0,
                                           const char *chunk, int64_t have,
                                           int V, int S, bool in_row) {
  if (!in_row || have <= 0) return tile0;
  return have >= V ? chunk : chunk + have * S - 16;
}
// The loaded bytes (lo = bytes 0-7, hi = 8-15) made into the chunk: the
// partial chunk's have * S bytes sit at the top of the load and move down
// to the start, zero above; chunks past the row's end or rows past the
// matrix become zero.
XPOSE_HD inline void edge_chunk_fix(uint64_t &lo, uint64_t &hi, int64_t have,
                                    int V, int S, bool in_row) {
  if (!in_row || have <= 0) {
    lo = hi = 0;
  } else if (have < V) {
    const int sh = (int)(16 - have * S) * 8;  // S * 8 .. 120 bits
    if (sh >= 64) {
      lo = hi >> (sh - 64);
      hi = 0;
    } else {
      lo = (lo >> sh) | (hi << (64 - sh));
      hi >>= sh;
    }
  }
}

// Cache policy of the global accesses: plain, non-temporal stores, or
// non-temporal loads and stores (the data is touched exactly once).
enum CachePolicy : int { kCacheDefault = 0, kNtStore = 1, kNtLoadStore = 2 };

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

template <int S> struct Elem;
template <> struct Elem<1> { using E = uint8_t;  using U = uint32_t; static constexpr int K = 4; };
template <> struct Elem<2> { using E = uint16_t; using U = uint32_t; static constexpr int K = 2; };
template <> struct Elem<4> { using E = uint32_t; using U = uint32_t; static constexpr int K = 1; };
template <> struct Elem<8> { using E = uint64_t; using U = uint64_t; static constexpr int K = 1; };

// Compile-time geometry of one tile kernel.
//   S   element bytes          TR x TC  tile in elements
//   NT  threads per workgroup  L        LDS layout      CP  cache policy
template <int S, int TR, int TC, int NT, int L, int CP, bool DIRECT = false>
struct Tile {
  static constexpr int CACHE = CP;
  // Interior tiles load straight from global memory into LDS
  // (global_load_lds_dwordx4), skipping the trip through registers.
  static constexpr bool DIRECT_LDS = DIRECT;
  using E = typename Elem<S>::E;
  using U = typename Elem<S>::U;
  static constexpr int K = Elem<S>::K;          // input rows per LDS unit
  static constexpr int UB = (int)sizeof(U);     // unit bytes
  static constexpr int V = 16 / S;              // elements per 16-byte vector
  static constexpr int UPV = 16 / UB;           // units per 16-byte vector
  static constexpr int P = TR / K;              // unit rows of the LDS tile
  static constexpr int NCI = TC / V;            // 16-B chunks per input tile row
  static constexpr int NCO = TR / V;            // 16-B chunks per output tile row
  static constexpr int NCL = TC / UPV;          // 16-B chunks per LDS row
  static constexpr int STRIDE = TC + (L == kPad1 ? 1 : 0);  // LDS row, units
  static constexpr int NW = NT / 64;            // waves per workgroup
  static constexpr int LIT = P * NCI / NT;      // load tasks per lane
  static constexpr int SIT = TC * NCO / NT;     // store tasks per lane
  static constexpr int LDS_UNITS = P * STRIDE;
  static constexpr int LDS_BYTES = LDS_UNITS * UB;
  // Row writes are 16-byte LDS stores unless the pad breaks their alignment.
  static constexpr bool WIDE_WRITE = (L != kPad1);
  static constexpr int LAYOUT = L;
  static constexpr int TCOLS = TC;

  static_assert(NT % 64 == 0, "whole wavefronts");
  static_assert(TR % V == 0 && TC % V == 0, "tile must hold whole vectors");
  static_assert(P * NCI % NT == 0 && TC * NCO % NT == 0, "even task split");
  static_assert(LIT >= 1 && SIT >= 1, "every lane has work");
  static_assert(NCL >= 1 && (NCL & (NCL - 1)) == 0, "power-of-two chunks");
  static_assert(NCL >= K, "rotation needs at least K chunks per LDS row");
  static_assert(!DIRECT || (K == 1 && L != kPad1 && NCI <= 64 && 64 % NCI == 0),
                "direct loads need whole 16-byte units in contiguous LDS rows");

  // Swizzle: 16-byte chunk lc of LDS row p is stored at chunk
  // rot(lc) ^ chunk_xor(p, lc mod K).
  //  * rot: with K > 1 a lane writes K adjacent chunks (siblings), one per
  //    instruction, so the chunk index is rotated right by log2(K) bits and
  //    the chunks one write instruction covers (stride K) become
  //    consecutive.
  //  * (p / UPV) * QSTEP: the UPV rows one lane gathers share the mask, and
  //    the row groups a half-wave gathers from one column land in different
  //    slots of the bank window.  8-byte units are read 256 bytes per pass,
  //    where the 4 columns a half-wave reads span two chunks, hence step 2.
  //  * sibling term: where a half-wave's column reads cover several sibling
  //    chunks (at most 4 output chunks per tile column, so a half-wave reads
  //    8 / NCO chunks of NCO row groups) and rotation has put the siblings a
  //    multiple of 8 chunks apart, each sibling gets its own block of NCO
  //    slots.
  //  * row term: where one 8-lane write group spans several LDS rows (fewer
  //    than 8 chunks per input row) of one row group, those rows get
  //    disjoint chunk blocks.  (It varies with p % UPV, which is constant
  //    within a read instruction.)
  static constexpr int QSTEP = S == 8 ? 2 : 1;
  static constexpr bool SIB = K > 1 && NCO <= 4 && NCL / K >= 8;
  static constexpr bool ROWX = NCI < 8 && NCL >= 8;
  XPOSE_HD static inline int chunk_xor(int p, int g) {
    int x = ((p / UPV) * QSTEP) & (NCL - 1);
    if constexpr (SIB) x ^= (g * NCO) & (NCL - 1);
    if constexpr (ROWX) x ^= ((p % UPV) * NCI) & (NCL - 1);
    return x;
  }
  // Unit index of logical unit (p, c) in the LDS tile.
  XPOSE_HD static inline int lds_index(int p, int c) {
    if constexpr (L == kSwizzle) {
      constexpr int NB = ilog2(NCL), KB = ilog2(K);
      const int lc = c / UPV;
      const int g = lc & (K - 1);
      const int rc = KB ? ((lc >> KB) | (g << (NB - KB))) : lc;
      const int chunk = rc ^ chunk_xor(p, g);
      return p * TC + chunk * UPV + (c % UPV);
    } else {
      return p * STRIDE + c;
    }
  }
};


// Lane -> (row, chunk) for one wave-wide task over a block of tile rows that
// are NCH 16-byte chunks long; wt numbers the wave tasks of a phase.
//   SPLIT == false or NCH <= 8: consecutive lanes take consecutive chunks of
//     a row, a wave covers 64 / NCH rows.
//   SPLIT and NCH >= 16: a half-wave covers 8 chunks of each of 4 rows and
//     the two halves take neighbouring 8-chunk groups of the same 4 rows, so
//     a half-wave never spans more than 8 chunks (128 bytes) of one row.
template <int NCH, bool SPLIT>
XPOSE_HD inline void lane_map(int wt, int lane, int &row,
                                         int &chunk) {
  if constexpr (!SPLIT || NCH <= 8) {
    if constexpr (NCH <= 64) {
      static_assert(64 % NCH == 0, "chunks per row divide the wave");
      row = wt * (64 / NCH) + lane / NCH;
      chunk = lane % NCH;
    } else {
      static_assert(NCH % 64 == 0, "rows span whole waves");
      row = wt / (NCH / 64);
      chunk = (wt % (NCH / 64)) * 64 + lane;
    }
  } else {
    static_assert(NCH % 16 == 0, "split map needs 16-chunk multiples");
    constexpr int CG = NCH / 16;
    const int h = lane >> 5, m = lane & 31;
    row = (wt / CG) * 4 + (m >> 3);
    chunk = ((wt % CG) * 2 + h) * 8 + (m & 7);
  }
}


// Line-aligned output tiles (2-, 4- and 8-byte elements): the LDS tile holds
// the HALO = 128 / S input rows above the tile as well, laid out as an
// ordinary swizzled tile of TR + HALO rows (Base); each output row's segment
// is shifted back onto a 128-byte line.  gather() assembles the 16-byte
// output vector whose first element is input row `rel` of the LDS tile
// (counted in input rows): for 2-byte elements `rel` may be odd, and the
// vector then straddles two packed units in each word, which one byte
// funnel shift (v_alignbyte) per word puts back together.
template <int S, int TR, int TC, int NT, int CP>
struct ShiftTile {
  static constexpr int HALO = 128 / S;        // elements per 128-byte line
  static constexpr int PR = TR + HALO;        // input rows held in LDS
  using Base = Tile<S, PR, TC, NT, kSwizzle, CP>;
  using U = typename Base::U;
  static constexpr int K = Base::K, V = Base::V, UPV = Base::UPV;
  static constexpr int NCO = TR / V;          // 16-B chunks per output segment
  static constexpr int NW = NT / 64;
  static constexpr int SIT = TC * NCO / NT;   // store tasks per lane
  // Packed units: one spare unit row after the tile, so the fifth unit a
  // gather reads (used only when the segment starts mid-unit) is always
  // inside the array and never aliases a bank the other lanes read.
  static constexpr int LDS_UNITS = Base::LDS_UNITS + (K > 1 ? TC : 0);
  static constexpr int LDS_BYTES = LDS_UNITS * (int)sizeof(U);
  static_assert(S == 2 || S == 4 || S == 8, "2-, 4- or 8-byte elements");
  static_assert(TR % HALO == 0, "segments must stay line-aligned");
  static_assert(TC * NCO % NT == 0 && SIT >= 1, "even store split");
  // Unit (Base::U) index of unit row `ur` (at most Base::P, the spare
  // row), column c.
  XPOSE_HD static inline int unit_index(int ur, int c) {
    return Base::lds_index(ur, c);
  }
  // First unit row and byte shift of the vector starting at input row rel.
  XPOSE_HD static inline void gather_rows(int rel, int &ur, int &shift) {
    ur = rel / K;
    shift = (rel % K) * S;
  }
  // Unit rows gather() reads: UPV, plus one to funnel-shift across units.
  static constexpr int GATHER_UNITS = K > 1 ? UPV + 1 : UPV;
};

// Transpose-read tiles (1- and 2-byte elements): input rows unchanged in
// LDS, 8-byte units XOR-permuted per row (the full reasoning is with the
// kernel).
template <int S, int TR, int TC, int NT, int CP, bool DIRECT>
struct TrTile {
  static constexpr int V = 16 / S;          // elements per output vector
  static constexpr int HR = V / 2;          // rows per transpose read
  static constexpr int NQ = 16 / HR;        // row vectors per group
  static constexpr int RB = TC * S;         // bytes per LDS row
  static constexpr int NCL = RB / 16;       // 16-byte chunks per row
  static constexpr int NU = RB / 8;         // 8-byte units per row
  static constexpr int NW = NT / 64;
  static constexpr int NRB = TR / 32;       // 32-row blocks
  static constexpr int LIT = TR * NCL / NT; // load tasks per lane
  static constexpr int SIT = NRB * NU / (4 * NW);  // store tasks per lane
  static constexpr int LDS_BYTES = TR * RB;
  static constexpr int WB = ilog2(256 / RB);  // log2(rows per 256 B)
  static_assert(S == 1 || S == 2, "transpose reads move 8- or 16-bit elements");
  static_assert(NQ * V == 32, "a group covers 32 rows");
  static_assert(NCL >= 4 && NCL <= 16, "rows of 64 to 256 bytes");
  static_assert(NRB % 2 == 0, "a half-wave takes two 32-row blocks");
  static_assert(TR * NCL % NT == 0 && LIT >= 1, "even load split");
  static_assert(NRB * NU % (4 * NW) == 0 && SIT >= 1, "even store split");
  static_assert(64 % NCL == 0, "rows fit a wave");
  // XOR mask of the 8-byte unit index in row `row`.
  XPOSE_HD static inline int swz(int row) {
    const int v = (row & (HR - 1)) | ((row >> 1) & ~(HR - 1) & 31);
    const int f = (v >> WB) & (NU - 1);
    return DIRECT ? (f & ~1) : f;
  }
  // Byte offset of 8-byte unit `u` of row `row`.
  XPOSE_HD static inline int unit_at(int row, int u) {
    return row * RB + ((u ^ swz(row)) << 3);
  }
  // The 16-byte chunk `ch` of row `row`: its offset, and whether its two
  // halves are stored swapped.
  XPOSE_HD static inline void chunk_at(int row, int ch, int &off,
                                                  bool &swap) {
    const int f = swz(row);
    off = row * RB + ((ch ^ (f >> 1)) << 4);
    swap = f & 1;
  }
};


}  // namespace xpose
