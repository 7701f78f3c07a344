// LDS geometry and lane maps of the tiled SGEMM kernel: where each lane puts
// A's and B's tile elements in LDS, where the matrix-core operands are read
// from, and which block of C each workgroup takes.  Host and device code:
// the kernel uses it, and a host program lists the LDS addresses of every
// lane so the bank behaviour of each built layout is checked without a GPU.
// Internal, not part of the ABI.
//
// The structure is the SGEMM of "Padded Shared Memory: Eliminating Bank
// Conflicts": A's tile is stored transposed (As[l][i]) so the product reads
// consecutive rows i, and that store is the conflicted one when As's row
// stride is a multiple of the bank count ("How Shared Memory Is Addressed").
// Here the bank count and the lanes served per pass are gfx950's, as
// measured for 4-byte LDS accesses: 32 banks, one 32-lane half-wave per pass
// (the same figures as the pages' 32-lane hardware, so the pads come out
// the same, but they are derived from the measured geometry below).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sgemm_kernels.h"

#define SGEMM_HD __host__ __device__

namespace xpose {

// As layouts; values match xpose_as_layout in include/xpose_sgemm.h.
enum AsLayout : int { kAsUnpadded = 1, kAsPadded = 2, kAsSwizzle = 3 };

// Compile-time geometry of one SGEMM kernel: BK is the k step, L the As
// layout, BM_ the rows of C per workgroup (64, 128 or 256).  A workgroup of
// BM_ / 32 waves computes a BM_ x 128 block of C; wave w computes the
// 64 x 64 block at (64 * (w / 2), 64 * (w % 2)) as 2 x 2 matrix-core tiles
// of 32 x 32.
template <int BK, int L, int BM_ = 128>
struct SgemmTile {
  static constexpr int BM = BM_, BN = 128, NT = 2 * BM_;
  static constexpr int WM = 64, WN = 64;  // C block of one wave

  // A's BM x BK tile is read in strips of LK = min(BK, 32) columns: each
  // lane reads one 16-byte vector (4 consecutive l) of one row i of a
  // strip, LPR lanes per strip row.
  static constexpr int LK = BK < 32 ? BK : 32;
  static constexpr int LPR = LK / 4;
  static constexpr int A_ROWS_PER_PASS = NT / LPR;
  static constexpr int A_ROW_PASSES = BM / A_ROWS_PER_PASS;
  static constexpr int A_PASSES = A_ROW_PASSES * (BK / LK);  // vectors per lane
  // B's BK x 128 tile: 32 lanes per row of 128 floats.
  static constexpr int B_LPR = BN / 4;
  static constexpr int B_ROWS_PER_PASS = NT / B_LPR;
  static constexpr int B_PASSES = BK / B_ROWS_PER_PASS;

  // The transposed store of element e of a lane's vector writes
  // As[s LK + 4c + e][i] for the strip s, the lane's chunk c < LPR and row i.
  // One half-wave (the 32 lanes one pass serves) holds HG = 32 / LPR
  // consecutive rows i (starting at a multiple of HG) times LPR chunks of
  // one strip.  With row stride BM + p (BM a multiple of 32) the lane lands
  // on bank (s LK p + 4 c p + e p + i) mod 32, the first term the same for
  // the whole half-wave, so
  //   p = 0:      the bank is i mod 32 alone: LPR lanes per bank, LPR-way;
  //   4 p = HG:   the chunks fall HG banks apart, covering all 32 once;
  // hence the padded stride BM + HG / 4 = BM + 32 / LK.
  static constexpr int HG = 32 / LPR;
  static constexpr int PAD = L == kAsPadded ? HG / 4 : 0;
  static constexpr int AS_STRIDE = BM + PAD;
  static constexpr int AS_FLOATS = BK * AS_STRIDE;
  static constexpr int BS_FLOATS = BK * BN;
  static constexpr int LDS_BYTES = 4 * (AS_FLOATS + BS_FLOATS);
  static constexpr int LAYOUT = L;
  static constexpr int KSTEP = BK;
  // Waves per SIMD the register budget is set for.  A workgroup has
  // NT / 64 waves spread over the compute unit's 4 SIMDs; as many
  // workgroups as the LDS of `stages` buffers lets share the compute unit's
  // 160 KiB give LDS_WGS * NT / 256 waves per SIMD (rounded up: a
  // 128-thread workgroup puts one wave on two of the four SIMDs).  The
  // budget is at most four waves (128 registers per lane) where the k
  // step's prefetch registers (one 16-byte vector per A and B pass) fit
  // beside the 64 accumulators, at most four vectors, else three waves;
  // and for workgroups of more than one wave per SIMD it is a whole number
  // of workgroups, since a partial one never fits (256-row blocks, two
  // waves per SIMD: 4, i.e. two workgroups, or 2).
  SGEMM_HD static constexpr int waves_per_simd(int stages) {
    return whole_workgroups(
        min_int((A_PASSES + B_PASSES <= 4 ? 4 : 3),
                ((160 * 1024) / (stages * LDS_BYTES) * NT + 255) / 256));
  }
  SGEMM_HD static constexpr int min_int(int a, int b) { return a < b ? a : b; }
  SGEMM_HD static constexpr int whole_workgroups(int w) {
    return NT <= 256 ? (w > 0 ? w : 1)
                     : (w / (NT / 256) > 0 ? w / (NT / 256) * (NT / 256)
                                           : NT / 256);
  }

  static_assert(BK == 8 || BK == 16 || BK == 32 || BK == 64, "built k steps");
  static_assert(BM == 64 || BM == 128 || BM == 256, "built block heights");
  static_assert(B_PASSES >= 1, "every lane loads part of B's tile");
  static_assert(A_ROW_PASSES * A_ROWS_PER_PASS == BM, "whole A tile");
  static_assert(B_PASSES * B_ROWS_PER_PASS == BK, "whole B tile");
  static_assert(L != kAsPadded || 4 * PAD == HG, "pad spreads the chunks");

  // Swizzle: row l of As keeps stride BM and holds element i at column
  // i ^ x(l), x(l) = ((l / 4) mod LPR) * HG.  In one half-wave's store
  // (l / 4) mod LPR is the chunk c and i runs over HG consecutive rows from
  // a multiple of HG, so the banks (i ^ c HG) mod 32 are all distinct;
  // x(l) < 32 only
  // permutes i inside its aligned group of 32, so the product's reads of 32
  // consecutive i stay one full row of banks.
  SGEMM_HD static constexpr int swz(int l) {
    return L == kAsSwizzle ? ((l >> 2) & (LPR - 1)) * HG : 0;
  }
  SGEMM_HD static constexpr int as_index(int l, int i) {
    return l * AS_STRIDE + (i ^ swz(l));
  }
  SGEMM_HD static constexpr int bs_index(int l, int j) { return l * BN + j; }

  // Loader lane maps: thread t, pass p (A: row passes within a strip, then
  // strips).
  SGEMM_HD static constexpr int a_row(int t, int p) {
    return (p % A_ROW_PASSES) * A_ROWS_PER_PASS + t / LPR;
  }
  SGEMM_HD static constexpr int a_col(int t, int p) {
    return (p / A_ROW_PASSES) * LK + 4 * (t % LPR);
  }
  SGEMM_HD static constexpr int b_row(int t, int p) {
    return p * B_ROWS_PER_PASS + t / B_LPR;
  }
  SGEMM_HD static constexpr int b_col(int t) { return 4 * (t % B_LPR); }

  // Matrix-core operands (v_mfma_f32_32x32x2_f32): for the k pair starting
  // at kk, lane q supplies A[i0 + q % 32][kk + q / 32] and
  // B[kk + q / 32][j0 + q % 32]; its 16 results are C[i0 + r_row][j0 + q % 32]
  // with r_row = 8 (r / 4) + 4 (q / 32) + r % 4 for r < 16.
  SGEMM_HD static constexpr int wave_row(int w) { return WM * (w / 2); }
  SGEMM_HD static constexpr int wave_col(int w) { return WN * (w % 2); }
  SGEMM_HD static constexpr int acc_row(int q, int r) {
    return 8 * (r / 4) + 4 * (q / 32) + r % 4;
  }
};

// A 64-bit value rebuilt from the first lane's copies of its two 32-bit
// halves; `first_lane` has the signature of the lane-broadcast builtin,
// int(int).  Both halves are taken back as unsigned: a low half with bit 31
// set, converted from int straight to 64 bits, would sign-extend over the
// high half and turn an address into 0xffffffff'xxxxxxxx.
template <class F>
SGEMM_HD inline uint64_t uniform_bits(uint64_t v, F first_lane) {
  const uint32_t lo = (uint32_t)first_lane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)first_lane((int)(uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// Block order: workgroup `block` of `tiles_m * tiles_n` -> block row and
// column of C, a bijection whenever group_m >= 1.
//   xcd_remap: the hardware hands consecutive workgroups to the 8 XCDs in
//     turn; the remap gives each XCD one contiguous range of blocks (XCD x
//     receives the blocks b with b mod 8 = x and numbers them from the end
//     of XCD x - 1's range), so the blocks sharing one XCD's L2 also share
//     rows of A and columns of B.
//   group_m: blocks are walked in groups of group_m block rows, block column
//     by block column inside a group (the last group may be shorter), so
//     the resident blocks reuse a few rows of A and columns of B.
SGEMM_HD inline void sgemm_block(uint32_t block, uint32_t tiles_m,
                                 uint32_t tiles_n, uint32_t group_m,
                                 int32_t xcd_remap, uint32_t &bm,
                                 uint32_t &bn) {
  const uint32_t total = tiles_m * tiles_n;
  uint32_t g = block;
  if (xcd_remap) {
    const uint32_t q = total / 8, r = total % 8, x = block % 8;
    g = x * q + (x < r ? x : r) + block / 8;
  }
  const uint32_t span = group_m * tiles_n;
  const uint32_t grp = g / span, first = grp * group_m;
  const uint32_t rows = tiles_m - first < group_m ? tiles_m - first : group_m;
  const uint32_t in = g - grp * span;
  bm = first + in % rows;
  bn = in / rows;
}

}  // namespace xpose
