// Internal interface between the C-ABI front end (xpose_api.cpp) and the
// gfx950 kernels (xpose_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xpose {

// LDS tile layouts; values match xpose_layout in include/xpose.h.
enum Layout : int {
  kUnpadded = 1,
  kPad1 = 2,
  kSwizzle = 3,
  kNaiveRead = 4,  // no LDS: one element per thread, reads coalesced
  kNaiveWrite = 5  // no LDS: one element per thread, writes coalesced
};

// Arguments of one tiled-transpose launch.  Sizes, pitches and strides are
// in elements; the grid is tiles_r * tiles_c * batch_count workgroups and
// workgroup g handles batch entry batch_first + g / (tiles_r * tiles_c).
struct TileArgs {
  void *out;
  const void *in;
  int64_t rows, cols, ld_in, ld_out, stride_in, stride_out;
  uint32_t tiles_r, tiles_c;
  uint32_t batch_first;
  int32_t vec_ok;      // 1: interior tiles may use 128-bit global accesses
  uint32_t group_rows; // tile order: super-tile height in tiles (>= 1)
  uint32_t group_cols; // tile order: super-tile width in tiles (>= 1)
  int32_t xcd_remap;   // 1: one contiguous tile range per XCD
  int32_t order;       // kOrderSuperTiles, kOrderDiagonal or kOrderColumnBands
};

// Tile orders (values match xpose_order in include/xpose.h).
enum TileOrder : int {
  kOrderSuperTiles = 1,
  kOrderDiagonal = 2,
  kOrderColumnBands = 3
};

// Workgroup index -> (batch entry, tile row, tile column), for `block` of a
// grid of `nblocks` workgroups.  A bijection from [0, nblocks) onto
// batch x tiles_r x tiles_c whenever nblocks = batch_count * tiles_r * tiles_c
// and 1 <= group_rows <= tiles_r, 1 <= group_cols <= tiles_c.
//   xcd_remap: the hardware hands consecutive workgroups to the 8 XCDs in
//     turn; remapping gives each XCD one contiguous range of tiles instead.
//   group_rows GR x group_cols GC: tiles are walked in super-tiles of GR tile
//     rows by GC tile columns, super-tiles row-major, tile rows fastest
//     inside a super-tile.  The workgroups resident at one time then cover a
//     compact block of the input AND of the output, instead of whole rows of
//     one and a thin column band of the other.  GR = 1 with GC = tiles_c is
//     plain row-band order.
//   diagonal: workgroup g takes tile row g mod tiles_r and tile column
//     (g / tiles_r + tile row) mod tiles_c, so consecutive workgroups differ
//     in both tile row and tile column.  With power-of-two pitches the
//     resident tiles then spread over all address offsets on both the read
//     and the write side, instead of camping on the few memory channels one
//     narrow offset range maps to.
//   column bands: bands of group_cols tile columns, left to right; inside a
//     band, tile rows top to bottom, the band's tile columns left to right
//     inside each tile row (the last band may be narrower).  Each tile's
//     left and upper neighbours then ran shortly before it, except in a
//     band's first column: what a tile shares with them (input lines that
//     straddle the tile's column edge, the halo rows of line-aligned output
//     tiles) is still in L2.
__host__ __device__ inline void tile_coords(const TileArgs &a, uint32_t block,
                                            uint32_t nblocks, uint32_t &tr,
                                            uint32_t &tc, int64_t &b) {
  uint32_t g = block;
  if (a.xcd_remap) {
    const uint32_t q = nblocks / 8, r = nblocks % 8, x = g % 8;
    g = x * q + (x < r ? x : r) + g / 8;
  }
  const uint32_t per = a.tiles_r * a.tiles_c;
  b = (int64_t)(g / per) + a.batch_first;
  g %= per;
  if (a.order == kOrderDiagonal) {
    tr = g % a.tiles_r;
    tc = (g / a.tiles_r + tr) % a.tiles_c;
    return;
  }
  if (a.order == kOrderColumnBands) {
    const uint32_t GC = a.group_cols;
    const uint32_t band = g / (GC * a.tiles_r), rem = g % (GC * a.tiles_r);
    const uint32_t cols_here =
        (band + 1) * GC <= a.tiles_c ? GC : a.tiles_c - band * GC;
    tr = rem / cols_here;
    tc = band * GC + rem % cols_here;
    return;
  }
  const uint32_t GR = a.group_rows, GC = a.group_cols;
  const uint32_t band = GR * a.tiles_c;  // tiles in one full super-tile row
  const uint32_t sr = g / band, rem = g % band;
  const uint32_t rows_here =
      (sr + 1) * GR <= a.tiles_r ? GR : a.tiles_r - sr * GR;
  const uint32_t span = rows_here * GC;  // tiles in one full super-tile
  const uint32_t sc = rem / span, rem2 = rem % span;
  tr = sr * GR + rem2 % rows_here;
  tc = sc * GC + rem2 / rows_here;
}

// One compiled tile kernel.
struct TileKernel {
  int elem_bytes, tile_rows, tile_cols, threads, layout, cache, lds_bytes;
  // One workgroup per tile: grid = tiles.  lds_extra bytes of dynamic LDS
  // are reserved per workgroup (never touched): a cap on the workgroups that
  // share one compute unit.
  hipError_t (*launch)(const TileArgs &, uint32_t grid, uint32_t lds_extra,
                       hipStream_t);
  // Persistent, double-buffered variant (null if not built): `grid`
  // workgroups (a multiple of 8) walk `ntiles` tiles; LDS use is twice
  // lds_bytes.
  hipError_t (*launch_persistent)(const TileArgs &, uint32_t ntiles,
                                  uint32_t grid, hipStream_t);
  // Interior tiles are loaded straight into LDS (global_load_lds_dwordx4).
  bool direct_lds;
  // Line-aligned output tiles: each output row's segment is shifted back to
  // start on a 128-byte line; the grid needs ceil((rows + 128 / elem_bytes
  // - 1) / tile_rows) tile rows (2-, 4- and 8-byte elements).
  bool aligned_out;
  // Row-major LDS tile of raw elements read back with the LDS transpose
  // reads (ds_read_b64_tr_b16 / _b8; 1- and 2-byte elements only).
  bool tr_read = false;
  // Line-aligned tiles in column strips (null if not built): `grid` =
  // batch_count * nseg * tiles_c workgroups, each walking `seg` tile rows
  // (nseg = ceil(tiles_r / seg) segments per strip) with its input rows in
  // an LDS ring of strip_lds_bytes.
  hipError_t (*launch_strip)(const TileArgs &, uint32_t seg, uint32_t nseg,
                             uint32_t grid, hipStream_t) = nullptr;
  int strip_lds_bytes = 0;
};

// Every compiled tile kernel; *count receives the table length.
const TileKernel *tile_kernels(int *count);

// Packed batches of small matrices: dense rows x cols matrices (ld = the
// row length, stride = rows * cols), `per_block` whole matrices per
// workgroup.  The block's input bytes are one contiguous range and so are
// its output bytes: both move as 16-byte vectors, and the LDS holds the
// block while each lane gathers its output elements.
struct PackedArgs {
  void *out;
  const void *in;
  uint32_t rows, cols;   // of one matrix
  uint32_t per_block;    // matrices per workgroup
  uint32_t pad;          // LDS padding per input row, in elements (0 = none)
  int64_t count;         // matrices in this launch
};

struct PackedKernel {
  int elem_bytes, threads, block_bytes, cache;
  hipError_t (*launch)(const PackedArgs &, uint32_t grid, hipStream_t);
};
const PackedKernel *packed_kernels(int *count);

// Naive one-element-per-thread transpose (no LDS), `batch` matrices from
// a.in / a.out (a.batch_first is ignored); the ablation baseline.
hipError_t launch_naive(const TileArgs &a, int64_t batch, int elem_bytes,
                        bool read_coalesced, hipStream_t stream);

// One compiled 128-bit copy kernel.
struct CopyKernel {
  int threads, unroll, cache;
  hipError_t (*launch)(char *dst, const char *src, int64_t nvec, hipStream_t);
};
const CopyKernel *copy_kernels(int *count);

// Device-to-device copy with kernel k (byte path for unaligned pointers and
// the tail).
hipError_t launch_copy(const CopyKernel &k, void *dst, const void *src,
                       int64_t bytes, hipStream_t stream);

// LDS bank microbenchmark; lane_bytes is a host array of 64 byte offsets.
hipError_t launch_lds_probe(uint64_t *out, const int32_t *lane_bytes,
                            int width, bool is_write, int iters,
                            hipStream_t stream);

}  // namespace xpose
