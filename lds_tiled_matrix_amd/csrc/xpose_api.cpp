// C-ABI front end of libxpose.so: argument validation, kernel choice, launch
// and error mapping.  Validation and planning are pure host code that never
// touches the GPU, so every error path can be exercised on a machine without
// one.  The operation itself is defined in include/xpose.h.

#include "../../include/xpose.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "sgemm_kernels.h"
#include "xpose_kernels.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return XPOSE_EHIP;
}

int elem_bytes_of(int32_t dtype) {
  switch (dtype) {
    case XPOSE_F32: return 4;
    case XPOSE_F16: return 2;
    case XPOSE_BF16: return 2;
    case XPOSE_U8: return 1;
    case XPOSE_F64: return 8;
    default: return 0;
  }
}

// Default launch configuration, chosen from the measured sweeps over tile
// shape, workgroup size, cache policy and tile order on MI355X.
//   out_row128: every output row start is 128-byte aligned (pointer, pitch,
//     batch stride), so each output segment is whole cache lines and
//     non-temporal stores pay.  Otherwise segments straddle lines: plain
//     (write-back) stores then merge the partial lines in L2 and win over
//     non-temporal ones, which write partial lines straight to memory.  The
//     input side's alignment does not enter: misaligned reads cost little.
//   small: a batch of matrices of at most kSmallMatrixBytes each.  Resident
//     workgroups then cover a few whole matrices, a dense window on both the
//     input and the output side, and a taller tile with small super-tiles
//     streams at copy speed.
//   align: line-aligned output tiles (each output segment shifted onto a
//     line), the default for 2-, 4- and 8-byte elements whose output rows
//     are not line-aligned: every store is a whole line again, so
//     non-temporal stores win.  (1-byte elements: no gain measured, none
//     built.  2-byte elements in matrices of fewer than kShortAlignRows
//     rows: the extra halo tile row costs more than whole lines gain, e.g.
//     a batch of 150 x 150 fp16 runs 2.3 TB/s line-aligned, 3.6 without.
//     2-byte elements in big calls take 128 x 64 tiles: 16383^2 fp16 runs
//     5.0 TB/s with them, 4.3-4.4 with 64 x 64.)
//     Explicit knobs they are not built with (another layout,
//     elementwise or direct loads, persistent workgroups, a tile shape,
//     workgroup size or cache policy without such a kernel) select the
//     ordinary tiles with their own defaults instead.
//   big: the call moves at least kBigCallBytes (read + write), twice the
//     256 MB memory-side cache.  The diagonal order (resident tiles spread
//     over all row and column offsets) is then the one that holds up when
//     the bytes come from HBM: 8192^2 fp32 runs 5.9 TB/s cache-cold with
//     it, 0.97 of the cold copy, against 5.0-5.1 TB/s (0.82) for compact
//     32 x 32 super-tiles, which win only in back-to-back repeats of the
//     same call (7.3 against 6.8 TB/s) because the memory-side cache then
//     serves part of the bytes.  The diagonal order also runs best with few
//     workgroups per compute unit: every resident workgroup streams its own
//     set of rows on both sides, and HBM serves fewer, longer streams
//     better.  Measured caps: 8192^2 fp32 with 128 x 128 tiles 0.97 of the
//     cold copy at 1 workgroup per compute unit, 0.94 at 2 (no cap: LDS
//     allows 2); 16384^2 fp16 with 128 x 64 tiles 0.89 at 3, 0.86 uncapped
//     (8); 1-byte 0.84 at 4, 0.81-0.83 uncapped; 8-byte 32 x 32 0.86 at 4,
//     0.84 uncapped.  Below 512 MiB, compact super-tiles hold up cold as
//     well on most shapes (6144^2 fp32: 0.92 against 0.85).
// cache is an xpose_cache value; group_cols 0 means all tile columns;
// occupancy caps the workgroups per compute unit (0 = no cap).
struct Default {
  int tile_rows, tile_cols, threads, layout, cache, group_rows, group_cols,
      xcd_remap, order;
  bool align_out = false;
  int occupancy = 0;
};
constexpr int64_t kSmallMatrixBytes = 64ll << 20;
constexpr int64_t kShortAlignRows = 256;
constexpr int64_t kBigCallBytes = 512ll << 20;
constexpr int64_t kMidCallBytes = 128ll << 20;
// Single matrices with both sides at least kLargeMinDim take 128 KiB tiles
// (one workgroup per compute unit) in the diagonal order: 2-byte elements
// from kLargeCallBytes (read + write) on; 4-byte ones in the pitches below
// where the diagonal order wins, from kHugeCallBytes on and under
// kBigCallBytes; 8-byte ones in those pitches from kLargeCallBytes on.
// Measured against the tiles before them, fraction of the copy hot / cold:
// fp16 8192^2 1.03 / 0.94 against 0.94 / 0.78, 16384^2 0.94 / 0.92 against
// 0.89 / 0.88, 32768 x 16384 0.87 / 0.88 against 0.80 / 0.80 (256 x 256);
// fp32 16384 x 8192 0.93 / 0.93 against 0.90 / 0.90, 16384^2 0.89 / 0.89
// against 0.82 / 0.82 (256 x 128; at 8192^2 level hot and 0.94 against
// 0.97 cold, so 128 x 128 stays there); fp64 8192^2 0.92 / 0.93 against
// 0.86 / 0.88 (128 x 128).  fp16 6144^2 (144 MiB) loses (0.93 / 0.84
// against 1.04 / 0.88), hence the floor.
constexpr int64_t kLargeCallBytes = 256ll << 20;
constexpr int64_t kHugeCallBytes = 1024ll << 20;
constexpr int64_t kLargeMinDim = 1024;
// The output pitch decides the tile order of large 4- and 8-byte transposes.
// Where output rows lie within kPitchSlack bytes of a multiple of
// kPitchPeriod apart, the column walk of a compact super-tile keeps writing
// the same few address offsets and stalls on the memory channels they map
// to (fp32 8192^2: 0.82 of the cold copy with 32 x 32 super-tiles, 0.97
// diagonal; output pitch 8224 elements, 128 bytes off the period: 0.74
// against 0.84-0.86); there the diagonal order wins, from 64 MiB on for one
// fp32 matrix (8192 x 1024 1.10 / 1.07 of the copy hot / cold against 0.90 /
// 0.94, 8192 x 4096 0.96 / 0.96 against 0.98 / 0.73, 16384 x 2048 0.95 /
// 0.92 against 0.95 / 0.72, 256 x 128 tiles) and from 256 MiB for one fp64
// matrix (4096^2 0.92 / 0.92 against 0.97 / 0.77, 128 x 128).  At other
// pitches the super-tiles win both ways: fp32 12288^2 0.88 against 0.78
// diagonal, 10240^2 0.89 against 0.76, 20480^2 0.86 against 0.80; fp64
// 6000^2 0.91 / 0.83 against 0.75 / 0.72, 8000^2 0.78 against 0.74, 10000^2
// 0.80 against 0.76 (16 x 16 super-tiles).  Output rows 128 KiB apart
// (kSlowSegmentPitch) with more than kSlowSegmentCols columns are worst for
// 1 KiB output segments (fp32 256 x 128 and fp64 128 x 128 tiles): fp32
// 32768 x 4096 0.83 against 0.87 with 128 x 128 tiles (512-byte segments),
// 32768 x 8192 0.79 against 0.91, 32768 x 12288 0.72 against 0.82; fp64
// 16384 x 3000 0.78 against 0.90 with 32 x 32 super-tiles, 16384 x 8192
// 0.77 against 0.84, 16384^2 0.73 against 0.81 (hot and cold alike).  With
// 2048 columns or fewer, or at 256 or 384 KiB, the long segments keep their
// lead (fp32 32768 x 2048 0.94 / 0.87 against 0.95 / 0.73, 65536 x 2048
// 0.87 against 0.74; fp64 16384 x 2048 0.96 / 0.86 against 0.96 / 0.81,
// 49152 x 4096 0.86 against 0.81).  fp32 8192^2, both pitches 32 KiB, keeps
// 128 x 128 tiles at one per compute unit: level hot, 0.969 cold against
// 0.953 (8 interleaved rounds), where every other fp32 shape measured in the
// diagonal order runs at least as fast with 256 x 128 tiles.
constexpr int64_t kPitchPeriod = 32768, kPitchSlack = 512;
constexpr int64_t kSlowSegmentPitch = 131072, kSlowSegmentCols = 2048;
constexpr int kSwz = xpose::kSwizzle, kSup = XPOSE_ORDER_SUPER_TILES,
              kDiag = XPOSE_ORDER_DIAGONAL, kBands = XPOSE_ORDER_COLUMN_BANDS,
              kWB = XPOSE_CACHE_DEFAULT,
              kNT = XPOSE_CACHE_NT_STORE;

// What the default kernel depends on.
struct CallShape {
  bool out_row128;   // output rows start on 128-byte lines
  bool small;        // a batch of matrices of at most kSmallMatrixBytes
  bool big;          // at least kBigCallBytes read + write
  bool mid;          // at least kMidCallBytes read + write
  bool align;        // line-aligned output tiles
  bool single;       // one matrix, both sides at least kLargeMinDim
  bool large, huge;  // single, and at least kLargeCallBytes / kHugeCallBytes
  bool on_period;    // output pitch near a multiple of kPitchPeriod
  bool slow_1k;      // output pitch near kSlowSegmentPitch, more columns
                     // than kSlowSegmentCols
  bool square_32k;   // both pitches near kPitchPeriod
};

Default default_for(int s, const CallShape &c) {
  if (c.align) {
    switch (s) {
      // 2-byte elements from kMidCallBytes on: 128 x 64 tiles in column
      // bands of at most 32 tile columns, for the reason given for 4-byte
      // elements below: 16383^2 0.85 of the copy hot and cold against 0.80
      // with 16 x 16 super-tiles, 20001 x 12345 0.75 / 0.74 against 0.73.
      // Between 128 and 512 MiB they trade a little hot for more cold
      // against 64 x 64 super-tiles (fraction of the copy hot / cold:
      // 12345 x 6789 0.95 / 0.76 against 0.92 / 0.67, 9999^2 0.91 / 0.75
      // against 0.90 / 0.65, 8191^2 0.90 / 0.86 against 0.93 / 0.77, 6001^2
      // 0.87 / 0.76 against 0.91 / 0.71, 4 x 4097^2 0.93 / 0.78 against
      // 0.94 / 0.68).  Below 128 MiB the two are level (4097^2 0.94 /
      // 0.85 against 0.94 / 0.84) or the wider tile wastes rows (2049^2,
      // 1000^2), so 64 x 64 super-tiles stay there.
      case 2:
        if (c.mid) return {128, 64, 256, kSwz, kNT, 1, 32, 1, kBands, true};
        return {64, 64, 256, kSwz, kNT, 16, 16, 1, kSup, true};
      // Bands of 64 tile columns, per-XCD ranges: the tile above (whose last
      // rows are the halo) and the tile to the left (which shares the input
      // lines that straddle the tile's column edge when input rows are not
      // line-aligned) ran shortly before on the same XCD, so both re-reads
      // hit L2.  12345 x 6789: 1.019 x the algorithmic read bytes beyond L2
      // and 0.84 of the copy, against 1.067 x with 16 x 16 super-tiles (the
      // tile above missed at each super-tile's top) and 1.25 x with 128 x 4
      // super-tiles (the tile to the left ran 128 tiles earlier).
      // From kBigCallBytes on, 64 x 128 tiles (512-byte input segments, half
      // the halo rows per output byte) in the same bands: fraction of the
      // copy hot / cold 12345 x 6789 0.82-0.83 / 0.83 against 0.81-0.82 /
      // 0.82, 6789 x 12345 0.84 / 0.84 against 0.81 / 0.82, 20001 x 12345
      // 0.81 / 0.81 against 0.79 / 0.79, 9999^2, 12345^2 and 16383^2 level
      // or slightly ahead.  Below it they are mixed (8193 x 8191 hot 0.91
      // against 0.84, cold 0.89 against 0.91; 4097 x 3001 0.81 / 0.76
      // against 0.92 / 0.81).
      case 4:
        if (c.big) return {64, 128, 256, kSwz, kNT, 1, 64, 1, kBands, true};
        return {64, 64, 256, kSwz, kNT, 1, 64, 1, kBands, true};
      case 8: return {32, 32, 256, kSwz, kNT, 16, 16, 1, kSup, true};
      default: break;  // no line-aligned tiles for 1-byte elements
    }
  }
  if (!c.out_row128) {
    switch (s) {
      case 4: return {128, 64, 256, kSwz, kWB, 32, 32, 1, kSup};
      case 2: return {64, 64, 256, kSwz, kWB, 16, 16, 1, kSup};
      case 1: return {128, 128, 256, kSwz, kWB, 16, 16, 1, kSup};
      default: return {32, 32, 256, kSwz, kWB, 16, 16, 1, kSup};
    }
  }
  // Tiles of 128 KiB (one workgroup per compute unit) give 512-byte row
  // segments on both sides for 2- and 8-byte elements and 1 KiB output
  // segments for 4-byte ones; HBM serves the longer streams better.
  switch (s) {
    case 4: {
      if (c.small) return {128, 64, 256, kSwz, kNT, 8, 8, 0, kSup};
      const bool diag = c.big ? c.on_period : c.single && c.on_period;
      if (!diag) return {32, 32, 256, kSwz, kNT, 8, 32, 1, kSup};
      if (c.single && !c.slow_1k && !c.square_32k)
        return {256, 128, 256, kSwz, kNT, 1, 0, 0, kDiag};
      return {128, 128, 256, kSwz, kNT, 1, 0, 0, kDiag, false, 1};
    }
    case 2:
      if (c.large) return {256, 256, 256, kSwz, kNT, 1, 0, 0, kDiag};
      if (c.big) return {128, 64, 256, kSwz, kNT, 1, 0, 0, kDiag, false, 3};
      return {128, 64, 256, kSwz, kNT, 32, 8, 0, kSup};
    case 1:
      if (c.big) return {128, 64, 128, kSwz, kNT, 1, 0, 0, kDiag, false, 4};
      return {128, 128, 256, kSwz, kNT, 16, 16, 1, kSup};
    default:
      if (c.large && c.on_period && !c.slow_1k)
        return {128, 128, 256, kSwz, kNT, 1, 0, 0, kDiag};
      if (c.big && !c.single)
        return {32, 32, 256, kSwz, kNT, 1, 0, 0, kDiag, false, 4};
      if (c.big) return {32, 32, 256, kSwz, kNT, 16, 16, 1, kSup};
      return {32, 32, 256, kSwz, kNT, 8, 32, 1, kSup};
  }
}

// The copy yardstick: one 16-byte vector per lane, non-temporal stores (the
// fastest copy measured at every size from 512 MiB to 2 GiB).
constexpr int kDefaultCopyThreads = 256, kDefaultCopyUnroll = 1;
constexpr int kDefaultCopyCache = XPOSE_CACHE_NT_STORE;

bool mul_ok(int64_t a, int64_t b, int64_t *r) {
  return !__builtin_mul_overflow(a, b, r);
}
bool add_ok(int64_t a, int64_t b, int64_t *r) {
  return !__builtin_add_overflow(a, b, r);
}

// Number of elements from the first to one past the last element touched by
// `count` matrices of `r` rows x `c` cols, pitch ld, matrix stride st.
bool extent(int64_t count, int64_t r, int64_t c, int64_t ld, int64_t st,
            int64_t *out) {
  int64_t a, b, t;
  if (!mul_ok(count - 1, st, &a) || !mul_ok(r - 1, ld, &b) ||
      !add_ok(a, b, &t) || !add_ok(t, c, &t))
    return false;
  *out = t;
  return true;
}

struct Plan {
  const xpose::PackedKernel *packed;  // packed batch of small matrices
  xpose::PackedArgs pk;
  const xpose::TileKernel *kernel;  // null for the naive kernels
  int persistent;                   // persistent workgroups per CU, 0 = none
  int occupancy;                    // cap on workgroups per CU, 0 = none
  int naive;                        // 0, xpose::kNaiveRead or kNaiveWrite
  int elem_bytes;
  xpose::TileArgs args;
  int64_t batch;
  int64_t tiles_per_matrix;
  int64_t batch_per_launch;
  bool empty;
};

// Packed batches of small matrices (xpose::PackedArgs): taken by default,
// when no launch knob asks for a tile, for a batch of dense matrices of at
// most kPackedMaxBytes each, or of at most kPackedRaggedBytes when the
// matrix is not a whole number of 64 x 64 tiles (128 x 128 for 1-byte
// elements; whole-tile matrices of that size run faster on the tiles);
// XPOSE_FLAG_PACKED asks for it for any dense matrix that fits the largest
// block, XPOSE_FLAG_NO_PACKED never.  Returns kNotPacked to fall through to
// the tile kernels.
constexpr int kNotPacked = 1;
constexpr int64_t kPackedMaxBytes = 16384, kPackedRaggedBytes = 32768;

int plan_packed(const void *out, const void *in, int64_t batch, int64_t rows,
                int64_t cols, int64_t ld_in, int64_t ld_out, int64_t stride_in,
                int64_t stride_out, int s, const xpose_opts *opts,
                Plan *plan) {
  const int flags = opts ? opts->flags : 0;
  const bool want = flags & XPOSE_FLAG_PACKED;
  const bool knobs =
      opts && (opts->layout || opts->tile_rows || opts->tile_cols ||
               opts->threads || opts->persistent || opts->occupancy ||
               opts->order ||
               opts->group_rows || opts->group_cols ||
               (flags & ~(XPOSE_FLAG_XCD_REMAP | XPOSE_FLAG_NO_XCD_REMAP |
                          XPOSE_FLAG_PACKED)));
  if (!want && (knobs || (flags & XPOSE_FLAG_NO_PACKED) || batch < 2))
    return kNotPacked;
  const int64_t m = rows * cols;  // fits: the extents were checked
  const bool dense = ld_in == cols && ld_out == rows &&
                     (batch == 1 || (stride_in == m && stride_out == m));
  int n = 0;
  const xpose::PackedKernel *table = xpose::packed_kernels(&n);
  const int largest_block = table[n - 1].block_bytes;
  const int64_t edge = s == 1 ? 128 : 64;
  const bool ragged = rows % edge || cols % edge;
  const int64_t limit = ragged ? kPackedRaggedBytes : kPackedMaxBytes;
  if (!dense || m * s > largest_block || (!want && m * s > limit))
    return want ? XPOSE_ENOTILE : kNotPacked;
  // Whole matrices per workgroup.  Where a multiple of 128 / gcd(m s, 128)
  // fits a block (the smallest such block size is taken), blocks are whole
  // cache lines and non-temporal stores pay; otherwise the smallest block
  // that holds a matrix, filled, with write-back stores.
  const int64_t mb = m * s;
  int64_t g = 128, x = mb;
  while (x) {  // gcd(mb, 128)
    const int64_t t = g % x;
    g = x;
    x = t;
  }
  const int64_t unit = 128 / g;
  int block = 0;
  for (int i = 0; i < n && !block; ++i)
    if (unit * mb <= table[i].block_bytes) block = table[i].block_bytes;
  for (int i = 0; i < n && !block; ++i)
    if (mb <= table[i].block_bytes) block = table[i].block_bytes;
  const int64_t fit = block / mb;
  const bool lines = unit <= fit;
  const int64_t per = lines ? fit / unit * unit : fit;
  const int cache =
      (opts && opts->cache)
          ? opts->cache
          : ((lines && (uintptr_t)out % 128 == 0) ? XPOSE_CACHE_NT_STORE
                                                 : XPOSE_CACHE_DEFAULT);
  const xpose::PackedKernel *k = nullptr;
  for (int i = 0; i < n && !k; ++i)
    if (table[i].elem_bytes == s && table[i].block_bytes == block &&
        table[i].cache == cache - 1)
      k = &table[i];
  if (!k) return want ? XPOSE_ENOTILE : kNotPacked;
  plan->packed = k;
  plan->elem_bytes = s;
  plan->batch = batch;
  plan->pk.out = const_cast<void *>(out);
  plan->pk.in = in;
  plan->pk.rows = (uint32_t)rows;
  plan->pk.cols = (uint32_t)cols;
  plan->pk.per_block = (uint32_t)per;
  // Rows of 64 bytes or a multiple: pad the LDS rows (see the kernel).
  plan->pk.pad = (cols * s) % 64 == 0 ? (s == 8 ? 1 : 4 / s) : 0;
  plan->tiles_per_matrix = 1;
  // At most 2^30 workgroups per launch.
  plan->batch_per_launch = per << 30;
  return XPOSE_OK;
}

int make_plan(const void *out, const void *in, int64_t batch, int64_t rows,
              int64_t cols, int64_t ld_in, int64_t ld_out, int64_t stride_in,
              int64_t stride_out, int32_t dtype, const xpose_opts *opts,
              Plan *plan) {
  memset(plan, 0, sizeof(*plan));
  const int s = elem_bytes_of(dtype);
  if (s == 0) return XPOSE_EDTYPE;
  if (batch < 0 || rows < 0 || cols < 0) return XPOSE_EINVAL;
  const int known_flags = XPOSE_FLAG_ELEMENTWISE | XPOSE_FLAG_XCD_REMAP |
                          XPOSE_FLAG_NO_XCD_REMAP | XPOSE_FLAG_DIRECT_LDS |
                          XPOSE_FLAG_ALIGN_OUT | XPOSE_FLAG_NO_ALIGN_OUT |
                          XPOSE_FLAG_TR_READ | XPOSE_FLAG_PACKED |
                          XPOSE_FLAG_NO_PACKED;
  if (opts && (opts->layout < XPOSE_LAYOUT_AUTO ||
               opts->layout > XPOSE_LAYOUT_NAIVE_WRITE ||
               (opts->flags & ~known_flags) != 0 ||
               ((opts->flags & XPOSE_FLAG_XCD_REMAP) &&
                (opts->flags & XPOSE_FLAG_NO_XCD_REMAP)) ||
               ((opts->flags & XPOSE_FLAG_ALIGN_OUT) &&
                (opts->flags & (XPOSE_FLAG_NO_ALIGN_OUT |
                                XPOSE_FLAG_ELEMENTWISE |
                                XPOSE_FLAG_DIRECT_LDS |
                                XPOSE_FLAG_TR_READ))) ||
               ((opts->flags & XPOSE_FLAG_PACKED) &&
                (opts->flags & (XPOSE_FLAG_NO_PACKED | XPOSE_FLAG_ELEMENTWISE |
                                XPOSE_FLAG_DIRECT_LDS | XPOSE_FLAG_ALIGN_OUT |
                                XPOSE_FLAG_TR_READ))) ||
               opts->cache < XPOSE_CACHE_AUTO ||
               opts->cache > XPOSE_CACHE_NT_ALL || opts->group_rows < 0 ||
               opts->group_cols < 0 || opts->threads < 0 ||
               opts->order < XPOSE_ORDER_AUTO || opts->persistent < 0 ||
               opts->persistent > 64 || opts->occupancy < -1 ||
               opts->occupancy > 64 ||
               (opts->occupancy && opts->persistent) ||
               opts->order > XPOSE_ORDER_COLUMN_BANDS ||
               opts->tile_rows < 0 || opts->tile_cols < 0))
    return XPOSE_EINVAL;
  if (batch == 0 || rows == 0 || cols == 0) {
    plan->empty = true;
    return XPOSE_OK;
  }
  if (!out || !in) return XPOSE_EINVAL;
  if (ld_in < cols || ld_out < rows) return XPOSE_EINVAL;
  if (batch > 1 && stride_in < 0) return XPOSE_EINVAL;
  if (batch == 1) stride_in = stride_out = 0;

  int64_t ext_in, ext_out;
  if (!extent(batch, rows, cols, ld_in, stride_in, &ext_in) ||
      !extent(1, cols, rows, ld_out, 0, &ext_out))
    return XPOSE_EINVAL;
  if (batch > 1) {
    // Output matrices must not overlap one another.
    if (stride_out < ext_out) return XPOSE_EINVAL;
    if (!extent(batch, cols, rows, ld_out, stride_out, &ext_out))
      return XPOSE_EINVAL;
  }
  int64_t bytes_in, bytes_out;
  if (!mul_ok(ext_in, s, &bytes_in) || !mul_ok(ext_out, s, &bytes_out))
    return XPOSE_EINVAL;

  const uintptr_t pi = (uintptr_t)in, po = (uintptr_t)out;
  if ((pi % s) || (po % s)) return XPOSE_EALIGN;
  if (pi + (uint64_t)bytes_in < pi || po + (uint64_t)bytes_out < po)
    return XPOSE_EINVAL;
  if (pi < po + (uint64_t)bytes_out && po < pi + (uint64_t)bytes_in)
    return XPOSE_EALIAS;

  // Kernel choice.
  const bool out_row128 = po % 128 == 0 && (ld_out * s) % 128 == 0 &&
                          (batch == 1 || (stride_out * s) % 128 == 0);
  {
    const int rc = plan_packed(out, in, batch, rows, cols, ld_in, ld_out,
                               stride_in, stride_out, s, opts, plan);
    if (rc != kNotPacked) return rc;
  }
  const bool small = batch > 1 && rows * cols * s <= kSmallMatrixBytes;
  int64_t call_bytes;
  const bool big = !mul_ok(2 * batch, rows * cols * s, &call_bytes) ||
                   call_bytes >= kBigCallBytes;
  const bool mid = big || call_bytes >= kMidCallBytes;
  const bool direct = opts && (opts->flags & XPOSE_FLAG_DIRECT_LDS);
  const bool tr_read = opts && (opts->flags & XPOSE_FLAG_TR_READ);
  // Line-aligned output tiles are the default where they apply, unless a
  // knob asks for something they are not built with; XPOSE_FLAG_ALIGN_OUT
  // requests them outright.
  const bool want_align = opts && (opts->flags & XPOSE_FLAG_ALIGN_OUT);
  const bool align_ok =
      want_align ||
      !(opts && ((opts->flags & (XPOSE_FLAG_NO_ALIGN_OUT |
                                 XPOSE_FLAG_ELEMENTWISE |
                                 XPOSE_FLAG_DIRECT_LDS |
                                 XPOSE_FLAG_TR_READ)) ||
                 (opts->layout && opts->layout != XPOSE_LAYOUT_SWIZZLE) ||
                 opts->persistent));
  const bool short_rows = s == 2 && rows < kShortAlignRows;
  auto near = [](int64_t pitch, int64_t target) {
    return pitch >= target - kPitchSlack && pitch <= target + kPitchSlack;
  };
  auto near_multiple = [](int64_t pitch, int64_t period) {
    const int64_t off = pitch % period;
    return off <= kPitchSlack || period - off <= kPitchSlack;
  };
  // One large matrix (not a batch): the 128 KiB tiles.
  const bool single =
      batch == 1 && rows >= kLargeMinDim && cols >= kLargeMinDim;
  const bool huge = single && (!mul_ok(2, rows * cols * s, &call_bytes) ||
                               call_bytes >= kHugeCallBytes);
  const bool large = single && (!mul_ok(2, rows * cols * s, &call_bytes) ||
                                call_bytes >= kLargeCallBytes);
  CallShape shape;
  shape.out_row128 = out_row128;
  shape.small = small;
  shape.big = big;
  shape.mid = mid;
  shape.align = want_align || (align_ok && !out_row128 && !short_rows);
  shape.single = single;
  shape.large = large;
  shape.huge = huge;
  shape.on_period = near_multiple(ld_out * s, kPitchPeriod);
  shape.slow_1k =
      near(ld_out * s, kSlowSegmentPitch) && cols > kSlowSegmentCols;
  shape.square_32k =
      near(ld_in * s, kPitchPeriod) && near(ld_out * s, kPitchPeriod);
  Default d = default_for(s, shape);
  const int layout = (opts && opts->layout) ? opts->layout : d.layout;
  plan->elem_bytes = s;
  if (layout == XPOSE_LAYOUT_NAIVE_READ || layout == XPOSE_LAYOUT_NAIVE_WRITE) {
    plan->naive = layout;
    plan->batch = batch;
    xpose::TileArgs &a = plan->args;
    a.out = const_cast<void *>(out);
    a.in = in;
    a.rows = rows;
    a.cols = cols;
    a.ld_in = ld_in;
    a.ld_out = ld_out;
    a.stride_in = stride_in;
    a.stride_out = stride_out;
    const int64_t run = layout == XPOSE_LAYOUT_NAIVE_READ ? cols : rows;
    const int64_t other = layout == XPOSE_LAYOUT_NAIVE_READ ? rows : cols;
    plan->tiles_per_matrix = (run + 255) / 256 * other;
    return XPOSE_OK;
  }
  int n = 0;
  const xpose::TileKernel *table = xpose::tile_kernels(&n);
  const bool explicit_tile = opts && (opts->tile_rows || opts->tile_cols);
  // Kernel with the resolved knobs.  any_tile: the default tile shape is not
  // built with the requested layout, flags or workgroup size, so take the
  // first built shape (table order) that is.
  auto lookup = [&](const Default &dd, bool align, bool any_tile) {
    int tr = dd.tile_rows, tc = dd.tile_cols, nt = dd.threads;
    if (explicit_tile) {
      tr = opts->tile_rows;
      tc = opts->tile_cols;
      nt = 0;  // any built workgroup size; the largest is preferred
    }
    if (any_tile) nt = 0;
    if (opts && opts->threads) nt = opts->threads;
    // An explicit cache policy must be built; otherwise the default one is
    // preferred, then any policy built for the requested kernel.
    const int want[3] = {(opts && opts->cache) ? opts->cache : dd.cache, kWB,
                         kNT};
    const int tries = (opts && opts->cache) ? 1 : 3;
    const xpose::TileKernel *k = nullptr;
    for (int t = 0; t < tries && !k; ++t)
      for (int i = 0; i < n; ++i) {
        const xpose::TileKernel &c = table[i];
        if (c.elem_bytes != s || c.layout != layout ||
            c.cache != want[t] - 1 || c.direct_lds != direct ||
            c.aligned_out != align || c.tr_read != tr_read)
          continue;
        if (any_tile) {
          if (!k && (!nt || c.threads == nt)) k = &c;
        } else if (c.tile_rows == tr && c.tile_cols == tc &&
                   (nt ? c.threads == nt : (!k || c.threads > k->threads))) {
          k = &c;
        }
      }
    return k;
  };
  const xpose::TileKernel *k = lookup(d, d.align_out || want_align, false);
  if (!k && d.align_out && !want_align) {
    // The explicit tile, threads or cache exist only as ordinary tiles:
    // fall back to those, with their own defaults for the other knobs.
    shape.align = false;
    d = default_for(s, shape);
    k = lookup(d, false, false);
  }
  if (!k && !explicit_tile) k = lookup(d, d.align_out || want_align, true);
  if (!k) return XPOSE_ENOTILE;
  const int tr = k->tile_rows, tc = k->tile_cols;
  // persistent: n workgroups per compute unit walking the tiles; for
  // line-aligned tiles, column strips of n tile rows per workgroup.
  const int persistent = opts ? opts->persistent : 0;
  if (persistent && (k->aligned_out ? k->launch_strip == nullptr
                                     : k->launch_persistent == nullptr))
    return XPOSE_ENOTILE;

  // Line-aligned output tiles shift each segment back by up to 128 / s - 1
  // rows, so one more partial tile row may be needed to reach the last row.
  const int64_t tiles_r =
      (rows + (k->aligned_out ? 128 / s - 1 : 0) + tr - 1) / tr;
  const int64_t tiles_c = (cols + tc - 1) / tc;
  if (tiles_r > 0x7fffffff || tiles_c > 0x7fffffff) return XPOSE_EINVAL;
  int64_t tiles;
  if (!mul_ok(tiles_r, tiles_c, &tiles) || tiles > 0x7fffffff)
    return XPOSE_EINVAL;

  // Interior tiles take 128-bit accesses at any alignment, except that
  // direct global->LDS loads need every row start 4-byte aligned.
  bool vec = true;
  if (s < 4 && k->direct_lds) {
    const int64_t q = 4 / s;  // elements per dword
    vec = (pi % 4 == 0) && (ld_in % q == 0) &&
          (batch == 1 || stride_in % q == 0);
  }
  if (opts && (opts->flags & XPOSE_FLAG_ELEMENTWISE)) vec = false;

  int64_t group_r = (opts && opts->group_rows) ? opts->group_rows : d.group_rows;
  int64_t group_c = (opts && opts->group_cols) ? opts->group_cols : d.group_cols;
  const int order = (opts && opts->order) ? opts->order : d.order;
  if (order == XPOSE_ORDER_COLUMN_BANDS && !(opts && opts->group_cols) &&
      group_c > 0 && group_c < tiles_c) {
    // Default bands: equal widths of at most d.group_cols tile columns
    // (12345 x 6789 fp32: two bands of 54 and 53, 2-3% faster than 64 + 43).
    const int64_t nb = (tiles_c + group_c - 1) / group_c;
    group_c = (tiles_c + nb - 1) / nb;
  }
  if (group_r > tiles_r) group_r = tiles_r;
  if (group_c > tiles_c || group_c == 0) group_c = tiles_c;
  int xcd = d.xcd_remap;
  if (opts && (opts->flags & XPOSE_FLAG_XCD_REMAP)) xcd = 1;
  if (opts && (opts->flags & XPOSE_FLAG_NO_XCD_REMAP)) xcd = 0;

  // The default cap belongs to the default tile and order: it applies when
  // the resolved kernel has the default shape and workgroup size and the
  // tile order is the default one.
  int occupancy = (opts && opts->occupancy) ? opts->occupancy : 0;
  if (!occupancy && !persistent && tr == d.tile_rows && tc == d.tile_cols &&
      k->threads == d.threads && (!opts || !opts->order || opts->order == d.order))
    occupancy = d.occupancy;
  plan->kernel = k;
  plan->persistent = persistent;
  plan->occupancy = occupancy > 0 ? occupancy : 0;
  plan->batch = batch;
  plan->tiles_per_matrix = tiles;
  plan->batch_per_launch = 0x7fffffff / tiles;
  xpose::TileArgs &a = plan->args;
  a.out = const_cast<void *>(out);
  a.in = in;
  a.rows = rows;
  a.cols = cols;
  a.ld_in = ld_in;
  a.ld_out = ld_out;
  a.stride_in = stride_in;
  a.stride_out = stride_out;
  a.tiles_r = (uint32_t)tiles_r;
  a.tiles_c = (uint32_t)tiles_c;
  a.batch_first = 0;
  a.vec_ok = vec ? 1 : 0;
  a.order = order;
  a.group_rows = (uint32_t)group_r;
  a.group_cols = (uint32_t)group_c;
  a.xcd_remap = xcd;
  return XPOSE_OK;
}

// Compute units of the current device, looked up once per device.
hipError_t compute_units(int *out) {
  static std::atomic<int> cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *out = c;
      return hipSuccess;
    }
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (n <= 0) return hipErrorInvalidDevice;
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  *out = n;
  return hipSuccess;
}

// LDS bytes per compute unit and per workgroup of the current device,
// looked up once per device.
hipError_t device_lds(int *per_cu, int *per_block) {
  static std::atomic<int> cache_cu[64], cache_block[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64) {
    const int c = cache_cu[dev].load(std::memory_order_relaxed);
    const int b = cache_block[dev].load(std::memory_order_relaxed);
    if (c > 0 && b > 0) {
      *per_cu = c;
      *per_block = b;
      return hipSuccess;
    }
  }
  int c = 0, b = 0;
  e = hipDeviceGetAttribute(
      &c, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&b, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess) return e;
  if (c <= 0 || b <= 0) return hipErrorInvalidDevice;
  if (dev >= 0 && dev < 64) {
    cache_cu[dev].store(c, std::memory_order_relaxed);
    cache_block[dev].store(b, std::memory_order_relaxed);
  }
  *per_cu = c;
  *per_block = b;
  return hipSuccess;
}

// Dynamic LDS to reserve so that at most `occupancy` workgroups of a kernel
// with `static_lds` bytes of its own share one compute unit: each workgroup
// then holds floor(per_cu / occupancy) bytes, rounded down to 1 KiB (so
// `occupancy` of them fit and one more does not, for occupancy <= 64), but
// never more than a workgroup may hold.  0 where the kernel's own LDS
// already caps it that low.
uint32_t reserve_lds(int occupancy, int static_lds, int per_cu,
                     int per_block) {
  if (occupancy <= 0) return 0;
  int64_t total = (int64_t)per_cu / occupancy / 1024 * 1024;
  if (total > per_block) total = per_block;
  return total > static_lds ? (uint32_t)(total - static_lds) : 0;
}

int run_plan(Plan &plan, void *stream) {
  if (plan.empty) return XPOSE_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (plan.packed) {
    const int64_t mb = (int64_t)plan.pk.rows * plan.pk.cols * plan.elem_bytes;
    for (int64_t b0 = 0; b0 < plan.batch; b0 += plan.batch_per_launch) {
      xpose::PackedArgs a = plan.pk;
      a.count = plan.batch - b0;
      if (a.count > plan.batch_per_launch) a.count = plan.batch_per_launch;
      a.in = static_cast<const char *>(a.in) + b0 * mb;
      a.out = static_cast<char *>(a.out) + b0 * mb;
      const uint32_t grid =
          (uint32_t)((a.count + a.per_block - 1) / a.per_block);
      const hipError_t e = plan.packed->launch(a, grid, st);
      if (e != hipSuccess) return hip_fail(e);
    }
    return XPOSE_OK;
  }
  if (plan.naive) {
    const hipError_t e =
        xpose::launch_naive(plan.args, plan.batch, plan.elem_bytes,
                            plan.naive == XPOSE_LAYOUT_NAIVE_READ, st);
    return e == hipSuccess ? XPOSE_OK : hip_fail(e);
  }
  uint32_t lds_extra = 0;
  if (plan.occupancy) {
    int per_cu = 0, per_block = 0;
    const hipError_t e = device_lds(&per_cu, &per_block);
    if (e != hipSuccess) return hip_fail(e);
    lds_extra = reserve_lds(plan.occupancy, plan.kernel->lds_bytes, per_cu,
                            per_block);
  }
  for (int64_t b0 = 0; b0 < plan.batch; b0 += plan.batch_per_launch) {
    int64_t nb = plan.batch - b0;
    if (nb > plan.batch_per_launch) nb = plan.batch_per_launch;
    // batch_first is a 32-bit field: advance the base pointers instead once
    // the batch index would not fit.
    xpose::TileArgs a = plan.args;
    const int s = plan.kernel->elem_bytes;
    a.in = static_cast<const char *>(a.in) + b0 * a.stride_in * s;
    a.out = static_cast<char *>(a.out) + b0 * a.stride_out * s;
    const uint32_t ntiles = (uint32_t)(nb * plan.tiles_per_matrix);
    hipError_t e;
    if (plan.persistent && plan.kernel->aligned_out) {
      const uint32_t seg = (uint32_t)plan.persistent;
      const uint32_t nseg = (a.tiles_r + seg - 1) / seg;
      const int64_t grid = nb * (int64_t)nseg * a.tiles_c;  // <= nb * tiles
      e = plan.kernel->launch_strip(a, seg, nseg, (uint32_t)grid, st);
    } else if (plan.persistent) {
      int cus = 0;
      e = compute_units(&cus);
      if (e != hipSuccess) return hip_fail(e);
      // A multiple of 8, so each tile stays on the XCD the remap gives it;
      // no more than the tiles need.
      int64_t grid = (int64_t)plan.persistent * cus;
      const int64_t cap = ((int64_t)ntiles + 7) / 8 * 8;
      if (grid > cap) grid = cap;
      grid = (grid + 7) / 8 * 8;
      e = plan.kernel->launch_persistent(a, ntiles, (uint32_t)grid, st);
    } else {
      e = plan.kernel->launch(a, ntiles, lds_extra, st);
    }
    if (e != hipSuccess) return hip_fail(e);
  }
  return XPOSE_OK;
}

}  // namespace

int xpose::record_hip_error(hipError_t e) { return hip_fail(e); }

extern "C" {

int xpose_batched_ex(void *out, const void *in, int64_t batch, int64_t rows,
                     int64_t cols, int64_t ld_in, int64_t ld_out,
                     int64_t stride_in, int64_t stride_out, int32_t dtype,
                     const xpose_opts *opts, void *stream) {
  Plan plan;
  const int rc = make_plan(out, in, batch, rows, cols, ld_in, ld_out,
                           stride_in, stride_out, dtype, opts, &plan);
  if (rc != XPOSE_OK) return rc;
  return run_plan(plan, stream);
}

int xpose_batched(void *out, const void *in, int64_t batch, int64_t rows,
                  int64_t cols, int64_t ld_in, int64_t ld_out,
                  int64_t stride_in, int64_t stride_out, int32_t dtype,
                  void *stream) {
  return xpose_batched_ex(out, in, batch, rows, cols, ld_in, ld_out,
                          stride_in, stride_out, dtype, nullptr, stream);
}

int xpose_2d(void *out, const void *in, int64_t rows, int64_t cols,
             int64_t ld_in, int64_t ld_out, int32_t dtype, void *stream) {
  return xpose_batched_ex(out, in, 1, rows, cols, ld_in, ld_out, 0, 0, dtype,
                          nullptr, stream);
}

int xpose_2d_ex(void *out, const void *in, int64_t rows, int64_t cols,
                int64_t ld_in, int64_t ld_out, int32_t dtype,
                const xpose_opts *opts, void *stream) {
  return xpose_batched_ex(out, in, 1, rows, cols, ld_in, ld_out, 0, 0, dtype,
                          opts, stream);
}

int xpose_plan(const void *out, const void *in, int64_t batch, int64_t rows,
               int64_t cols, int64_t ld_in, int64_t ld_out, int64_t stride_in,
               int64_t stride_out, int32_t dtype, const xpose_opts *opts,
               xpose_plan_info *info) {
  Plan plan;
  const int rc = make_plan(out, in, batch, rows, cols, ld_in, ld_out,
                           stride_in, stride_out, dtype, opts, &plan);
  if (info) {
    memset(info, 0, sizeof(*info));
    if (rc == XPOSE_OK && !plan.empty && plan.packed) {
      const int64_t per = plan.pk.per_block;
      info->tile_rows = (int32_t)plan.pk.rows;
      info->tile_cols = (int32_t)plan.pk.cols;
      info->threads = plan.packed->threads;
      info->lds_bytes = plan.packed->block_bytes + plan.packed->block_bytes / 8;
      info->vector_path = 1;
      info->tiles = (plan.batch + per - 1) / per;
      info->launches = (int32_t)((plan.batch + plan.batch_per_launch - 1) /
                                 plan.batch_per_launch);
      info->cache = plan.packed->cache + 1;
      info->packed = (int32_t)per;
    } else if (rc == XPOSE_OK && !plan.empty && plan.naive) {
      const bool rd = plan.naive == XPOSE_LAYOUT_NAIVE_READ;
      info->layout = plan.naive;
      info->tile_rows = rd ? 1 : 256;
      info->tile_cols = rd ? 256 : 1;
      info->threads = 256;
      info->tiles = plan.tiles_per_matrix * plan.batch;
      info->launches = 1;
      info->cache = XPOSE_CACHE_DEFAULT;
    } else if (rc == XPOSE_OK && !plan.empty) {
      info->layout = plan.kernel->layout;
      info->tile_rows = plan.kernel->tile_rows;
      info->tile_cols = plan.kernel->tile_cols;
      info->threads = plan.kernel->threads;
      info->lds_bytes = plan.persistent && plan.kernel->aligned_out
                            ? plan.kernel->strip_lds_bytes
                            : plan.kernel->lds_bytes;
      info->vector_path = plan.args.vec_ok;
      info->tiles = plan.tiles_per_matrix * plan.batch;
      info->launches = (int32_t)((plan.batch + plan.batch_per_launch - 1) /
                                 plan.batch_per_launch);
      info->cache = plan.kernel->cache + 1;
      info->group_rows = (int32_t)plan.args.group_rows;
      info->group_cols = (int32_t)plan.args.group_cols;
      info->order = plan.args.order;
      info->persistent = plan.persistent;
      info->direct_lds = plan.kernel->direct_lds ? 1 : 0;
      info->aligned_out = plan.kernel->aligned_out ? 1 : 0;
      info->tr_read = plan.kernel->tr_read ? 1 : 0;
      info->xcd_remap = plan.args.xcd_remap;
      info->occupancy = plan.occupancy;
    }
  }
  return rc;
}

int xpose_copy_ex(void *dst, const void *src, int64_t bytes,
                  const xpose_copy_opts *opts, void *stream) {
  if (bytes < 0) return XPOSE_EINVAL;
  if (opts && (opts->threads < 0 || opts->unroll < 0 ||
               opts->cache < XPOSE_CACHE_AUTO ||
               opts->cache > XPOSE_CACHE_NT_ALL))
    return XPOSE_EINVAL;
  const int threads = (opts && opts->threads) ? opts->threads : kDefaultCopyThreads;
  const int unroll = (opts && opts->unroll) ? opts->unroll : kDefaultCopyUnroll;
  const int cache = (opts && opts->cache) ? opts->cache : kDefaultCopyCache;
  int n = 0;
  const xpose::CopyKernel *table = xpose::copy_kernels(&n);
  const xpose::CopyKernel *k = nullptr;
  for (int i = 0; i < n; ++i)
    if (table[i].threads == threads && table[i].unroll == unroll &&
        table[i].cache == cache - 1)
      k = &table[i];
  if (!k) return XPOSE_ENOTILE;
  if (bytes == 0) return XPOSE_OK;
  if (!dst || !src) return XPOSE_EINVAL;
  const uintptr_t d = (uintptr_t)dst, s = (uintptr_t)src;
  if (d + (uint64_t)bytes < d || s + (uint64_t)bytes < s) return XPOSE_EINVAL;
  if (d < s + (uint64_t)bytes && s < d + (uint64_t)bytes) return XPOSE_EALIAS;
  const hipError_t e = xpose::launch_copy(*k, dst, src, bytes,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? XPOSE_OK : hip_fail(e);
}

int xpose_copy(void *dst, const void *src, int64_t bytes, void *stream) {
  return xpose_copy_ex(dst, src, bytes, nullptr, stream);
}

int xpose_lds_probe(uint64_t *cycles_out, const int32_t *lane_bytes,
                    int32_t width, int32_t is_write, int32_t iters,
                    void *stream) {
  if (!cycles_out || !lane_bytes) return XPOSE_EINVAL;
  if (width != 4 && width != 8 && width != 16) return XPOSE_EINVAL;
  if (iters < 1 || iters > (1 << 20)) return XPOSE_EINVAL;
  if ((uintptr_t)cycles_out % 8) return XPOSE_EALIGN;
  for (int i = 0; i < 64; ++i)
    if (lane_bytes[i] < 0 || lane_bytes[i] >= 16384 || lane_bytes[i] % width)
      return XPOSE_EINVAL;
  const hipError_t e =
      xpose::launch_lds_probe(cycles_out, lane_bytes, width, is_write != 0,
                              iters, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? XPOSE_OK : hip_fail(e);
}

int xpose_last_hip_error(void) { return g_last_hip_error; }

const char *xpose_strerror(int code) {
  switch (code) {
    case XPOSE_OK: return "success";
    case XPOSE_EINVAL: return "invalid argument";
    case XPOSE_EALIAS: return "input and output ranges overlap";
    case XPOSE_EDTYPE: return "unknown dtype";
    case XPOSE_EHIP: return "HIP runtime error";
    case XPOSE_EALIGN: return "pointer not aligned to the element size";
    case XPOSE_ENOTILE: return "no kernel built for the requested options";
    case XPOSE_EWORKSPACE:
      return "workspace (or the 64 MiB no-allocation scratch) too small "
             "for the requested split of k";
    default: return "unknown status code";
  }
}

}  // extern "C"
