/*
 * xpose -- out-of-place 2-D and batched matrix transpose for MI355X (gfx950).
 *
 * C ABI of libxpose.so.  Every entry point takes plain pointers and sizes and
 * returns an int status (0 = success, negative = XPOSE_E* code); nothing
 * throws across this boundary.
 *
 * What is computed.  For b in [0, batch), i in [0, rows), j in [0, cols):
 *
 *     out[b*stride_out + j*ld_out + i] = in[b*stride_in + i*ld_in + j]
 *
 * i.e. every input matrix (rows x cols, row-major, row pitch ld_in) lands
 * transposed in the output (cols x rows, row-major, row pitch ld_out).  This
 * is the operation of the tiled transpose in "Shared memory and the bank
 * conflict" (section "Turn the tile around on chip": a block reads a tile in
 * rows, turns it around on chip and writes it in rows), in the non-square
 * form out[col * height + row] = in[row * width + col] of "Shared-memory
 * tiling and bank conflicts" (section "Reference summary"), extended with
 * row pitches and a batch stride.  Sizes, pitches and strides are counted in
 * ELEMENTS.  Values are moved as raw bits: no rounding, no NaN
 * canonicalisation, subnormals and -0 preserved.  Output elements outside
 * each output matrix's cols x rows region (pitch padding, gaps between batch
 * entries) are never written.
 *
 * Memory and streams.  `in` and `out` are DEVICE pointers on the current HIP
 * device, owned by the caller, aligned to the element size.  `stream` is a
 * hipStream_t (NULL = the null stream).  Calls are asynchronous on `stream`:
 * they enqueue kernels and return; they never synchronise, never allocate,
 * never copy to or from the host, and keep no state between calls except the
 * per-thread last HIP error (xpose_last_hip_error).  The caller must keep
 * both buffers alive until the stream has run the work.  Input and output
 * byte ranges must not overlap (in-place transpose is not supported: the
 * pages only show out-of-place kernels).
 *
 * Errors.  Arguments are validated on the host before anything is launched;
 * an invalid call returns a negative code and enqueues nothing.  A shape
 * with batch, rows or cols equal to zero is a successful no-op (pointers may
 * then be NULL).
 */
#ifndef XPOSE_H
#define XPOSE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  Only the size matters: 4, 2, 2, 1 and 8 bytes. */
typedef enum xpose_dtype {
  XPOSE_F32 = 0,
  XPOSE_F16 = 1,
  XPOSE_BF16 = 2,
  XPOSE_U8 = 3,
  XPOSE_F64 = 4
} xpose_dtype;

/* Status codes. */
enum {
  XPOSE_OK = 0,
  XPOSE_EINVAL = -1, /* NULL pointer with a non-empty shape, negative size,
                        pitch or stride too small, size overflow, bad opts  */
  XPOSE_EALIAS = -2, /* input and output byte ranges overlap               */
  XPOSE_EDTYPE = -3, /* unknown dtype                                       */
  XPOSE_EHIP = -4,   /* a HIP call failed; see xpose_last_hip_error()       */
  XPOSE_EALIGN = -5, /* a pointer is not aligned to the element size        */
  XPOSE_ENOTILE = -6, /* no kernel is built for the combination xpose_opts
                        asks for (tile shape, layout, flags, workgroup size,
                        cache policy)                                       */
  XPOSE_EWORKSPACE = -7 /* the split of k an SGEMM call asks for needs more
                        workspace than the call has (include/xpose_sgemm.h) */
};

/* LDS tile layouts (the row stride of the on-chip tile).  A padded or a
 * swizzled row is the remedy the pages give for conflicted column reads
 * ("Shared-memory tiling and bank conflicts", section "Reference summary");
 * the one-word pad is the 33-word row of "Shared Memory and Bank Conflicts",
 * section "the classic case".  All layouts give identical results; they
 * differ only in LDS bank conflicts. */
typedef enum xpose_layout {
  XPOSE_LAYOUT_AUTO = 0,     /* library default (the measured best)          */
  XPOSE_LAYOUT_UNPADDED = 1, /* row stride = tile width (conflicted column read) */
  XPOSE_LAYOUT_PAD1 = 2,     /* row stride = tile width + one 32-bit word     */
  XPOSE_LAYOUT_SWIZZLE = 3,  /* 16-byte chunks XOR-permuted per row            */
  /* Not tiled, for the ablation only: one element per thread, no LDS, so one
   * of the two global sides is uncoalesced (tile, cache and order options
   * are ignored). */
  XPOSE_LAYOUT_NAIVE_READ = 4,  /* threads along input rows: reads coalesced */
  XPOSE_LAYOUT_NAIVE_WRITE = 5  /* threads along input columns: writes coalesced */
} xpose_layout;

/* Cache policy of the global accesses.  The data is touched exactly once,
 * so marking it non-temporal can keep it from displacing other lines. */
typedef enum xpose_cache {
  XPOSE_CACHE_AUTO = 0,       /* library default for the case; where the
                                 requested kernel is not built with it, any
                                 policy it is built with                    */
  XPOSE_CACHE_DEFAULT = 1,    /* plain loads and stores                     */
  XPOSE_CACHE_NT_STORE = 2,   /* non-temporal stores                        */
  XPOSE_CACHE_NT_ALL = 3      /* non-temporal loads and stores              */
} xpose_cache;

/* Order in which workgroups walk the tiles (results are identical). */
typedef enum xpose_order {
  XPOSE_ORDER_AUTO = 0,        /* library default                          */
  XPOSE_ORDER_SUPER_TILES = 1, /* group_rows x group_cols super-tiles      */
  XPOSE_ORDER_DIAGONAL = 2,    /* consecutive workgroups step diagonally:
                                  tile row g mod R, column (g/R + row) mod C */
  XPOSE_ORDER_COLUMN_BANDS = 3 /* bands of group_cols tile columns, left to
                                  right; inside a band tile rows top to
                                  bottom, each row's tiles left to right    */
} xpose_order;

/* Option flags for xpose_batched_ex. */
enum {
  XPOSE_FLAG_ELEMENTWISE = 1, /* force the element-wise edge path everywhere */
  XPOSE_FLAG_XCD_REMAP = 2,   /* give each XCD one contiguous range of tiles */
  XPOSE_FLAG_NO_XCD_REMAP = 4, /* the opposite, overriding the default       */
  XPOSE_FLAG_DIRECT_LDS = 8,   /* interior tiles load straight into LDS
                                  (global_load_lds_dwordx4): 4- and 8-byte
                                  elements, unpadded or swizzled layout, or
                                  1- and 2-byte elements together with
                                  XPOSE_FLAG_TR_READ                         */
  XPOSE_FLAG_ALIGN_OUT = 16,   /* line-aligned output tiles (2-, 4- and
                                  8-byte elements, swizzled layout): each
                                  output row's segment is shifted to start on
                                  a 128-byte line, so stores are whole lines
                                  even when output rows are not line-aligned.
                                  The default for such output rows; with this
                                  flag, a call whose element size, tile,
                                  workgroup size or cache policy has no such
                                  kernel returns XPOSE_ENOTILE                */
  XPOSE_FLAG_NO_ALIGN_OUT = 32, /* ordinary tiles even where line-aligned
                                  output tiles are the default               */
  XPOSE_FLAG_TR_READ = 64,     /* 1- and 2-byte elements, swizzled layout: the
                                  LDS tile holds the input rows unchanged and
                                  the column walk uses gfx950's LDS transpose
                                  reads (ds_read_b64_tr_b16 / _tr_b8) instead
                                  of packing rows in registers.  Not combined
                                  with XPOSE_FLAG_ALIGN_OUT (XPOSE_EINVAL);
                                  sizes without such a kernel return
                                  XPOSE_ENOTILE                              */
  XPOSE_FLAG_PACKED = 128,     /* packed batch of small matrices: each
                                  workgroup moves whole dense matrices
                                  (ld_in = cols, ld_out = rows, strides =
                                  rows * cols) as one contiguous block per
                                  side.  The default, when no other knob is
                                  set, for batches of dense matrices of at
                                  most 16 KiB, or 32 KiB when the matrix is
                                  not a whole number of 64 x 64 tiles (128 x
                                  128 for 1-byte elements); with this flag,
                                  for any dense matrix of at most 32 KiB,
                                  a single one too (else XPOSE_ENOTILE).  Not
                                  combined with the tile flags (XPOSE_EINVAL)*/
  XPOSE_FLAG_NO_PACKED = 256   /* tiles even where the packed kernel is the
                                  default                                     */
};

/* Optional knobs for the measured ablation.  Zero-initialise for defaults.
 * Every choice gives bit-identical results. */
typedef struct xpose_opts {
  int32_t layout;     /* xpose_layout                                        */
  int32_t tile_rows;  /* 0 = default (if the default shape is not built with
                         the requested layout, flags or workgroup size: the
                         first built shape that is); else one of the built
                         tile shapes                                         */
  int32_t tile_cols;  /* 0 = default                                         */
  int32_t flags;      /* XPOSE_FLAG_*                                        */
  int32_t cache;      /* xpose_cache                                         */
  int32_t group_rows; /* tile order: workgroups walk super-tiles of
                         group_rows x group_cols tiles, super-tiles
                         row-major, tile rows fastest inside one;
                         0 = default                                         */
  int32_t group_cols; /* 0 = default                                         */
  int32_t threads;    /* workgroup size of the tile kernel; 0 = the default
                         (with an explicit tile: the largest one built)     */
  int32_t order;      /* xpose_order                                         */
  int32_t persistent; /* 0 = one workgroup per tile (default); n > 0 = n
                         persistent workgroups per compute unit, each
                         walking many tiles with two LDS buffers so the
                         next tile's loads overlap the current tile's
                         stores (swizzled layout only).  For line-aligned
                         output tiles (4- and 8-byte elements; built for
                         fp32 64x64, 128x64, 128x32 and fp64 32x32, 64x32,
                         non-temporal stores): column strips instead, each
                         workgroup walking n (1..64) tile rows of one tile
                         column top to bottom with its input rows in an
                         LDS ring of twice the tile height, so the one-line
                         halo is not read again; order and group_* are
                         ignored there                                      */
  int32_t occupancy;  /* tile kernels: at most this many workgroups of the
                         launch share one compute unit (1..64), enforced by
                         reserving LDS that is never touched; 0 = the
                         library default for the case; -1 = no cap.  Not
                         combined with persistent (XPOSE_EINVAL)             */
} xpose_opts;

/* What xpose_plan reports about the kernel a call would launch. */
typedef struct xpose_plan_info {
  int32_t layout;      /* resolved xpose_layout                              */
  int32_t tile_rows;   /* tile shape in elements                             */
  int32_t tile_cols;
  int32_t threads;     /* threads per workgroup                              */
  int32_t lds_bytes;   /* LDS per workgroup                                  */
  int32_t vector_path; /* 1: interior tiles use 128-bit global accesses (at
                          any alignment; direct global->LDS loads need
                          4-byte aligned input rows);
                          0: every tile takes the element-wise path          */
  int64_t tiles;       /* workgroups over the whole batch                    */
  int32_t launches;    /* kernel launches the call will enqueue              */
  int32_t cache;       /* resolved xpose_cache                               */
  int32_t group_rows;  /* resolved super-tile height in tiles                 */
  int32_t group_cols;  /* resolved super-tile width in tiles                  */
  int32_t xcd_remap;   /* 1 if tiles are remapped per XCD                    */
  int32_t order;       /* resolved xpose_order                               */
  int32_t persistent;  /* persistent workgroups per compute unit (line-
                          aligned column strips: tile rows per workgroup),
                          0 = none                                          */
  int32_t direct_lds;  /* 1 if interior tiles load straight into LDS         */
  int32_t aligned_out; /* 1 if output segments are shifted onto lines        */
  int32_t tr_read;     /* 1 if the column walk uses LDS transpose reads      */
  int32_t packed;      /* packed small-matrix kernel: matrices per workgroup
                          (tile_rows x tile_cols = one matrix, tiles =
                          workgroups); 0 = tile kernels                      */
  int32_t occupancy;   /* resolved cap on workgroups per compute unit (0 =
                          none: as many as registers and LDS allow)          */
} xpose_plan_info;

/* Knobs of the copy yardstick (zero-initialise for defaults). */
typedef struct xpose_copy_opts {
  int32_t threads; /* workgroup size; 0 = default                           */
  int32_t unroll;  /* 16-byte vectors per lane; 0 = default                 */
  int32_t cache;   /* xpose_cache                                           */
  int32_t reserved;
} xpose_copy_opts;

/* 2-D transpose of one rows x cols matrix: the definition above with
 * batch = 1.  ld_in >= cols, ld_out >= rows.  dtype is an xpose_dtype. */
int xpose_2d(void *out, const void *in, int64_t rows, int64_t cols,
             int64_t ld_in, int64_t ld_out, int32_t dtype, void *stream);

/* xpose_2d with an explicit LDS layout, tile shape and launch knobs (opts
 * may be NULL, which is exactly xpose_2d).  This is the per-call switch for
 * the record "Shared memory and the bank conflict" asks for (section "What
 * to record": the same tile with the 32-word row and with the 33-word row,
 * the copy and the best naive kernel, timed the same way): opts->layout
 * selects the unpadded row, the one-word pad, the swizzle or a naive kernel,
 * opts->tile_rows / tile_cols the tile.  Arguments, layout, ownership and
 * errors as xpose_2d, plus XPOSE_EINVAL for an invalid opts field and
 * XPOSE_ENOTILE for a combination no kernel is built for.  Results are
 * bit-identical for every choice. */
int xpose_2d_ex(void *out, const void *in, int64_t rows, int64_t cols,
                int64_t ld_in, int64_t ld_out, int32_t dtype,
                const xpose_opts *opts, void *stream);

/* Batched transpose: `batch` independent matrices, input matrix b starting
 * stride_in elements after matrix b-1, output matrix b stride_out elements
 * after output b-1.  Output matrices must not overlap each other:
 * stride_out >= (cols-1)*ld_out + rows when batch > 1.  stride_in >= 0
 * (input matrices may overlap or coincide; they are only read). */
int xpose_batched(void *out, const void *in, int64_t batch, int64_t rows,
                  int64_t cols, int64_t ld_in, int64_t ld_out,
                  int64_t stride_in, int64_t stride_out, int32_t dtype,
                  void *stream);

/* xpose_batched with explicit layout and tile choice (opts may be NULL).
 * Used for the layout ablation; results are identical for every choice. */
int xpose_batched_ex(void *out, const void *in, int64_t batch, int64_t rows,
                     int64_t cols, int64_t ld_in, int64_t ld_out,
                     int64_t stride_in, int64_t stride_out, int32_t dtype,
                     const xpose_opts *opts, void *stream);

/* Host-only: validate a call and report the kernel it would launch, without
 * touching the GPU.  Returns the same status the call would return (pointers
 * are only compared and checked for alignment, never dereferenced).  `info`
 * may be NULL. */
int xpose_plan(const void *out, const void *in, int64_t batch, int64_t rows,
               int64_t cols, int64_t ld_in, int64_t ld_out, int64_t stride_in,
               int64_t stride_out, int32_t dtype, const xpose_opts *opts,
               xpose_plan_info *info);

/* Device-to-device copy of `bytes` bytes with 128-bit loads and stores: the
 * practical bandwidth roofline the transpose is measured against (the
 * "copy" yardstick of "Shared memory and the bank conflict", sections "Turn
 * the tile around on chip" and "What to record").  Same pointer, stream and
 * error rules as the transposes; the ranges must not overlap. */
int xpose_copy(void *dst, const void *src, int64_t bytes, void *stream);

/* xpose_copy with an explicit copy kernel (opts may be NULL): the copy
 * variants are measured so the yardstick is the fastest copy built.
 * Returns XPOSE_ENOTILE if no kernel matches the requested knobs. */
int xpose_copy_ex(void *dst, const void *src, int64_t bytes,
                  const xpose_copy_opts *opts, void *stream);

/* LDS bank microbenchmark: one 64-lane wavefront repeatedly issues one LDS
 * instruction in which lane l accesses byte address lane_bytes[l] (host
 * array of 64 entries, each a multiple of `width`, below 16384) with
 * `width` = 4, 8 or 16 bytes, as a read (is_write = 0) or a write (1).
 * Each of `iters` iterations issues 8 such instructions.  The wave's elapsed
 * shader-clock cycles are written to cycles_out[0] (a DEVICE buffer of two
 * uint64), a checksum of what was read to cycles_out[1].  Used to measure
 * the gfx950 bank model that the tile layouts are designed against
 * ("Shared Memory and Bank Conflicts", section "the wave size
 * complication": the conflict group on 64-lane hardware must be measured,
 * not assumed). */
int xpose_lds_probe(uint64_t *cycles_out, const int32_t *lane_bytes,
                    int32_t width, int32_t is_write, int32_t iters,
                    void *stream);

/* hipError_t of the most recent failing HIP call made by this thread inside
 * the library (0 if none). */
int xpose_last_hip_error(void);

/* Static string describing a status code (never NULL). */
const char *xpose_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* XPOSE_H */
