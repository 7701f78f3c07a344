/*
 * xpose_sgemm -- the tiled single-precision GEMM whose transposed LDS store
 * is the second bank-conflict workload of the pages, for MI355X (gfx950).
 *
 * C ABI of libxpose.so (the same library as include/xpose.h, whose status
 * codes and error rules apply here too).
 *
 * What is computed.  Row-major fp32 matrices A (m x k, row pitch lda),
 * B (k x n, pitch ldb) and C (m x n, pitch ldc); for i in [0, m), j in [0, n):
 *
 *     C[i*ldc + j] = alpha * sum_{l < k} A[i*lda + l] * B[l*ldb + j]
 *                    + beta * C[i*ldc + j]
 *
 * the operation of the SGEMM in "Padded Shared Memory: Eliminating Bank
 * Conflicts" (the kernel listed under "The Fix Is One Constant", measured at
 * m = n = k = 4096 in "Mechanics").  With beta == 0, C is write-only: it is
 * not read, so NaN or uninitialised contents do not reach the result (the
 * pages' kernel always reads C; where C is finite the two agree).  A and B
 * are always read when k > 0, also with alpha == 0, so NaN or Inf there
 * reach C as alpha * NaN.  Elements of C outside the m x n region (pitch
 * padding) are never written.
 *
 * How.  Each workgroup computes a 128 x 128 (or 256 x 128) block of C in
 * steps of bk along k.  Per step it loads A's tile with 16-byte row reads and stores
 * it TRANSPOSED in LDS (As[l][i], so the product reads consecutive i), the
 * store the pages show to be bank-conflicted when As's row stride is a
 * multiple of the bank count ("How Shared Memory Is Addressed"); B's bk x 128
 * tile goes to LDS as it is.  The products run on the matrix cores
 * (v_mfma_f32_32x32x2_f32: fp32 operands, fp32 accumulation).  The sum over
 * l is therefore taken in a different order than a sequential loop; every
 * element lies within (k + 3) * 2^-24 * (|alpha| * sum_l |A[i][l] B[l][j]|
 * + |beta * C[i][j]|) of the exact value (the standard bound of an fp32 dot
 * product of length k, plus the scaling), for operands and partial sums in
 * the normal range.  Integer-valued inputs whose partial sums stay below
 * 2^24 are reproduced exactly.
 *
 * Memory and streams.  a, b and c are DEVICE pointers on the current HIP
 * device, owned by the caller, 4-byte aligned.  16-byte aligned a and b with
 * lda and ldb multiples of 4 let the tile loads use 16-byte accesses; other
 * alignments take 4-byte loads.  Calls are asynchronous on `stream` (NULL =
 * the null stream), never synchronise, never allocate and keep no state.
 * C's byte range must not overlap A's or B's (XPOSE_EALIAS); A and B may
 * overlap each other.
 *
 * Split of k.  A product with few blocks of C (1024 x 1024 is 64 blocks of
 * 128 x 128, for 256 compute units) leaves most of the chip idle.  Given a
 * WORKSPACE (xpose_sgemm_ws), the call may split k into S slices of whole k
 * steps: S copies of the block grid run at once, copy z storing its slice's
 * raw sums sum_{l in slice z} A[i][l] B[l][j] into the z-th m x n partial
 * matrix of the workspace (pitch n), and a second kernel on the same stream
 * writes C = alpha * (P_0 + P_1 + ... + P_{S-1}) + beta * C, adding the
 * partials in the order z = 0, 1, ... (so results are deterministic and
 * repeat bit for bit).  The error bound above holds unchanged (a split only
 * regroups the same sum).  The workspace holds S * m * n floats; it is
 * written and read by the call's kernels only, so it may be reused as soon
 * as the call's work on the stream has finished, and two calls that share a
 * workspace must not overlap in time.  xpose_sgemm and xpose_sgemm_ex have
 * no workspace and never split.
 *
 * Errors (validated on the host before anything is launched):
 *   XPOSE_EINVAL  negative m, n or k; lda < max(k, 1), ldb < max(n, 1) or
 *                 ldc < max(n, 1); a NULL pointer that the call would use;
 *                 an extent overflowing 64 bits; unknown option values
 *   XPOSE_EALIGN  a pointer not 4-byte aligned
 *   XPOSE_EALIAS  C overlaps A or B
 *   XPOSE_ENOTILE no kernel built for the requested options
 *   XPOSE_EWORKSPACE  an explicit split (split_k >= 2) with a workspace
 *                 smaller than the split needs (or none: xpose_sgemm_ex)
 *   XPOSE_EHIP    the launch failed (xpose_last_hip_error())
 * A workspace that the call uses must be 4-byte aligned (XPOSE_EALIGN; 16
 * bytes lets the final sum use 16-byte accesses) and must not overlap A, B
 * or C (XPOSE_EALIAS); workspace_bytes < 0 is XPOSE_EINVAL.
 * m == 0 or n == 0 is a successful no-op (pointers may then be NULL);
 * k == 0 sets C = beta * C (a and b are not used and may be NULL).
 */
#ifndef XPOSE_SGEMM_H
#define XPOSE_SGEMM_H

#include <stdint.h>

#include "xpose.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Layout of the transposed A tile in LDS (As, bk rows of 128 floats).  All
 * give identical results; they differ only in bank conflicts of the
 * transposed store ("How Shared Memory Is Addressed", "The Fix Is One
 * Constant"). */
typedef enum xpose_as_layout {
  XPOSE_AS_AUTO = 0,     /* library default: XPOSE_AS_PADDED with 128-row
                            blocks; when no layout, k step, block height or
                            second buffer is asked for and the shape is large
                            and round (m a multiple of 256, n of 128,
                            k >= 1024, and (m / 256) (n / 128) a multiple of
                            512: whole rounds of two 512-thread workgroups
                            on each of MI355X's 256 compute units),
                            XPOSE_AS_SWIZZLE with 256-row blocks, measured
                            2.5-4% faster there                               */
  XPOSE_AS_UNPADDED = 1, /* row stride 128 floats, a multiple of the bank
                            count: the store is (min(bk, 32) / 4)-way
                            conflicted on gfx950's 32-bank, 32-lane 4-byte
                            LDS accesses                                      */
  XPOSE_AS_PADDED = 2,   /* row stride 128 + 32 / min(bk, 32) floats: the
                            smallest pad that spreads one half-wave's stores
                            over all 32 banks (the pages' (32 / BK) % 8 for
                            bk = 8, 16, 32; A's tile is read in strips of at
                            most 32 columns)                                 */
  XPOSE_AS_SWIZZLE = 3   /* row stride 128, the row index of each element
                            XOR-permuted by a multiple of 128 / min(bk, 32)
                            chosen from its k: conflict-free without
                            padding                                          */
} xpose_as_layout;

/* Option flags of xpose_sgemm_ex. */
enum {
  XPOSE_SGEMM_NO_XCD_REMAP = 1, /* keep the hardware's round-robin
                                   assignment of workgroups to XCDs instead
                                   of one contiguous range of blocks each    */
  XPOSE_SGEMM_DOUBLE_BUFFER = 2, /* two LDS buffers alternate, so one barrier
                                   per k step suffices instead of the two of
                                   the pages' loop (the remedy "What Could Be
                                   Improved" points to: both barriers stall
                                   the block).  Measured no faster on gfx950,
                                   where three or four other workgroups per
                                   compute unit fill the barrier stalls      */
  XPOSE_SGEMM_NO_BUFFER_LOADS = 4 /* load whole tiles like edge tiles, with
                                   bounds-checked 16-byte global loads,
                                   instead of buffer loads (a descriptor per
                                   k step, 32-bit lane offsets), which are
                                   the default where the pitches allow them
                                   (lda <= 2^31 / (4 (tile_m + 1)), i.e.
                                   4161790 or 2089014, and ldb <= 8323580)   */
};

/* Optional knobs (zero-initialise for defaults).  Every choice gives the
 * same result up to the summation order within a bk step (bk changes the
 * grouping of the sum). */
typedef struct xpose_sgemm_opts {
  int32_t layout;  /* xpose_as_layout                                         */
  int32_t bk;      /* k step per LDS stage: 0 = default (16), 8, 16, 32 or 64 */
  int32_t group_m; /* block order: groups of group_m block rows, walked
                      block-column by block-column; 0 = default (8)          */
  int32_t flags;   /* XPOSE_SGEMM_*                                           */
  int32_t tile_m;  /* rows of C per workgroup: 0 = default (128, or 256
                      or 64 under the rule of XPOSE_AS_AUTO), 64 (2 waves;
                      k step 16, one LDS buffer), 128 (4 waves) or 256 (8
                      waves; k steps 16 and 32, one LDS buffer); blocks are
                      128 columns wide                                       */
  int32_t split_k; /* k slices: 0 = the library's choice (with a workspace,
                      a split where the grid of blocks is too small to fill
                      the chip, as many slices as the workspace holds at
                      most; without one, none), 1 = no split, 2..64 = k
                      split into slices of ceil(k / split_k) rounded up to
                      whole k steps (so at most split_k slices; fewer when k
                      is short, none when one slice covers k)              */
} xpose_sgemm_opts;

/* What xpose_sgemm_plan reports about the kernel a call would launch. */
typedef struct xpose_sgemm_info {
  int32_t layout;       /* resolved xpose_as_layout                           */
  int32_t bk;           /* k step                                             */
  int32_t as_stride;    /* As row stride in floats                            */
  int32_t lds_bytes;    /* LDS per workgroup (all buffers)                    */
  int32_t threads;      /* threads per workgroup                              */
  int32_t tile_m;       /* rows of C per workgroup                            */
  int32_t tile_n;       /* columns of C per workgroup                         */
  int32_t vector_loads; /* 1: 16-byte tile loads; 0: 4-byte loads             */
  int32_t group_m;      /* resolved block-order group height                  */
  int32_t xcd_remap;    /* 1 if blocks are remapped per XCD                   */
  int32_t stages;       /* LDS buffers per workgroup (1 or 2)                 */
  int32_t buffer_loads; /* 1: whole tiles are read with buffer loads          */
  int64_t tiles;        /* workgroups launched                                */
  int32_t whole_matrix; /* 1: the kernel built for whole blocks only (no edge
                           code), taken when m and n are multiples of the
                           block, k of the k step, buffer loads are allowed,
                           ldc <= 2^29 / tile_m and one LDS buffer is used;
                           built for k step 16                               */
  int32_t edge_buffer_loads; /* 1: edge blocks and a ragged last k step read
                           with buffer loads too, their descriptors clipped
                           to the matrix (buffer loads allowed, k and n
                           multiples of 4); 0: those take bounds-checked
                           global loads                                      */
  int32_t splits;       /* k slices the call takes (1: no split)             */
  int64_t split_len;    /* k per slice (the last may be shorter); k if none  */
  int64_t workspace_bytes;  /* workspace the call uses: splits * m * n * 4,
                           0 without a split                                */
  int64_t workspace_wanted; /* workspace the library's split choice for this
                           shape and these options would use given enough
                           (an explicit split_k: that split's); 0 if it
                           would not split                                  */
} xpose_sgemm_info;

/* C = alpha * A * B + beta * C with the default kernel. */
int xpose_sgemm(int64_t m, int64_t n, int64_t k, float alpha, const float *a,
                int64_t lda, const float *b, int64_t ldb, float beta,
                float *c, int64_t ldc, void *stream);

/* xpose_sgemm with explicit knobs (opts may be NULL): the As layout
 * ablation of the pages' padded-store fix. */
int xpose_sgemm_ex(int64_t m, int64_t n, int64_t k, float alpha,
                   const float *a, int64_t lda, const float *b, int64_t ldb,
                   float beta, float *c, int64_t ldc,
                   const xpose_sgemm_opts *opts, void *stream);

/* Host-only: validate an xpose_sgemm_ex call and report the kernel it
 * would launch, without touching the GPU (pointers are compared and checked
 * for alignment, never dereferenced).  Returns the status the call would
 * return; `info` may be NULL. */
int xpose_sgemm_plan(int64_t m, int64_t n, int64_t k, const float *a,
                     int64_t lda, const float *b, int64_t ldb, const float *c,
                     int64_t ldc, const xpose_sgemm_opts *opts,
                     xpose_sgemm_info *info);

/* xpose_sgemm_ex with a caller-owned DEVICE workspace of workspace_bytes
 * (on the current device) for the partial sums of a split of k (see "Split
 * of k" above; `workspace` may be NULL when workspace_bytes is 0).  With
 * opts->split_k == 0 the library splits where the block grid is small, into
 * as many slices as its rule picks and the workspace holds; the workspace
 * is only touched when the call splits.  Two kernels are enqueued on
 * `stream` when it does (the split product, then the sum), one otherwise.
 * The split is for grids of blocks too small to occupy MI355X's 256
 * compute units. */
int xpose_sgemm_ws(int64_t m, int64_t n, int64_t k, float alpha,
                   const float *a, int64_t lda, const float *b, int64_t ldb,
                   float beta, float *c, int64_t ldc,
                   const xpose_sgemm_opts *opts, void *workspace,
                   int64_t workspace_bytes, void *stream);

/* Size of the device scratch array of xpose_sgemm_noalloc, per GPU. */
#define XPOSE_SGEMM_SCRATCH_BYTES ((int64_t)64 << 20)

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * as xpose_sgemm_ws, with the workspace replaced by the library's own
 * device array of XPOSE_SGEMM_SCRATCH_BYTES (64 MiB), a file-scope device
 * array of the library that each GPU it runs on holds until the process
 * ends; the call allocates nothing, and neither does any library routine it
 * calls.  A split of k the library chooses (opts->split_k == 0) is shrunk
 * to what the scratch holds (none when fewer than two m x n planes fit,
 * i.e. for m n > 8 Mi); an explicit split_k >= 2 whose partials (splits *
 * m * n * 4 bytes) exceed it is rejected with XPOSE_EWORKSPACE before
 * anything is launched.  xpose_sgemm_plan_ws with workspace_bytes =
 * XPOSE_SGEMM_SCRATCH_BYTES (and any non-NULL, 4-byte aligned workspace
 * address that overlaps none of A, B and C) reports the split it takes.
 *
 * Every call on one GPU shares that GPU's array, and it keeps the last
 * call's contents (nothing in it needs to start at zero: each split writes
 * all of its partials before summing them).  Calls that overlap in time on
 * one GPU -- on different streams, or from different threads -- race on the
 * array and give wrong results; serialise them (one stream, or events).  On
 * a device's first call the array's device address is looked up (a HIP
 * symbol query, XPOSE_EHIP if it fails) and kept. */
int xpose_sgemm_noalloc(int64_t m, int64_t n, int64_t k, float alpha,
                        const float *a, int64_t lda, const float *b,
                        int64_t ldb, float beta, float *c, int64_t ldc,
                        const xpose_sgemm_opts *opts, void *stream);

/* Host-only counterpart of xpose_sgemm_ws, as xpose_sgemm_plan is of
 * xpose_sgemm_ex (the workspace too is compared, never dereferenced).
 * With workspace NULL and workspace_bytes 0 it serves as the size query:
 * info->workspace_wanted is what to allocate.  On XPOSE_EWORKSPACE (from
 * either plan call) `info` is zeroed except for workspace_wanted. */
int xpose_sgemm_plan_ws(int64_t m, int64_t n, int64_t k, const float *a,
                        int64_t lda, const float *b, int64_t ldb,
                        const float *c, int64_t ldc,
                        const xpose_sgemm_opts *opts, const void *workspace,
                        int64_t workspace_bytes, xpose_sgemm_info *info);

#ifdef __cplusplus
}
#endif

#endif /* XPOSE_SGEMM_H */
