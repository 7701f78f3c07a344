// Internal interface between the SGEMM front end (sgemm_api.cpp) and its
// gfx950 kernels (sgemm_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xpose {

// Tiled SGEMM, C = alpha * A * B + beta * C (fp32, row-major; pitches in
// floats).  Grid = tiles_m * tiles_n workgroups of tile_m x 128 blocks of C.
struct SgemmArgs {
  const float *a, *b;
  float *c;
  int64_t m, n, k, lda, ldb, ldc;
  float alpha, beta;
  uint32_t tiles_m, tiles_n;
  uint32_t group_m;   // block order: group height in block rows (>= 1)
  int32_t xcd_remap;  // 1: one contiguous range of blocks per XCD
  // 1: whole tiles are loaded with buffer loads (a descriptor per k step
  // and 32-bit lane offsets); needs 16-byte tile loads and 128 * lda and
  // 32 * ldb floats to fit in a 31-bit byte offset
  int32_t buf_ok;
  // 1: edge blocks and ragged last k steps also use buffer loads, with
  // descriptor extents clipped to the matrix (needs buf_ok, and k and n
  // multiples of 4 so no 16-byte vector straddles an extent's end)
  int32_t edge_buf;
  // Split of the k range: with splits > 1 the grid is splits copies of the
  // tiles_m * tiles_n blocks; copy z sums k in [z * split_k, min(k, (z + 1)
  // * split_k)) and stores the raw sums (no alpha, beta or C) into the m x n
  // partial matrix at partial + z * m * n (pitch n).  split_k is a multiple
  // of the k step.
  int32_t splits;
  int64_t split_k;
  float *partial;
};

// C = alpha * (sum over z < splits of partial z) + beta * C, the partial
// matrices m x n with pitch n, summed in the order z = 0, 1, ...; with beta
// == 0 C is not read.
struct SgemmReduceArgs {
  const float *partial;
  float *c;
  int64_t m, n, ldc;
  int32_t splits;
  float alpha, beta;
};
hipError_t launch_sgemm_reduce(const SgemmReduceArgs &r, hipStream_t s);

// The partial sums of xpose_sgemm_noalloc live in a file-scope device array
// of kSgemmScratchBytes in sgemm_kernels.hip, one per GPU for the life of
// the process.  sgemm_scratch() gives its address on the current device:
// looked up with hipGetSymbolAddress on a device's first call (with that
// device current) and kept per device.  It allocates nothing.
constexpr int64_t kSgemmScratchBytes = (int64_t)64 << 20;
hipError_t sgemm_scratch(void **ptr);

struct SgemmKernel {
  int bk, layout, as_stride, lds_bytes, threads;
  bool vec;    // 16-byte tile loads (a, b 16-byte aligned, lda, ldb % 4 == 0)
  int stages;  // LDS buffers: 1 = two barriers per k step, 2 = one
  int tile_m;  // rows of C per workgroup (64, 128 or 256; 128 columns)
  hipError_t (*launch)(const SgemmArgs &, uint32_t grid, hipStream_t);
  // Built for matrices of whole blocks only: m and n multiples of the
  // block, k of the k step, buffer loads and the one-descriptor C tail
  // allowed.  No edge code at all.
  bool whole = false;
};

// Every compiled SGEMM kernel; *count receives the table length.
const SgemmKernel *sgemm_kernels(int *count);

// Records a failed HIP call for xpose_last_hip_error (kept by the transpose
// front end, xpose_api.cpp) and returns XPOSE_EHIP.
int record_hip_error(hipError_t e);

}  // namespace xpose
