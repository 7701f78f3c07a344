// Internal interface between the C-ABI front end (xpose_api.cpp) and the
// gfx950 kernels (xpose_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xpose {

// LDS tile layouts; values match xpose_layout in include/xpose.h.
enum Layout : int { kUnpadded = 1, kPad1 = 2, kSwizzle = 3 };

// Arguments of one tiled-transpose launch.  Sizes, pitches and strides are
// in elements; the grid is tiles_r * tiles_c * batch_count workgroups and
// workgroup g handles batch entry batch_first + g / (tiles_r * tiles_c).
struct TileArgs {
  void *out;
  const void *in;
  int64_t rows, cols, ld_in, ld_out, stride_in, stride_out;
  uint32_t tiles_r, tiles_c;
  uint32_t batch_first;
  int32_t vec_ok;  // 1: interior tiles may use 128-bit global accesses
};

// One compiled tile kernel.
struct TileKernel {
  int elem_bytes, tile_rows, tile_cols, threads, layout, lds_bytes;
  hipError_t (*launch)(const TileArgs &, uint32_t grid, hipStream_t);
};

// Every compiled tile kernel; *count receives the table length.
const TileKernel *tile_kernels(int *count);

// 128-bit device-to-device copy (byte path for unaligned ends).
hipError_t launch_copy(void *dst, const void *src, int64_t bytes,
                       hipStream_t stream);

// LDS bank microbenchmark; lane_bytes is a host array of 64 byte offsets.
hipError_t launch_lds_probe(uint64_t *out, const int32_t *lane_bytes,
                            int width, bool is_write, int iters,
                            hipStream_t stream);

}  // namespace xpose
