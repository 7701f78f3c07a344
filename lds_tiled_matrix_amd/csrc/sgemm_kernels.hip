// gfx950 kernel of the tiled SGEMM, C = alpha * A * B + beta * C (fp32,
// row-major), with A's tile stored transposed in LDS: the second workload of
// "Padded Shared Memory: Eliminating Bank Conflicts", where the transposed
// store is the bank-conflict site and padding As's row stride is the fix
// ("How Shared Memory Is Addressed", "The Fix Is One Constant").  Here the
// dense contraction runs on the matrix cores (v_mfma_f32_32x32x2_f32, fp32
// in and out); the LDS staging keeps the pages' structure: 16-byte row loads
// of A, scalar transposed stores into As, 16-byte copies of B into Bs, a
// barrier, the inner products, a second barrier (or, with two LDS buffers,
// one barrier per step).  The layouts and lane maps are in sgemm_lanes.h.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "sgemm_lanes.h"
#include "sgemm_kernels.h"

// The no-allocation entry point's partial sums: 64 MiB per GPU, held until
// the process ends.  In host code this name is only a stand-in for the
// device array, never a device address: host code takes the address from
// sgemm_scratch() below and passes that to kernels.
static __device__ __align__(256) float
    scratch[xpose::kSgemmScratchBytes / sizeof(float)];

namespace xpose {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Fourth word of a raw buffer descriptor on gfx9-family GPUs: 32-bit data
// format, no swizzle, no index stride.
constexpr int kBufferWord3 = 0x00020000;

// One 16-byte vector of row `row` (of `nrows`) starting at column `col` (of
// `ncols`) of a row-major matrix with pitch `ld`: a 16-byte load where the
// vector is whole and VEC allows it, else 4-byte loads of the elements that
// exist, zero elsewhere (zeros contribute nothing to the products).
template <bool VEC>
__device__ inline f32x4 load_vec(const float *base, int64_t row, int64_t col,
                                 int64_t nrows, int64_t ncols, int64_t ld) {
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  if (row >= nrows) return v;
  const float *p = base + row * ld + col;
  if (VEC && col + 4 <= ncols) return *reinterpret_cast<const f32x4 *>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (col + e < ncols) v[e] = p[e];
  return v;
}

// The same pointer in every lane, made visibly uniform so the buffer
// descriptor built from it lives in scalar registers (without this the
// compiler may wrap each buffer load in a loop over distinct descriptors).
__device__ inline float *uniform(const float *p) {
  return reinterpret_cast<float *>(uniform_bits(
      reinterpret_cast<uint64_t>(p),
      [](int x) { return __builtin_amdgcn_readfirstlane(x); }));
}

// STAGES = 1 is the pages' loop: stage the step's tiles, barrier, products,
// barrier.  STAGES = 2 keeps two LDS buffers: the next step's tiles are
// staged into the other buffer right after this step's products, so one
// barrier per step separates the writes of one buffer from the reads of
// the other.  Either way the next step's global loads are issued before
// this step's products and land in registers while the matrix cores run.
//
// WHOLE kernels serve calls whose every block is whole (the host checks m, n,
// k, the pitches and alignments): the same loop and tail without the edge
// code, which measured about 1% faster than keeping it in the kernel.
template <int BK, int L, bool VEC, int STAGES, int BM = 128, bool WHOLE = false>
__global__ __launch_bounds__(2 * BM) __attribute__((amdgpu_waves_per_eu(
    SgemmTile<BK, L, BM>::waves_per_simd(STAGES)))) void
xpose_sgemm_kernel(SgemmArgs args) {
  using T = SgemmTile<BK, L, BM>;
  static_assert(!WHOLE || (VEC && STAGES == 1), "whole-matrix kernels");
  __shared__ __attribute__((aligned(16))) float As[STAGES * T::AS_FLOATS];
  __shared__ __attribute__((aligned(16))) float Bs[STAGES * T::BS_FLOATS];

  // A split of k is the same product over a slice of k, stored raw into
  // its own partial matrix: shift A and B to the slice, shorten k, and
  // point the epilogue at the partial with alpha = 1, beta = 0.
  SgemmArgs a = args;
  uint32_t block = blockIdx.x;
  if (a.splits > 1) {
    const uint32_t tiles = a.tiles_m * a.tiles_n;
    const uint32_t z = block / tiles;
    block -= z * tiles;
    const int64_t k0 = (int64_t)z * a.split_k;
    a.a += k0;
    a.b += k0 * a.ldb;
    a.k = a.k - k0 < a.split_k ? a.k - k0 : a.split_k;
    a.c = a.partial + (int64_t)z * a.m * a.n;
    a.ldc = a.n;
    a.alpha = 1.f;
    a.beta = 0.f;
  }

  const int t = threadIdx.x, q = t & 63, w = t >> 6;
  uint32_t bm, bn;
  sgemm_block(block, a.tiles_m, a.tiles_n, a.group_m, a.xcd_remap, bm, bn);
  const int64_t m0 = (int64_t)bm * T::BM, n0 = (int64_t)bn * T::BN;
  f32x4 ra[T::A_PASSES], rb[T::B_PASSES];
  // Buffer loads of one whole k step's tiles: the A and B tiles each get a
  // descriptor (scalar base and extent), the lanes 32-bit byte offsets,
  // which saves the 64-bit address arithmetic of global loads.
  auto load_whole = [&](int64_t k0) __attribute__((always_inline)) {
    const float *ab = uniform(a.a + m0 * a.lda + k0);
    const float *bb = uniform(a.b + k0 * a.ldb + n0);
    const __amdgpu_buffer_rsrc_t ra_d = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(ab), 0, (int)(((T::BM - 1) * a.lda + BK) * 4),
        kBufferWord3);
    const __amdgpu_buffer_rsrc_t rb_d = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(bb), 0, (int)(((BK - 1) * a.ldb + T::BN) * 4),
        kBufferWord3);
#pragma unroll
    for (int p = 0; p < T::A_PASSES; ++p)
      ra[p] = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     ra_d, (int)((T::a_row(t, p) * a.lda + T::a_col(t, p)) * 4),
                     0, 0));
#pragma unroll
    for (int p = 0; p < T::B_PASSES; ++p)
      rb[p] = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     rb_d, (int)((T::b_row(t, p) * a.ldb + T::b_col(t)) * 4),
                     0, 0));
  };
  // Edge blocks, ragged k, and pitches or alignments that rule out buffer
  // loads: every 16-byte vector checked against the matrix.
  auto load_checked = [&](int64_t k0) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < T::A_PASSES; ++p)
      ra[p] = load_vec<VEC>(a.a, m0 + T::a_row(t, p), k0 + T::a_col(t, p), a.m,
                            a.k, a.lda);
#pragma unroll
    for (int p = 0; p < T::B_PASSES; ++p)
      rb[p] = load_vec<VEC>(a.b, k0 + T::b_row(t, p), n0 + T::b_col(t), a.k,
                            a.n, a.ldb);
  };
  // A's vectors go into As transposed, one 4-byte store per element: the
  // store whose banks the layout decides.  B's rows are copied as they are.
  auto stage = [&](int buf) __attribute__((always_inline)) {
    float *as = As + buf * T::AS_FLOATS;
    float *bs = Bs + buf * T::BS_FLOATS;
#pragma unroll
    for (int p = 0; p < T::A_PASSES; ++p) {
      const int i = T::a_row(t, p), l = T::a_col(t, p);
#pragma unroll
      for (int e = 0; e < 4; ++e) as[T::as_index(l + e, i)] = ra[p][e];
    }
#pragma unroll
    for (int p = 0; p < T::B_PASSES; ++p)
      *reinterpret_cast<f32x4 *>(&bs[T::bs_index(T::b_row(t, p), T::b_col(t))]) =
          rb[p];
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[x][y][r] = 0.f;

  const int wr = T::wave_row(w), wc = T::wave_col(w);
  const int half = q >> 5, lane32 = q & 31;
  auto products = [&](int buf) __attribute__((always_inline)) {
    const float *as = As + buf * T::AS_FLOATS;
    const float *bs = Bs + buf * T::BS_FLOATS;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 2) {
      const int l = kk + half;
      const float a0 = as[T::as_index(l, wr + lane32)];
      const float a1 = as[T::as_index(l, wr + 32 + lane32)];
      const float b0 = bs[T::bs_index(l, wc + lane32)];
      const float b1 = bs[T::bs_index(l, wc + 32 + lane32)];
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
    }
  };

  // The k loop, over one of the two loaders.  Blocks wholly inside C with
  // k a multiple of the k step and buffer loads allowed run the loop with
  // buffer loads only: no per-step choice of loader and no edge code inside
  // the loop (at 4096^3, 140 against 138 TFLOP/s with the choice made in
  // every step).  The lambdas are forced inline: an outlined one would keep
  // the captured tiles and accumulators in scratch memory.
  auto k_loop = [&](auto load) __attribute__((always_inline)) {
    if (a.k > 0) {
      load(0);
      stage(0);
      __syncthreads();
    }
    int buf = 0;
    for (int64_t k0 = 0; k0 < a.k; k0 += BK) {
      const bool more = k0 + BK < a.k;
      if (more) load(k0 + BK);
      products(buf);
      if (STAGES == 1) {
        __syncthreads();
        if (more) {
          stage(0);
          __syncthreads();
        }
      } else {
        if (more) stage(buf ^ 1);
        __syncthreads();
        buf ^= 1;
      }
    }
  };
  // Every block, whole or at an edge, where the host set edge_buf (buffer
  // loads allowed, k and n multiples of 4): the same buffer loads with each
  // descriptor's extent clipped to the matrix (for whole blocks and steps
  // the clip is the tile itself).  A
  // load past the extent returns zero without touching memory: A's rows at
  // or past m and the last valid row's columns at or past k, B's rows at or
  // past k and the last valid row's columns at or past n.  With k and n
  // multiples of 4 no 16-byte vector straddles an extent's end.  A's columns
  // at or past k in the other rows read the next row or pitch padding
  // (inside A), and are zeroed after the load, since padding may hold NaN
  // and B's zero rows would not cancel it.  B's columns at or past n and
  // A's rows past m only reach C entries that are never stored.
  const int rows_a = a.m - m0 < T::BM ? (int)(a.m - m0) : T::BM;
  const int cols_b = a.n - n0 < T::BN ? (int)(a.n - n0) : T::BN;
  auto load_clipped = [&](int64_t k0) __attribute__((always_inline)) {
    const int kk = a.k - k0 < BK ? (int)(a.k - k0) : BK;
    const float *ab = uniform(a.a + m0 * a.lda + k0);
    const float *bb = uniform(a.b + k0 * a.ldb + n0);
    const __amdgpu_buffer_rsrc_t ra_d = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(ab), 0, (int)(((rows_a - 1) * a.lda + kk) * 4),
        kBufferWord3);
    const __amdgpu_buffer_rsrc_t rb_d = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(bb), 0, (int)(((kk - 1) * a.ldb + cols_b) * 4),
        kBufferWord3);
#pragma unroll
    for (int p = 0; p < T::A_PASSES; ++p) {
      ra[p] = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     ra_d, (int)((T::a_row(t, p) * a.lda + T::a_col(t, p)) * 4),
                     0, 0));
      if (kk < BK) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (T::a_col(t, p) + e >= kk) ra[p][e] = 0.f;
      }
    }
#pragma unroll
    for (int p = 0; p < T::B_PASSES; ++p)
      rb[p] = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     rb_d, (int)((T::b_row(t, p) * a.ldb + T::b_col(t)) * 4),
                     0, 0));
  };
  // Whole blocks with a ragged k take buffer loads for every whole k step
  // and checked loads for the last, partial one.
  auto load_ragged_k = [&](int64_t k0) __attribute__((always_inline)) {
    if (k0 + BK <= a.k)
      load_whole(k0);
    else
      load_checked(k0);
  };
  if constexpr (WHOLE) {
    k_loop(load_whole);
  } else if (VEC && a.edge_buf) {
    k_loop(load_clipped);
  } else if (VEC && a.buf_ok && m0 + T::BM <= a.m && n0 + T::BN <= a.n) {
    if (a.k % BK == 0)
      k_loop(load_whole);
    else
      k_loop(load_ragged_k);
  } else {
    k_loop(load_checked);
  }

  // C = alpha * acc + beta * C; with beta == 0 C is not read.  32 lanes
  // cover 32 consecutive columns of one row per store.  When the grid is one
  // round of workgroups every block reaches this tail at the same time, so
  // it is not hidden behind other blocks' products.  Whole blocks with a
  // pitch that keeps the block within 31-bit byte offsets therefore go
  // through one buffer descriptor: each row's offset is a uniform scalar,
  // each lane's a single register, and all 32 C values of one 32-row half
  // are loaded before the first is used (one memory round trip per half
  // instead of one per element).
  if (WHOLE || (m0 + T::BM <= a.m && n0 + T::BN <= a.n &&
                a.ldc <= ((int64_t)1 << 29) / T::BM)) {
    const float *cb = uniform(a.c + m0 * a.ldc + n0);
    const __amdgpu_buffer_rsrc_t c_d = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(cb), 0,
        (int)(((T::BM - 1) * a.ldc + T::BN) * 4), kBufferWord3);
    const int lane_off =
        (int)(((wr + T::acc_row(q, 0)) * a.ldc + wc + lane32) * 4);
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      float old[2][16];
      if (a.beta != 0.f) {
#pragma unroll
        for (int y = 0; y < 2; ++y)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            old[y][r] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(
                           c_d, lane_off + 128 * y,
                           (int)((32 * x + T::acc_row(0, r)) * a.ldc * 4), 0));
      }
#pragma unroll
      for (int y = 0; y < 2; ++y)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = a.alpha * acc[x][y][r];
          if (a.beta != 0.f) v = fmaf(a.beta, old[y][r], v);
          __builtin_amdgcn_raw_buffer_store_b32(
              __builtin_bit_cast(uint32_t, v), c_d, lane_off + 128 * y,
              (int)((32 * x + T::acc_row(0, r)) * a.ldc * 4), 0);
        }
    }
    return;
  }
  if constexpr (!WHOLE) {
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 2; ++y) {
      const int64_t j = n0 + wc + 32 * y + lane32;
      if (j >= a.n) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t i = m0 + wr + 32 * x + T::acc_row(q, r);
        if (i >= a.m) continue;
        float *p = a.c + i * a.ldc + j;
        float v = a.alpha * acc[x][y][r];
        if (a.beta != 0.f) v = fmaf(a.beta, *p, v);
        *p = v;
      }
    }
  }
}

template <int BK, int L, bool VEC, int STAGES, int BM, bool WHOLE = false>
hipError_t launch_sgemm(const SgemmArgs &a, uint32_t grid, hipStream_t s) {
  SgemmArgs copy = a;
  void *args[] = {&copy};
  return hipLaunchKernel(
      reinterpret_cast<const void *>(
          &xpose_sgemm_kernel<BK, L, VEC, STAGES, BM, WHOLE>),
      dim3(grid), dim3(SgemmTile<BK, L, BM>::NT), args, 0, s);
}

#define XPOSE_SGEMM(BK, L, VEC, ST, BM)                                      \
  SgemmKernel {                                                              \
    BK, L, SgemmTile<BK, L, BM>::AS_STRIDE,                                  \
        ST * SgemmTile<BK, L, BM>::LDS_BYTES, SgemmTile<BK, L, BM>::NT, VEC, \
        ST, BM, &launch_sgemm<BK, L, VEC, ST, BM>                            \
  }
#define XPOSE_SGEMM_L(BK, L, ST, BM)                                         \
  XPOSE_SGEMM(BK, L, true, ST, BM), XPOSE_SGEMM(BK, L, false, ST, BM)
#define XPOSE_SGEMM_WHOLE(BK, L, BM)                                         \
  SgemmKernel {                                                              \
    BK, L, SgemmTile<BK, L, BM>::AS_STRIDE, SgemmTile<BK, L, BM>::LDS_BYTES,  \
        SgemmTile<BK, L, BM>::NT, true, 1, BM,                               \
        &launch_sgemm<BK, L, true, 1, BM, true>, true                        \
  }
#define XPOSE_SGEMM_BK(BK, ST, BM)                                           \
  XPOSE_SGEMM_L(BK, kAsUnpadded, ST, BM), XPOSE_SGEMM_L(BK, kAsPadded, ST, BM), \
      XPOSE_SGEMM_L(BK, kAsSwizzle, ST, BM)

// 128-row blocks for every k step and buffer count; 256-row blocks (8
// waves) for the k steps whose B tile covers every lane (16 and 32), one
// LDS buffer; 64-row blocks (2 waves: finer grids where 128-row blocks
// leave compute units idle) for k step 16, one LDS buffer; whole-matrix
// twins of the k-step-16 kernels.
const SgemmKernel kSgemmKernels[] = {
    XPOSE_SGEMM_BK(8, 1, 128),  XPOSE_SGEMM_BK(16, 1, 128),
    XPOSE_SGEMM_BK(32, 1, 128), XPOSE_SGEMM_BK(64, 1, 128),
    XPOSE_SGEMM_BK(8, 2, 128),  XPOSE_SGEMM_BK(16, 2, 128),
    XPOSE_SGEMM_BK(32, 2, 128), XPOSE_SGEMM_BK(64, 2, 128),
    XPOSE_SGEMM_BK(16, 1, 256), XPOSE_SGEMM_BK(32, 1, 256),
    XPOSE_SGEMM_BK(16, 1, 64),
    // whole-matrix twins of the k-step-16 kernels, every layout and height
    XPOSE_SGEMM_WHOLE(16, kAsUnpadded, 128), XPOSE_SGEMM_WHOLE(16, kAsPadded, 128),
    XPOSE_SGEMM_WHOLE(16, kAsSwizzle, 128), XPOSE_SGEMM_WHOLE(16, kAsUnpadded, 256),
    XPOSE_SGEMM_WHOLE(16, kAsPadded, 256), XPOSE_SGEMM_WHOLE(16, kAsSwizzle, 256),
    XPOSE_SGEMM_WHOLE(16, kAsUnpadded, 64), XPOSE_SGEMM_WHOLE(16, kAsPadded, 64),
    XPOSE_SGEMM_WHOLE(16, kAsSwizzle, 64)};

// The sum of the split partials, 4 consecutive elements of a row per lane
// where n is a multiple of 4 and C's rows are 16-byte aligned, else one.
// A grid-stride loop over the m x n elements; the partials are read once
// and C read (beta != 0) and written once.  The planes are read kGroup at a
// time, every load of a group issued before the first add (lanes past the
// last plane reread plane z0, in bounds, and do not add it), and added in
// plane order z = 0, 1, ..., so the sum is the same as a plain loop's.
constexpr int kReduceGroup = 8;
template <bool VEC4>
__global__ __launch_bounds__(256) void xpose_sgemm_reduce_kernel(
    SgemmReduceArgs r) {
  using V = typename std::conditional<VEC4, f32x4, float>::type;
  const int64_t per_row = VEC4 ? r.n / 4 : r.n;
  const int64_t total = r.m * per_row, plane = r.m * r.n;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < total;
       v += step) {
    const int64_t i = v / per_row, j = (v - i * per_row) * (VEC4 ? 4 : 1);
    const float *p = r.partial + i * r.n + j;
    float *c = r.c + i * r.ldc + j;
    V s = *reinterpret_cast<const V *>(p);
    for (int z0 = 1; z0 < r.splits; z0 += kReduceGroup) {
      V t[kReduceGroup];
#pragma unroll
      for (int u = 0; u < kReduceGroup; ++u) {
        const int z = z0 + u < r.splits ? z0 + u : z0;
        t[u] = *reinterpret_cast<const V *>(p + z * plane);
      }
#pragma unroll
      for (int u = 0; u < kReduceGroup; ++u)
        if (z0 + u < r.splits) s += t[u];
    }
    if constexpr (VEC4) {
      f32x4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = r.alpha * s[e];
      if (r.beta != 0.f) {
        const f32x4 old = *reinterpret_cast<const f32x4 *>(c);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = fmaf(r.beta, old[e], o[e]);
      }
      *reinterpret_cast<f32x4 *>(c) = o;
    } else {
      float o = r.alpha * s;
      if (r.beta != 0.f) o = fmaf(r.beta, *c, o);
      *c = o;
    }
  }
}

}  // namespace

const SgemmKernel *sgemm_kernels(int *count) {
  *count = (int)(sizeof kSgemmKernels / sizeof kSgemmKernels[0]);
  return kSgemmKernels;
}

hipError_t launch_sgemm_reduce(const SgemmReduceArgs &r, hipStream_t s) {
  SgemmReduceArgs copy = r;
  void *args[] = {&copy};
  const bool vec4 = r.n % 4 == 0 && r.ldc % 4 == 0 &&
                    (uintptr_t)r.c % 16 == 0 && (uintptr_t)r.partial % 16 == 0;
  const int64_t work = vec4 ? r.m * (r.n / 4) : r.m * r.n;
  int64_t blocks = (work + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  return hipLaunchKernel(
      vec4 ? reinterpret_cast<const void *>(&xpose_sgemm_reduce_kernel<true>)
           : reinterpret_cast<const void *>(&xpose_sgemm_reduce_kernel<false>),
      dim3((uint32_t)blocks), dim3(256), args, 0, s);
}

// Once per device, with that device current: the device address of
// `scratch`, kept per device (each GPU holds its own copy of the array at
// its own address).  Concurrent first calls may both look it up; they store
// the same value.
hipError_t sgemm_scratch(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void *> cache[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void *p = cache[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    cache[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace xpose
