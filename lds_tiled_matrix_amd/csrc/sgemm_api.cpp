// C-ABI front end of the tiled SGEMM (include/xpose_sgemm.h): argument
// validation, kernel choice and launch.  Validation and planning are host
// code that never touches the GPU.

#include "../../include/xpose_sgemm.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sgemm_kernels.h"

namespace {

constexpr int kTileN = 128;         // columns of C per workgroup
constexpr int kDefaultTileM = 128;
constexpr int kDefaultBk = 16;
constexpr int kDefaultLayout = XPOSE_AS_PADDED;
constexpr int kDefaultGroupM = 8;
// Large shapes whose 256-row blocks fill whole rounds of the grid take
// 256-row blocks with the swizzled As layout by default: two 512-thread
// workgroups run on each of MI355X's 256 compute units, 512 blocks a round.
// Measured from k = 1024 on, 4096 to 16384 rows and columns: 137.7-146.3
// against 132.3-143.0 TFLOP/s for 128-row padded blocks.  Level at k = 512;
// with a partial round (3072 x 4096 x 4096: 109 against 138) they lose.
constexpr int64_t kTallRound = 512;
constexpr int64_t kTallMinK = 1024;
// Largest pitches for buffer loads: the tile_m rows of A's tile (plus the k
// step) and the at most 64 rows of B's tile within a 31-bit byte offset.
constexpr int64_t max_buffer_lda(int tile_m) {
  return ((int64_t)1 << 31) / (4 * (tile_m + 1));
}
constexpr int64_t kMaxBufferLdb = ((int64_t)1 << 31) / (4 * 129) * 2;

struct SgemmPlan {
  bool empty = false;
  const xpose::SgemmKernel *kernel = nullptr;
  xpose::SgemmArgs args{};
  int64_t tiles = 0;
};

// a * b + c without overflow, all >= 0; false if it does not fit.
bool mul_add(int64_t a, int64_t b, int64_t c, int64_t *out) {
  int64_t p;
  if (__builtin_mul_overflow(a, b, &p)) return false;
  return !__builtin_add_overflow(p, c, out);
}

// Byte range [lo, hi) of a rows x cols matrix with pitch ld at p.
bool byte_range(const void *p, int64_t rows, int64_t cols, int64_t ld,
                uintptr_t *lo, uintptr_t *hi) {
  int64_t last, bytes;
  if (!mul_add(rows - 1, ld, cols, &last)) return false;
  if (__builtin_mul_overflow(last, (int64_t)4, &bytes)) return false;
  *lo = (uintptr_t)p;
  if (__builtin_add_overflow(*lo, (uintptr_t)bytes, hi)) return false;
  return true;
}

bool overlaps(uintptr_t a0, uintptr_t a1, uintptr_t b0, uintptr_t b1) {
  return a0 < b1 && b0 < a1;
}

int make_plan(int64_t m, int64_t n, int64_t k, const float *a, int64_t lda,
              const float *b, int64_t ldb, const float *c, int64_t ldc,
              const xpose_sgemm_opts *opts, SgemmPlan &plan) {
  int layout = kDefaultLayout, bk = kDefaultBk, group_m = kDefaultGroupM,
      tile_m = kDefaultTileM;
  bool remap = true, buffers = true;
  int stages = 1;
  if (opts) {
    if (opts->layout < XPOSE_AS_AUTO || opts->layout > XPOSE_AS_SWIZZLE)
      return XPOSE_EINVAL;
    if (opts->bk != 0 && opts->bk != 8 && opts->bk != 16 && opts->bk != 32 &&
        opts->bk != 64)
      return XPOSE_EINVAL;
    if (opts->group_m < 0) return XPOSE_EINVAL;
    if (opts->tile_m != 0 && opts->tile_m != 64 && opts->tile_m != 128 &&
        opts->tile_m != 256)
      return XPOSE_EINVAL;
    if (opts->flags & ~(XPOSE_SGEMM_NO_XCD_REMAP | XPOSE_SGEMM_DOUBLE_BUFFER |
                        XPOSE_SGEMM_NO_BUFFER_LOADS))
      return XPOSE_EINVAL;
    if (opts->layout) layout = opts->layout;
    if (opts->bk) bk = opts->bk;
    if (opts->group_m) group_m = opts->group_m;
    if (opts->tile_m) tile_m = opts->tile_m;
    remap = !(opts->flags & XPOSE_SGEMM_NO_XCD_REMAP);
    if (opts->flags & XPOSE_SGEMM_DOUBLE_BUFFER) stages = 2;
    if (opts->flags & XPOSE_SGEMM_NO_BUFFER_LOADS) buffers = false;
  }
  if (m < 0 || n < 0 || k < 0) return XPOSE_EINVAL;
  const bool chosen = opts && (opts->layout || opts->bk || opts->tile_m ||
                               (opts->flags & XPOSE_SGEMM_DOUBLE_BUFFER));
  if (!chosen && m > 0 && n > 0 && m % 256 == 0 && n % kTileN == 0 &&
      k >= kTallMinK && m / 256 <= INT32_MAX && n / kTileN <= INT32_MAX &&
      (m / 256) * (n / kTileN) % kTallRound == 0) {
    layout = XPOSE_AS_SWIZZLE;
    tile_m = 256;
  }
  if (lda < (k > 1 ? k : 1) || ldb < (n > 1 ? n : 1) ||
      ldc < (n > 1 ? n : 1))
    return XPOSE_EINVAL;
  if (m == 0 || n == 0) {
    plan.empty = true;
    return XPOSE_OK;
  }
  const bool uses_ab = k > 0;
  if (!c || (uses_ab && (!a || !b))) return XPOSE_EINVAL;
  if ((uintptr_t)c % 4 || (uses_ab && ((uintptr_t)a % 4 || (uintptr_t)b % 4)))
    return XPOSE_EALIGN;
  uintptr_t c0, c1;
  if (!byte_range(c, m, n, ldc, &c0, &c1)) return XPOSE_EINVAL;
  if (uses_ab) {
    uintptr_t a0, a1, b0, b1;
    if (!byte_range(a, m, k, lda, &a0, &a1) ||
        !byte_range(b, k, n, ldb, &b0, &b1))
      return XPOSE_EINVAL;
    if (overlaps(c0, c1, a0, a1) || overlaps(c0, c1, b0, b1))
      return XPOSE_EALIAS;
  }
  const int64_t tiles_m = (m + tile_m - 1) / tile_m;
  const int64_t tiles_n = (n + kTileN - 1) / kTileN;
  int64_t tiles;
  if (__builtin_mul_overflow(tiles_m, tiles_n, &tiles) || tiles > INT32_MAX)
    return XPOSE_EINVAL;
  const bool vec = !uses_ab || ((uintptr_t)a % 16 == 0 &&
                                (uintptr_t)b % 16 == 0 && lda % 4 == 0 &&
                                ldb % 4 == 0);
  const bool buf_ok = buffers && vec && uses_ab &&
                      lda <= max_buffer_lda(tile_m) && ldb <= kMaxBufferLdb;
  // Every block, k step, load and C tail whole: the kernel without edge
  // code, where one is built.
  const bool whole = buf_ok && stages == 1 && m % tile_m == 0 &&
                     n % kTileN == 0 && k % bk == 0 &&
                     ldc <= ((int64_t)1 << 29) / tile_m;
  int count = 0;
  const xpose::SgemmKernel *table = xpose::sgemm_kernels(&count);
  const xpose::SgemmKernel *kern = nullptr;
  for (int pass = whole ? 0 : 1; pass < 2 && !kern; ++pass)
    for (int i = 0; i < count && !kern; ++i)
      if (table[i].bk == bk && table[i].layout == layout &&
          table[i].vec == vec && table[i].stages == stages &&
          table[i].tile_m == tile_m && table[i].whole == (pass == 0))
        kern = &table[i];
  if (!kern) return XPOSE_ENOTILE;
  if (group_m > tiles_m) group_m = (int)tiles_m;

  xpose::SgemmArgs &g = plan.args;
  g.a = a;
  g.b = b;
  g.c = const_cast<float *>(c);
  g.m = m;
  g.n = n;
  g.k = k;
  g.lda = lda;
  g.ldb = ldb;
  g.ldc = ldc;
  g.tiles_m = (uint32_t)tiles_m;
  g.tiles_n = (uint32_t)tiles_n;
  g.group_m = (uint32_t)group_m;
  g.xcd_remap = remap ? 1 : 0;
  // Buffer-load byte offsets within one k step's tiles must fit in 31 bits.
  g.buf_ok = buf_ok;
  g.edge_buf = buf_ok && k % 4 == 0 && n % 4 == 0;
  plan.kernel = kern;
  plan.tiles = tiles;
  return XPOSE_OK;
}

int run(int64_t m, int64_t n, int64_t k, float alpha, const float *a,
        int64_t lda, const float *b, int64_t ldb, float beta, float *c,
        int64_t ldc, const xpose_sgemm_opts *opts, void *stream) {
  SgemmPlan plan;
  const int rc = make_plan(m, n, k, a, lda, b, ldb, c, ldc, opts, plan);
  if (rc != XPOSE_OK || plan.empty) return rc;
  plan.args.alpha = alpha;
  plan.args.beta = beta;
  const hipError_t e = plan.kernel->launch(plan.args, (uint32_t)plan.tiles,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? XPOSE_OK : xpose::record_hip_error(e);
}

}  // namespace

extern "C" {

int xpose_sgemm(int64_t m, int64_t n, int64_t k, float alpha, const float *a,
                int64_t lda, const float *b, int64_t ldb, float beta,
                float *c, int64_t ldc, void *stream) {
  return run(m, n, k, alpha, a, lda, b, ldb, beta, c, ldc, nullptr, stream);
}

int xpose_sgemm_ex(int64_t m, int64_t n, int64_t k, float alpha,
                   const float *a, int64_t lda, const float *b, int64_t ldb,
                   float beta, float *c, int64_t ldc,
                   const xpose_sgemm_opts *opts, void *stream) {
  return run(m, n, k, alpha, a, lda, b, ldb, beta, c, ldc, opts, stream);
}

int xpose_sgemm_plan(int64_t m, int64_t n, int64_t k, const float *a,
                     int64_t lda, const float *b, int64_t ldb, const float *c,
                     int64_t ldc, const xpose_sgemm_opts *opts,
                     xpose_sgemm_info *info) {
  SgemmPlan plan;
  const int rc = make_plan(m, n, k, a, lda, b, ldb, c, ldc, opts, plan);
  if (rc != XPOSE_OK || !info) return rc;
  *info = xpose_sgemm_info{};
  if (plan.empty) return rc;
  const xpose::SgemmKernel &kern = *plan.kernel;
  info->layout = kern.layout;
  info->bk = kern.bk;
  info->as_stride = kern.as_stride;
  info->lds_bytes = kern.lds_bytes;
  info->threads = kern.threads;
  info->tile_m = kern.tile_m;
  info->tile_n = kTileN;
  info->vector_loads = kern.vec ? 1 : 0;
  info->group_m = (int32_t)plan.args.group_m;
  info->xcd_remap = plan.args.xcd_remap;
  info->stages = kern.stages;
  info->buffer_loads = plan.args.buf_ok;
  info->tiles = plan.tiles;
  info->whole_matrix = kern.whole ? 1 : 0;
  info->edge_buffer_loads = kern.vec && plan.args.edge_buf ? 1 : 0;
  return rc;
}

}  // extern "C"
