// C-ABI front end of the tiled SGEMM (include/xpose_sgemm.h): argument
// validation, kernel choice and launch.  Validation and planning are host
// code that never touches the GPU.

#include "../../include/xpose_sgemm.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

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

// Split of k: at most this many slices; the library's own choice keeps
// slices at least kMinAutoSplitLen long (the shortest measured to pay).
constexpr int kMaxSplits = 64;
constexpr int64_t kMinAutoSplitLen = 64;

struct SgemmPlan {
  bool empty = false;
  const xpose::SgemmKernel *kernel = nullptr;
  xpose::SgemmArgs args{};
  int64_t tiles = 0;
  int64_t workspace_wanted = 0;
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

// Slice length for at most `want` slices of k, in whole k steps.
int64_t split_len(int64_t k, int64_t want, int bk) {
  const int64_t per = (k + want - 1) / want;
  return (per + bk - 1) / bk * bk;
}

// Slices of k taken for at most `want` of length `len`.
int64_t slice_count(int64_t k, int64_t want, int64_t len) {
  return want < 2 || len >= k ? 1 : (k + len - 1) / len;
}

// Estimated busy time of the compute unit holding `w` workgroups of
// `len` k elements each: they run four at a time (the register budget of
// the 128-row kernels), and w of them together go at kShare[w] times one
// alone (one workgroup leaves the matrix cores idle while it waits on
// memory and barriers).
double cu_time(int64_t w, double len) {
  static const double kShare[5] = {0, 1.0, 1.2, 1.3, 1.4};
  const int64_t full = w / 4, rem = w % 4;
  double t = (double)full * 4 * len / kShare[4];
  if (rem) t += rem * len / kShare[rem];
  return t;
}

// The library's split: the slice count (1 = none) whose estimated time is
// least, among slices of at least kMinAutoSplitLen.  Blocks count as units
// of 128 rows (tiles * tile_m / 128).  The units * slices workgroups spread
// over 256 compute units, so the busiest holds w = ceil(units * slices /
// 256), and the product takes cu_time(w, slice length).  A split adds its
// partial sums, written once and read once, 6 (slices + 1) m n / (256 *
// 1024) in the same units, and 40 for the second kernel's launch (about
// 3 us; a unit is one k element of a lone workgroup, 1024 of which take
// 73 us).  The constants are fitted to measured times of 1 to 32 slices
// over 23 shapes from 512^3 to 8192 x 8192 x 2048 on MI355X: the choice
// lands within 0.96 of the fastest measured split everywhere, 0.997 on
// average.
int64_t auto_splits(int64_t tiles, int tile_m, int64_t m, int64_t n,
                    int64_t k, int bk) {
  const double units = (double)tiles * tile_m / 128;
  double best_cost = 0;
  int64_t best = 1, last = 0;
  for (int64_t want = 1; want <= kMaxSplits; ++want) {
    const int64_t len = split_len(k, want, bk);
    const int64_t slices = slice_count(k, want, len);
    if (slices == last) continue;
    if (slices > 1 && len < kMinAutoSplitLen) break;
    last = slices;
    const int64_t w = (int64_t)std::ceil(units * slices / 256);
    double cost = cu_time(w, (double)(slices > 1 ? len : k));
    if (slices > 1)
      cost += 6.0 * (slices + 1) * ((double)m * n) / (256 * 1024) + 40;
    if (want == 1 || cost < best_cost) {
      best_cost = cost;
      best = want;
    }
  }
  return best;
}

// Validates a call and fills `plan`.  has_ws: the entry point takes a
// workspace (`ws`, ws_bytes), so it may split k.  scratch: the workspace is
// the library's own device array (ws_bytes = kSgemmScratchBytes, `ws`
// ignored), whose address is only looked up once every argument has been
// validated and the call does split.
int make_plan(int64_t m, int64_t n, int64_t k, const float *a, int64_t lda,
              const float *b, int64_t ldb, const float *c, int64_t ldc,
              const xpose_sgemm_opts *opts, bool has_ws, const void *ws,
              int64_t ws_bytes, SgemmPlan &plan, bool scratch = false) {
  int layout = kDefaultLayout, bk = kDefaultBk, group_m = kDefaultGroupM,
      tile_m = kDefaultTileM, split = 0;
  bool remap = true, buffers = true;
  int stages = 1;
  if (has_ws && ws_bytes < 0) return XPOSE_EINVAL;
  if (opts) {
    if (opts->split_k < 0 || opts->split_k > kMaxSplits) return XPOSE_EINVAL;
    split = opts->split_k;
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
  g.splits = 1;
  g.split_k = k;
  plan.kernel = kern;
  plan.tiles = tiles;

  // Split of k.  Slices are whole k steps, so every slice but the last is
  // whole, and the last is whole exactly when k is: the kernel chosen above
  // (whole-matrix or not) serves every slice, and its partials' pitch n is
  // at most ldc.
  const int64_t plane = m * n;  // fits: C's byte range did
  auto slices_of = [&](int64_t want, int64_t *len) {
    *len = split_len(k, want, bk);
    return slice_count(k, want, *len);
  };
  int64_t want = split == 1   ? 1
                 : split >= 2 ? split
                 : k > 0      ? auto_splits(tiles, tile_m, m, n, k, bk)
                              : 1;
  int64_t len, slices = k > 0 ? slices_of(want, &len) : 1;
  if (slices > 1) {
    int64_t floats, bytes;
    if (__builtin_mul_overflow(slices, plane, &floats) ||
        __builtin_mul_overflow(floats, (int64_t)4, &bytes) ||
        tiles * slices > INT32_MAX)
      return XPOSE_EINVAL;
    plan.workspace_wanted = bytes;
  }
  if (slices > 1 && split == 0) {
    // The library's choice shrinks to what the workspace holds.
    const int64_t fit = has_ws ? ws_bytes / 4 / plane : 0;
    if (fit < slices) slices = fit < 2 ? 1 : slices_of(fit, &len);
  } else if (slices > 1 && (!has_ws || ws_bytes / 4 / plane < slices)) {
    return XPOSE_EWORKSPACE;
  }
  if (slices > 1) {
    if (scratch) {
      void *p = nullptr;
      const hipError_t e = xpose::sgemm_scratch(&p);
      if (e != hipSuccess) return xpose::record_hip_error(e);
      ws = p;
    }
    uintptr_t w0 = (uintptr_t)ws, w1;
    if (!ws) return XPOSE_EINVAL;
    if (w0 % 4) return XPOSE_EALIGN;
    if (__builtin_add_overflow(w0, (uintptr_t)(slices * plane * 4), &w1))
      return XPOSE_EINVAL;
    uintptr_t a0, a1, b0, b1;
    byte_range(a, m, k, lda, &a0, &a1);
    byte_range(b, k, n, ldb, &b0, &b1);
    if (overlaps(w0, w1, a0, a1) || overlaps(w0, w1, b0, b1) ||
        overlaps(w0, w1, c0, c1))
      return XPOSE_EALIAS;
    g.splits = (int32_t)slices;
    g.split_k = len;
    g.partial = static_cast<float *>(const_cast<void *>(ws));
    plan.tiles = tiles * slices;
  }
  return XPOSE_OK;
}

int run(int64_t m, int64_t n, int64_t k, float alpha, const float *a,
        int64_t lda, const float *b, int64_t ldb, float beta, float *c,
        int64_t ldc, const xpose_sgemm_opts *opts, bool has_ws, void *ws,
        int64_t ws_bytes, void *stream, bool scratch = false) {
  SgemmPlan plan;
  const int rc = make_plan(m, n, k, a, lda, b, ldb, c, ldc, opts, has_ws, ws,
                           ws_bytes, plan, scratch);
  if (rc != XPOSE_OK || plan.empty) return rc;
  plan.args.alpha = alpha;
  plan.args.beta = beta;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = plan.kernel->launch(plan.args, (uint32_t)plan.tiles, s);
  if (e == hipSuccess && plan.args.splits > 1) {
    xpose::SgemmReduceArgs r{};
    r.partial = plan.args.partial;
    r.c = c;
    r.m = m;
    r.n = n;
    r.ldc = ldc;
    r.splits = plan.args.splits;
    r.alpha = alpha;
    r.beta = beta;
    e = xpose::launch_sgemm_reduce(r, s);
  }
  return e == hipSuccess ? XPOSE_OK : xpose::record_hip_error(e);
}

int plan_info(int64_t m, int64_t n, int64_t k, const float *a, int64_t lda,
              const float *b, int64_t ldb, const float *c, int64_t ldc,
              const xpose_sgemm_opts *opts, bool has_ws, const void *ws,
              int64_t ws_bytes, xpose_sgemm_info *info) {
  SgemmPlan plan;
  const int rc = make_plan(m, n, k, a, lda, b, ldb, c, ldc, opts, has_ws, ws,
                           ws_bytes, plan);
  if (rc == XPOSE_EWORKSPACE && info) {
    *info = xpose_sgemm_info{};
    info->workspace_wanted = plan.workspace_wanted;
  }
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
  info->splits = plan.args.splits;
  info->split_len = plan.args.split_k;
  info->workspace_bytes =
      plan.args.splits > 1 ? (int64_t)plan.args.splits * m * n * 4 : 0;
  info->workspace_wanted = plan.workspace_wanted;
  return rc;
}

}  // namespace

extern "C" {

int xpose_sgemm(int64_t m, int64_t n, int64_t k, float alpha, const float *a,
                int64_t lda, const float *b, int64_t ldb, float beta,
                float *c, int64_t ldc, void *stream) {
  return run(m, n, k, alpha, a, lda, b, ldb, beta, c, ldc, nullptr, false,
             nullptr, 0, stream);
}

int xpose_sgemm_ex(int64_t m, int64_t n, int64_t k, float alpha,
                   const float *a, int64_t lda, const float *b, int64_t ldb,
                   float beta, float *c, int64_t ldc,
                   const xpose_sgemm_opts *opts, void *stream) {
  return run(m, n, k, alpha, a, lda, b, ldb, beta, c, ldc, opts, false,
             nullptr, 0, stream);
}

int xpose_sgemm_plan(int64_t m, int64_t n, int64_t k, const float *a,
                     int64_t lda, const float *b, int64_t ldb, const float *c,
                     int64_t ldc, const xpose_sgemm_opts *opts,
                     xpose_sgemm_info *info) {
  return plan_info(m, n, k, a, lda, b, ldb, c, ldc, opts, false, nullptr, 0,
                   info);
}

int xpose_sgemm_ws(int64_t m, int64_t n, int64_t k, float alpha,
                   const float *a, int64_t lda, const float *b, int64_t ldb,
                   float beta, float *c, int64_t ldc,
                   const xpose_sgemm_opts *opts, void *workspace,
                   int64_t workspace_bytes, void *stream) {
  return run(m, n, k, alpha, a, lda, b, ldb, beta, c, ldc, opts, true,
             workspace, workspace_bytes, stream);
}

int xpose_sgemm_noalloc(int64_t m, int64_t n, int64_t k, float alpha,
                        const float *a, int64_t lda, const float *b,
                        int64_t ldb, float beta, float *c, int64_t ldc,
                        const xpose_sgemm_opts *opts, void *stream) {
  return run(m, n, k, alpha, a, lda, b, ldb, beta, c, ldc, opts, true,
             nullptr, xpose::kSgemmScratchBytes, stream, true);
}

int xpose_sgemm_plan_ws(int64_t m, int64_t n, int64_t k, const float *a,
                        int64_t lda, const float *b, int64_t ldb,
                        const float *c, int64_t ldc,
                        const xpose_sgemm_opts *opts, const void *workspace,
                        int64_t workspace_bytes, xpose_sgemm_info *info) {
  return plan_info(m, n, k, a, lda, b, ldb, c, ldc, opts, true, workspace,
                   workspace_bytes, info);
}

}  // extern "C"
