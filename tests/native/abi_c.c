/* The C ABI from plain C99: include/xpose.h must compile as C with every
 * warning an error, and a C caller must see the same struct layouts and
 * host-only results as the Python binding.  Prints:
 *   size <struct> <bytes>
 *   offset <struct>.<field> <bytes>
 *   const <name> <value>
 *   plan <rc> <field>=<value> ...     (for the calls in main)
 *   strerror <code> <text>
 */
#include <stddef.h>
#include <stdio.h>
#include <string.h>

#include "xpose.h"
#include "xpose_sgemm.h"

#define SIZE(T) printf("size %s %zu\n", #T, sizeof(T))
#define OFF(T, F) printf("offset %s.%s %zu\n", #T, #F, offsetof(T, F))
#define CONST(N) printf("const %s %d\n", #N, (int)(N))

static void plan(const char *tag, void *out, const void *in, int64_t batch,
                 int64_t rows, int64_t cols, int64_t ld_in, int64_t ld_out,
                 int32_t dtype, const xpose_opts *opts) {
  xpose_plan_info info;
  memset(&info, 0xff, sizeof info);
  const int rc = xpose_plan(out, in, batch, rows, cols, ld_in, ld_out,
                            rows * ld_in, cols * ld_out, dtype, opts, &info);
  printf("plan %s %d", tag, rc);
  if (rc == XPOSE_OK)
    printf(" layout=%d tile_rows=%d tile_cols=%d threads=%d lds_bytes=%d "
           "vector_path=%d tiles=%lld launches=%d cache=%d aligned_out=%d "
           "tr_read=%d occupancy=%d",
           info.layout, info.tile_rows, info.tile_cols, info.threads,
           info.lds_bytes, info.vector_path, (long long)info.tiles,
           info.launches, info.cache, info.aligned_out, info.tr_read,
           info.occupancy);
  printf("\n");
}

int main(void) {
  SIZE(xpose_opts);
  OFF(xpose_opts, layout); OFF(xpose_opts, flags); OFF(xpose_opts, threads);
  OFF(xpose_opts, persistent); OFF(xpose_opts, occupancy);
  SIZE(xpose_plan_info);
  OFF(xpose_plan_info, vector_path); OFF(xpose_plan_info, tiles);
  OFF(xpose_plan_info, launches); OFF(xpose_plan_info, tr_read);
  OFF(xpose_plan_info, occupancy);
  SIZE(xpose_copy_opts);
  OFF(xpose_copy_opts, cache);
  CONST(XPOSE_F32); CONST(XPOSE_F16); CONST(XPOSE_BF16); CONST(XPOSE_U8);
  CONST(XPOSE_F64);
  CONST(XPOSE_OK); CONST(XPOSE_EINVAL); CONST(XPOSE_EALIAS);
  CONST(XPOSE_EDTYPE); CONST(XPOSE_EHIP); CONST(XPOSE_EALIGN);
  CONST(XPOSE_ENOTILE);
  CONST(XPOSE_FLAG_TR_READ); CONST(XPOSE_FLAG_ALIGN_OUT);

  char *const out = (char *)0x100000000000ull, *const in = (char *)0x200000000000ull;
  plan("c2", out, in, 1, 8192, 8192, 8192, 8192, XPOSE_F32, NULL);
  plan("c3", out, in, 1, 12345, 6789, 6789, 12345, XPOSE_F32, NULL);
  plan("c4", out, in, 1, 16384, 16384, 16384, 16384, XPOSE_F16, NULL);
  xpose_opts tr;
  memset(&tr, 0, sizeof tr);
  tr.flags = XPOSE_FLAG_TR_READ;
  plan("c4tr", out, in, 1, 16384, 16384, 16384, 16384, XPOSE_F16, &tr);
  plan("null", NULL, in, 1, 64, 64, 64, 64, XPOSE_F32, NULL);
  plan("alias", in, in, 1, 64, 64, 64, 64, XPOSE_F32, NULL);
  plan("dtype", out, in, 1, 64, 64, 64, 64, 9, NULL);
  {
    /* xpose_2d_ex rejects invalid calls on the host before any launch, and a
     * zero-sized shape is a no-op; NULL opts is xpose_2d. */
    xpose_opts bad;
    memset(&bad, 0, sizeof bad);
    bad.layout = 9;
    printf("ex pitch %d\n", xpose_2d_ex(out, in, 64, 64, 63, 64, XPOSE_F32, NULL, NULL));
    printf("ex alias %d\n", xpose_2d_ex(in, in, 64, 64, 64, 64, XPOSE_F32, &tr, NULL));
    printf("ex layout %d\n", xpose_2d_ex(out, in, 64, 64, 64, 64, XPOSE_F32, &bad, NULL));
    printf("ex dtype %d\n", xpose_2d_ex(out, in, 64, 64, 64, 64, 9, NULL, NULL));
    printf("ex empty %d\n", xpose_2d_ex(NULL, NULL, 0, 64, 64, 0, XPOSE_F16, &tr, NULL));
  }
  SIZE(xpose_sgemm_opts);
  OFF(xpose_sgemm_opts, bk); OFF(xpose_sgemm_opts, flags);
  OFF(xpose_sgemm_opts, tile_m); OFF(xpose_sgemm_opts, split_k);
  SIZE(xpose_sgemm_info);
  OFF(xpose_sgemm_info, as_stride); OFF(xpose_sgemm_info, xcd_remap);
  OFF(xpose_sgemm_info, tiles); OFF(xpose_sgemm_info, whole_matrix);
  OFF(xpose_sgemm_info, edge_buffer_loads); OFF(xpose_sgemm_info, splits);
  OFF(xpose_sgemm_info, split_len); OFF(xpose_sgemm_info, workspace_bytes);
  OFF(xpose_sgemm_info, workspace_wanted);
  CONST(XPOSE_EWORKSPACE);
  CONST(XPOSE_AS_UNPADDED); CONST(XPOSE_AS_PADDED); CONST(XPOSE_AS_SWIZZLE);
  CONST(XPOSE_SGEMM_NO_XCD_REMAP); CONST(XPOSE_SGEMM_DOUBLE_BUFFER); CONST(XPOSE_SGEMM_NO_BUFFER_LOADS);
  {
    xpose_sgemm_info gi;
    memset(&gi, 0xff, sizeof gi);
    const float *a = (const float *)0x300000000000ull;
    const float *b = (const float *)0x310000000000ull;
    const float *c = (const float *)0x320000000000ull;
    const int rc = xpose_sgemm_plan(4096, 4096, 4096, a, 4096, b, 4096, c,
                                    4096, NULL, &gi);
    printf("sgemm %d layout=%d bk=%d as_stride=%d lds_bytes=%d tiles=%lld\n",
           rc, gi.layout, gi.bk, gi.as_stride, gi.lds_bytes,
           (long long)gi.tiles);
    /* a small grid with a workspace: the library's split */
    const void *ws = (const void *)0x330000000000ull;
    memset(&gi, 0xff, sizeof gi);
    const int rs = xpose_sgemm_plan_ws(1024, 1024, 1024, a, 1024, b, 1024, c,
                                       1024, NULL, ws, (int64_t)1 << 30, &gi);
    printf("sgemmws %d splits=%d split_len=%lld workspace_bytes=%lld "
           "workspace_wanted=%lld tiles=%lld\n",
           rs, gi.splits, (long long)gi.split_len,
           (long long)gi.workspace_bytes, (long long)gi.workspace_wanted,
           (long long)gi.tiles);
  }
  for (int code = 0; code >= -7; --code)
    printf("strerror %d %s\n", code, xpose_strerror(code));
  return 0;
}
