// Host-side exhaustive check of the workgroup -> tile mapping the kernels
// use: for many grid shapes, super-tile shapes, batch counts and with and
// without the per-XCD remap, every workgroup must land on a tile inside the
// grid and every tile must be hit exactly once.  Prints "ok <cases>" or the
// first failing case and exits non-zero.
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "../../lds_tiled_matrix_amd/csrc/xpose_kernels.h"

int main() {
  const uint32_t dims[] = {1, 2, 3, 5, 7, 8, 13, 16, 31, 64, 107, 128, 193};
  long cases = 0;
  for (uint32_t tr_n : dims)
    for (uint32_t tc_n : dims)
      for (uint32_t batch : {1u, 3u})
        for (uint32_t gr : {1u, 2u, 3u, 8u, 16u, 1000u})
          for (uint32_t gc : {1u, 3u, 8u, 32u, 1000u})
            for (int xcd = 0; xcd < 6; ++xcd) {
              xpose::TileArgs a = {};
              a.order = xcd < 2   ? xpose::kOrderSuperTiles
                        : xcd < 4 ? xpose::kOrderDiagonal
                                  : xpose::kOrderColumnBands;
              a.tiles_r = tr_n;
              a.tiles_c = tc_n;
              a.group_rows = gr < tr_n ? gr : tr_n;
              a.group_cols = gc < tc_n ? gc : tc_n;
              a.xcd_remap = xcd & 1;
              const uint32_t n = batch * tr_n * tc_n;
              std::vector<int> hit(n, 0);
              for (uint32_t blk = 0; blk < n; ++blk) {
                uint32_t tr, tc;
                int64_t b;
                xpose::tile_coords(a, blk, n, tr, tc, b);
                if (tr >= tr_n || tc >= tc_n || b < 0 || b >= (int64_t)batch) {
                  printf("out of range: tiles %ux%u batch %u group %ux%u xcd %d "
                         "block %u -> (%lld, %u, %u)\n",
                         tr_n, tc_n, batch, a.group_rows, a.group_cols, xcd,
                         blk, (long long)b, tr, tc);
                  return 1;
                }
                ++hit[(b * tr_n + tr) * tc_n + tc];
              }
              for (uint32_t i = 0; i < n; ++i)
                if (hit[i] != 1) {
                  printf("tile %u hit %d times: tiles %ux%u batch %u group "
                         "%ux%u xcd %d\n",
                         i, hit[i], tr_n, tc_n, batch, a.group_rows,
                         a.group_cols, xcd);
                  return 1;
                }
              ++cases;
            }
  printf("ok %ld\n", cases);
  return 0;
}
