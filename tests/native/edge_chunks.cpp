// Host check of the edge-tile chunk loads of the transpose
// (edge_chunk_src / edge_chunk_fix in
// lds_tiled_matrix_amd/csrc/xpose_lanes.h).  A row whose last byte ends a
// readable page (the next page has no access) holds W elements from the
// tile's first one, W >= V (the tile holds at least one whole chunk); for
// every element size, every W up to 3 chunks, every chunk of the tile row
// and both row states (inside or past the matrix), the 16 bytes read at the
// chosen address and fixed up must equal the chunk's elements inside the
// row followed by zeros, or all zeros.  An over-read faults.
// Prints "ok" or the first failure.
#include <stdio.h>
#include <string.h>
#include <sys/mman.h>
#include <unistd.h>

#include "../../lds_tiled_matrix_amd/csrc/xpose_lanes.h"

using namespace xpose;

int main() {
  const long page = sysconf(_SC_PAGESIZE);
  char *m = (char *)mmap(nullptr, 2 * page, PROT_READ | PROT_WRITE,
                         MAP_PRIVATE | MAP_ANONYMOUS, -1, 0);
  if (m == MAP_FAILED) return 2;
  if (mprotect(m + page, page, PROT_NONE)) return 2;
  char *end = m + page;  // first inaccessible byte: the row's end
  for (int i = 0; i < page; ++i) m[i] = (char)(i * 37 + 11);
  int cases = 0;
  for (int S = 1; S <= 8; S *= 2) {
    const int V = 16 / S;
    for (int W = V; W <= 3 * V; ++W) {           // row elements from tile0
      const char *tile0 = end - (int64_t)W * S;  // the tile's first element
      for (int ch = 0; ch * V < W + 2 * V; ++ch) {  // chunks past the end too
        const int64_t have = W - (int64_t)ch * V;
        const char *chunk = tile0 + (int64_t)ch * V * S;
        for (int in_row = 0; in_row < 2; ++in_row) {
          const char *at = edge_chunk_src(tile0, chunk, have, V, S, in_row);
          if (at < tile0 || at + 16 > end) {
            printf("S=%d W=%d ch=%d in_row=%d: address out of the row\n", S,
                   W, ch, in_row);
            return 1;
          }
          uint64_t lo, hi;
          memcpy(&lo, at, 8);  // the 16-byte load
          memcpy(&hi, at + 8, 8);
          edge_chunk_fix(lo, hi, have, V, S, in_row);
          unsigned char got[16], want[16] = {0};
          memcpy(got, &lo, 8);
          memcpy(got + 8, &hi, 8);
          if (in_row && have > 0)
            memcpy(want, chunk, (size_t)((have < V ? have : V) * S));
          if (memcmp(got, want, 16)) {
            printf("S=%d W=%d ch=%d in_row=%d: wrong bytes\n", S, W, ch,
                   in_row);
            return 1;
          }
          ++cases;
        }
      }
    }
  }
  printf(cases > 0 ? "ok\n" : "no cases\n");
  return 0;
}
