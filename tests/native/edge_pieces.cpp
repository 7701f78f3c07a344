// Host check of the partial-vector pieces of the transpose edge path
// (load_head / store_head in lds_tiled_matrix_amd/csrc/xpose_lanes.h): for
// every length n < 16 and every start offset, a vector placed so that its
// n-th byte ends a readable page (the next page has no access) must load
// exactly its n bytes, zero above, and a store must write exactly n bytes.
// Prints "ok" or the first failure; an over-read or over-write faults.
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
  char *end = m + page;  // first inaccessible byte
  for (int i = 0; i < page; ++i) m[i] = (char)(i * 37 + 11);
  for (int n = 0; n < 16; ++n) {
    for (int shift = 0; shift < 16; ++shift) {
      // the vector's first byte, so that byte n - 1 is the page's last one
      // (shift moves it down to vary the alignment)
      char *p = end - n - shift;
      uint64_t lo, hi;
      load_head(p, n, lo, hi);
      unsigned char want[16] = {0}, got[16];
      memcpy(want, p, n);
      memcpy(got, &lo, 8);
      memcpy(got + 8, &hi, 8);
      if (memcmp(want, got, 16)) {
        printf("load n=%d shift=%d wrong\n", n, shift);
        return 1;
      }
      // store a distinct pattern and check exactly [p, p + n) changed
      unsigned char before[64];
      char *lo_guard = p - 16;
      memcpy(before, lo_guard, 16 + n + shift);
      uint64_t slo = 0x0123456789abcdefull ^ (uint64_t)n,
               shi = 0xfedcba9876543210ull ^ (uint64_t)shift;
      store_head(p, n, slo, shi);
      unsigned char pat[16];
      memcpy(pat, &slo, 8);
      memcpy(pat + 8, &shi, 8);
      if (memcmp(lo_guard, before, 16) || memcmp(p, pat, n) ||
          memcmp(p + n, before + 16 + n, shift)) {
        printf("store n=%d shift=%d wrong\n", n, shift);
        return 1;
      }
      memcpy(lo_guard, before, 16 + n + shift);
    }
  }
  printf("ok\n");
  return 0;
}
