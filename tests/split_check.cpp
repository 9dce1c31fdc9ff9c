// Host driver for the kernel's GEMV work splits (dec_internal.h), for
// tests/test_splits.py.  Reads "npairs K G skip" lines from stdin and prints,
// per workgroup g, its row pairs [p0, p1) and each streamer's unit range.  A
// line with skip -1 asks for the batched kernel's split of npairs 16-row
// groups instead: per workgroup, its groups [b, e).
#include <cstdio>

#include "dec_internal.h"

using namespace decmono;

int main() {
  int npairs, K, G, skip;
  const int kStreamers = kWaves - 1;
  while (std::scanf("%d %d %d %d", &npairs, &K, &G, &skip) == 4) {
    if (skip == -1) {
      for (int g = 0; g < G; ++g) {
        int b, e;
        split_tail(npairs, g, G, b, e);
        std::printf("%d %d %d\n", g, b, e);
      }
      std::printf("end\n");
      continue;
    }
    const int npc = gemv_piece_cols(K);
    for (int g = 0; g < G; ++g) {
      int p0 = 0, p1 = 0;
      if (g >= skip) split_even(npairs, g - skip, G - skip, p0, p1);
      std::printf("%d %d %d", g, p0, p1);
      for (int s = 1; s <= kStreamers; ++s) {
        int u0, u1;
        streamer_range((p1 - p0) * npc, npc, kStreamers, s, u0, u1);
        std::printf(" %d %d", u0, u1);
      }
      std::printf("\n");
    }
    std::printf("end\n");
  }
  return 0;
}
