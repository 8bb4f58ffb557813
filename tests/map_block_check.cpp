// Host check of the workgroup -> (head, tile) order of the MFMA kernels
// (map_block in bwd_rope_apply_amd/csrc/tile.h) over many launch shapes:
//  - every (head, tile) pair is produced exactly once (a bijection);
//  - with a head count divisible by 8, workgroup idx runs on XCD idx % 8
//    and that XCD only ever sees its own BH / 8 heads;
//  - each head's tiles come heaviest first (descending tile index when
//    heavy_high) or in ascending order otherwise;
//  - an XCD with more than `group` heads (a multiple of it) finishes one
//    group of heads before it starts the next.
// Prints "<checks> checks, <failures> failed"; exit status 0 when all pass.
#include <stdio.h>

#include <vector>

#include "tile.h"

int main() {
  long checks = 0, fails = 0;
  auto expect = [&](bool ok, const char* what, int BH, int nt, int idx) {
    ++checks;
    if (!ok && fails++ < 20) fprintf(stderr, "%s: BH=%d ntiles=%d idx=%d\n", what, BH, nt, idx);
  };
  const int bhs[] = {1, 2, 3, 5, 7, 8, 9, 15, 16, 24, 32, 40, 48, 64, 96, 100, 128, 136, 256, 512, 4100};
  const int nts[] = {1, 2, 3, 7, 16, 31, 64, 256};
  for (int BH : bhs) {
    for (int nt : nts) {
      if ((long)BH * nt > 300000) continue;
      for (int heavy = 0; heavy < 2; ++heavy) {
        for (int group : {2, 4, 8}) {
          const int n = BH * nt;
          std::vector<char> seen((size_t)n, 0);
          std::vector<int> last((size_t)BH, -1);
          const int hpx = BH / 8;
          const bool grouped = BH % 8 == 0 && hpx > group && hpx % group == 0;
          for (int idx = 0; idx < n; ++idx) {
            int bh = -1, t = -1;
            ra::map_block(idx, BH, nt, heavy != 0, bh, t, group);
            const bool in = bh >= 0 && bh < BH && t >= 0 && t < nt;
            expect(in, "out of range", BH, nt, idx);
            if (!in) continue;
            char& s = seen[(size_t)bh * nt + t];
            expect(s == 0, "pair produced twice", BH, nt, idx);
            s = 1;
            if (BH % 8 == 0) expect(bh / hpx == idx % 8, "head off its XCD", BH, nt, idx);
            const int k = heavy ? nt - 1 - t : t;   // position in the head's order
            expect(k == last[bh] + 1, "head's tiles out of order", BH, nt, idx);
            last[bh] = k;
            if (grouped)
              expect((bh % hpx) / group == (idx >> 3) / (group * nt), "head outside its group", BH, nt,
                     idx);
          }
          for (int i = 0; i < n; ++i) expect(seen[(size_t)i] == 1, "pair never produced", BH, nt, i);
        }
      }
    }
  }
  printf("%ld checks, %ld failed\n", checks, fails);
  return fails == 0 ? 0 : 1;
}
