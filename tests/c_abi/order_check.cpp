// Host-side check of the workgroup order (exact_tiled_attention_26_amd/csrc/
// fa_order.h): head_and_tile must be a bijection of the workgroup ids onto
// (head, tile) for every group size, keep the tiles of a group together and
// heaviest first, and head_group_for must pick the plain order while the
// device holds 4 workgroups per head and otherwise a group size that is a
// multiple of 8 (or all heads).  Prints the number of cases checked; exits
// nonzero on the first failure.
#include <cstdio>
#include <vector>

#include "../../exact_tiled_attention_26_amd/csrc/fa_order.h"

static int fail(const char* what, int bh, int nt, int hg) {
  std::printf("FAIL %s bh=%d ntiles=%d hg=%d\n", what, bh, nt, hg);
  return 1;
}

int main() {
  long cases = 0;
  const int bhs[] = {1, 2, 3, 5, 7, 8, 9, 15, 16, 17, 31, 32, 33, 64, 100, 128, 300, 512, 2048};
  const int nts[] = {1, 2, 3, 7, 8, 16, 31, 32, 64, 128};
  for (int bh : bhs) {
    for (int nt : nts) {
      std::vector<int> hgs = {1, 8, bh};
      for (int resident : {256, 512, 1024}) hgs.push_back(fa::head_group_for(bh, nt, resident));
      for (int hg : hgs) {
        if (hg < 1 || hg > bh) continue;
        std::vector<int> seen((size_t)bh * nt, 0);
        int prev_grp = 0;
        for (int id = 0; id < bh * nt; ++id) {
          int head = -1, tile = -1;
          fa::head_and_tile(id, bh, nt, hg, head, tile);
          if (head < 0 || head >= bh || tile < 0 || tile >= nt) return fail("range", bh, nt, hg);
          if (seen[(size_t)head * nt + tile]++) return fail("duplicate", bh, nt, hg);
          // groups in id order, each a block of whole heads
          const int grp = head / hg;
          if (grp < prev_grp) return fail("group order", bh, nt, hg);
          prev_grp = grp;
          // within a group, tile ranks never decrease with id
          if (id > 0) {
            int h0, t0;
            fa::head_and_tile(id - 1, bh, nt, hg, h0, t0);
            if (h0 / hg == grp && t0 > tile) return fail("tile order", bh, nt, hg);
          }
          // hg = bh is the plain order
          if (hg == bh && (head != id % bh || tile != id / bh)) return fail("plain order", bh, nt, hg);
        }
        ++cases;
      }
      for (int resident : {64, 256, 512, 1024, 4096}) {
        const int hg = fa::head_group_for(bh, nt, resident);
        if (hg < 1 || hg > bh) return fail("group size range", bh, nt, hg);
        if (resident >= 4 * bh && hg != bh) return fail("plain order kept", bh, nt, hg);
        if (hg != bh && (hg % 8 != 0 || hg < 8)) return fail("multiple of 8", bh, nt, hg);
        if (hg != bh && hg > 8 && hg * nt > resident) return fail("group resident", bh, nt, hg);
        ++cases;
      }
    }
  }
  // the shapes the measurements were taken on (resident = 256: one
  // workgroup per CU on 256 CUs): plain order at the headline (32 heads),
  // groups of heads past 64 heads
  struct Spot { int bh, nt, resident, hg; };
  const Spot spots[] = {{32, 32, 256, 32}, {32, 64, 256, 32}, {64, 32, 256, 64}, {65, 32, 256, 8},
                        {128, 16, 256, 16}, {512, 8, 256, 32}, {2048, 4, 256, 64}, {100, 2, 256, 100},
                        {8, 64, 256, 8}};
  for (const Spot& s : spots) {
    if (fa::head_group_for(s.bh, s.nt, s.resident) != s.hg) return fail("spot", s.bh, s.nt, s.hg);
    ++cases;
  }
  std::printf("order ok: %ld cases\n", cases);
  return 0;
}
