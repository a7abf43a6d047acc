// Workgroup order over (head, tile), shared by the kernels (device) and the
// launchers and the host-side check of the order (host).
//
// Workgroups are dispatched in id order and dealt to the 8 XCDs round robin,
// each XCD with its own L2.  Heads go in groups of hg (a multiple of 8
// unless it is all bh heads): id runs over the tiles of one group before
// the next, tile index = rank within the group, heaviest first, and head =
// first head of the group + id mod the group's size, so all tiles of a head
// land on one XCD and a group's tiles are in flight together, sharing the
// head's K/V (or Q/dO) through that L2.  With hg = bh this is the plain
// order head = id mod bh, tile = id / bh.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

// (head, tile) of workgroup id; a bijection of [0, bh * ntiles) onto
// [0, bh) x [0, ntiles) for any 1 <= hg <= bh
__host__ __device__ inline void head_and_tile(int id, int bh, int ntiles, int hg, int& head, int& tile) {
  const int span = hg * ntiles;
  const int grp = id / span;
  const int r = id - grp * span;
  const int gsz = (bh - grp * hg) < hg ? (bh - grp * hg) : hg;
  head = grp * hg + r % gsz;
  tile = r / gsz;
}

// Heads per group when `resident` workgroups run at once: all bh heads (the
// plain order) while there are at least 4 resident workgroups per head, else
// as many heads as have all their ntiles tiles resident together, rounded
// down to a multiple of 8, at least 8 and at most bh.  (Grouping the heads
// when the plain order already keeps several tiles of each head in flight
// measured 2-5 % slower on the causal N 8192 headline; past that, grouping
// measured 10-17 % faster with hundreds of heads.)
__host__ __device__ inline int head_group_for(int bh, int ntiles, int resident) {
  if (resident >= 4 * bh) return bh;
  int hg = resident / (ntiles > 0 ? ntiles : 1);
  hg -= hg % 8;
  if (hg < 8) hg = 8;
  return hg >= bh ? bh : hg;
}

}  // namespace fa
