// Work order of the causal prefill's grid when it has more workgroups than
// the chip holds at once (host and device: a CPU test checks that it maps
// the grid one to one onto the work items, for any grid shape).
//
// Workgroups go round-robin over the 8 XCDs, so workgroup x + 8 i runs on
// XCD x, and each XCD takes its workgroups in order as its slots free up.
// The (sequence, head) pairs, padded to a multiple of 8, each own q_tiles
// query tiles, tile 0 the heaviest (it walks the most keys):
//   * first round, as many whole groups of 8 pairs as the chip holds:
//     workgroup x + 8 (qi + q_tiles grp) is tile qi of pair 8 grp + x, so all
//     tiles of a pair run on one XCD together and walk the same keys while
//     the K/V tiles sit in that XCD's L2;
//   * the rest: each XCD takes tile 0 of each of its remaining pairs, then
//     tile 1, and so on, so the slots that free up first (light first-round
//     tiles) get the heaviest tiles and the last to free up the lightest.
#pragma once

#include <hip/hip_runtime.h>

namespace pa {

// pairs of the first round: whole groups of 8 whose q_tiles workgroups each fit
// in `slots` (the workgroups the chip holds at once), at most pairs_p
__host__ __device__ inline int grouped_first_round_pairs(int slots, int q_tiles, int pairs_p) {
  const int p1 = slots / (8 * q_tiles) * 8;
  return p1 < pairs_p ? p1 : pairs_p;
}

// pair and query tile (0 = heaviest) of workgroup b of a grid of q_tiles *
// pairs_p workgroups (pairs_p a multiple of 8), p1 pairs in the first round
__host__ __device__ inline void grouped_item(int b, int q_tiles, int pairs_p, int p1, int& pair, int& qi) {
  if (b < p1 * q_tiles) {
    const int rest = b >> 3;
    pair = (rest / q_tiles) * 8 + (b & 7);
    qi = rest % q_tiles;
  } else {  // p1 * q_tiles is a multiple of 8: r keeps b's XCD
    const int r = b - p1 * q_tiles;
    const int n2 = (pairs_p - p1) >> 3;  // remaining pairs per XCD
    const int k = r >> 3;
    pair = p1 + 8 * (k % n2) + (r & 7);
    qi = k / n2;
  }
}

}  // namespace pa
