// Workgroup orders for the 8 XCDs of the MI355X. The hardware deals a launch's workgroups to the
// XCDs round-robin (workgroup i runs on XCD i mod 8) and each XCD has its own L2, so the order in
// which a kernel maps blockIdx to work decides both which XCD does which work and which blocks
// meet in one L2. The blocks of one (sequence, head) pair read the same K and V (forward, dQ) or
// the same Q and dO (dK/dV); they should run together, on one XCD.
#pragma once

#include <hip/hip_runtime.h>

namespace fattn {

// Dense batches, every pair the same size: give XCD x a contiguous range of the logical order
// (pair-major, then block), so that each XCD works through whole pairs.
__device__ __forceinline__ int xcd_contiguous(int id, int total) {
  const int xcd = id & 7, k = id >> 3;
  const int q8 = total >> 3, r8 = total & 7;
  return xcd * q8 + (xcd < r8 ? xcd : r8) + k;
}

// Dense batches, causal blocks of different sizes: XCD x gets the same contiguous range of whole
// pairs as with xcd_contiguous, but within it the pairs are taken G at a time and the blocks of
// those G pairs run block-major (block 0 of each, then block 1, ...). Workgroups are dispatched
// in order as CUs free up, so a long causal block dispatched next to blocks of its own size
// (rather than next to a whole pair's mix of sizes) keeps the CUs of an XCD finishing together;
// G pairs at a time keep the K and V (or Q and dO) those blocks read few enough to share L2.
// Ranges that do not cover whole pairs (pair counts not a multiple of 8) fall back to
// xcd_contiguous. `id` is blockIdx over `total` = nbh * nblk blocks.
template <int G>
__device__ __forceinline__ void xcd_pair_groups(int id, int total, int nblk, int& bh, int& blk) {
  const int x = id & 7, k = id >> 3;
  const int q8 = total >> 3, r8 = total & 7;
  const int nx = q8 + (x < r8 ? 1 : 0);
  const int sx = x * q8 + (x < r8 ? x : r8);
  if (sx % nblk != 0 || nx % nblk != 0) {
    const int lin = sx + k;
    bh = lin / nblk;
    blk = lin - bh * nblk;
    return;
  }
  const int pairs = nx / nblk;
  const int grp = k / (G * nblk);
  const int w = k - grp * (G * nblk);
  const int in_grp = min(G, pairs - grp * G);
  bh = sx / nblk + grp * G + w % in_grp;
  blk = w / in_grp;
}

// Packed batches, whose sequences differ in length: a contiguous range of pairs would hand one
// XCD one long sequence. Instead pair bh goes to XCD bh mod 8 (pairs are sequence-major, so with
// a head count that is a multiple of 8 every XCD gets every sequence, with an eighth of its
// heads). Within an XCD the pairs run G at a time, the blocks of those G pairs block-major, as
// in xcd_pair_groups (G = 1: each pair's blocks together). Pair counts that are not a multiple
// of 8 keep the deal by bh mod 8 with G = 1.
// `id` is blockIdx over nbh pairs of nblk blocks; returns the pair and the block index within it.
template <int G>
__device__ __forceinline__ void xcd_grouped_pairs(int id, int nbh, int nblk, int& bh, int& blk) {
  if ((nbh & 7) == 0) {
    // XCD x runs exactly the nbh / 8 pairs x, x + 8, ...: the k-th workgroup it is dealt
    const int x = id & 7, k = id >> 3, px = nbh >> 3;
    const int grp = k / (G * nblk);
    const int w = k - grp * (G * nblk);
    const int in_grp = min(G, px - grp * G);
    bh = x + 8 * (grp * G + w % in_grp);
    blk = w / in_grp;
    return;
  }
  const int lin = xcd_contiguous(id, nbh * nblk);
  const int pos = lin / nblk;  // position in the order of pairs grouped by bh mod 8
  blk = lin - pos * nblk;
  // group x holds the pairs x, x + 8, x + 16, ...: nbh / 8 of them, one more for x < nbh mod 8
  const int q = nbh >> 3, r = nbh & 7;
  const int x = pos < r * (q + 1) ? pos / (q + 1) : r + (pos - r * (q + 1)) / q;
  bh = x + 8 * (pos - (x * q + (x < r ? x : r)));
}

}  // namespace fattn
