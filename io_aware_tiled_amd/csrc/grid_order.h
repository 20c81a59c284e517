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

// Packed batches, whose sequences differ in length: a contiguous range of pairs would hand one
// XCD one long sequence. Instead pair bh goes to XCD bh mod 8 (pairs are sequence-major, so with
// a head count that is a multiple of 8 every XCD gets every sequence, with an eighth of its
// heads) and, within an XCD, the pairs run one after another with their blocks together.
// `id` is blockIdx over nbh pairs of nblk blocks; returns the pair and the block index within it.
__device__ __forceinline__ void xcd_grouped_pairs(int id, int nbh, int nblk, int& bh, int& blk) {
  const int lin = xcd_contiguous(id, nbh * nblk);
  const int pos = lin / nblk;  // position in the order of pairs grouped by bh mod 8
  blk = lin - pos * nblk;
  // group x holds the pairs x, x + 8, x + 16, ...: nbh / 8 of them, one more for x < nbh mod 8
  const int q = nbh >> 3, r = nbh & 7;
  const int x = pos < r * (q + 1) ? pos / (q + 1) : r + (pos - r * (q + 1)) / q;
  bh = x + 8 * (pos - (x * q + (x < r ? x : r)));
}

}  // namespace fattn
