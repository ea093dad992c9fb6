// decompose.h -- work decomposition shared by the attention kernels (host and device code): which
// (sequence, head, query block) a workgroup computes.  The FlashAttention-3 pages parallelise the
// forward pass over batch x head x query blocks, one block of O per thread block (zenmind
// digest, section 4, data path step 1); the mapping below also places that work on gfx950's 8
// XCDs, each with its own L2.
#pragma once

#include <hip/hip_runtime.h>

namespace attn {

// Bijection from hardware workgroup id to a logical id such that each XCD (hardware id mod 8)
// receives one contiguous range of logical ids.
__host__ __device__ __forceinline__ int xcd_remap(int wg, int total) {
  constexpr int kXcd = 8;
  const int q = total / kXcd, r = total % kXcd;
  const int x = wg % kXcd, i = wg / kXcd;
  return x * q + (x < r ? x : r) + i;
}

// Work decomposition: hardware workgroup id -> (query block, head, sequence).  Workgroups are
// dispatched round-robin over the 8 XCDs (id mod 8), each XCD running its share in id order.
// When the heads split evenly over the XCDs, every XCD owns the same heads of every sequence,
// so packed sequences of unequal length load all XCDs alike; whole KV groups stay on one XCD
// (their query heads share the group's K/V in that XCD's L2) when the KV heads split evenly too.
// Inside an XCD, causal grids run all query blocks longest first (a block's work grows with
// its index); non-causal grids keep the blocks of one head together.  Otherwise each XCD
// takes one contiguous range of (sequence, head, block) ids, causal blocks longest first.
template <bool CAUSAL>
__host__ __device__ __forceinline__ void decompose(int wg, int nqb, int Hq, int Hkv, int B, int& qb, int& h, int& b) {
  constexpr int kXcd = 8;
  if (Hq % kXcd == 0) {
    const int x = wg % kXcd, slot = wg / kXcd;
    const int hpx = Hq / kXcd;  // heads per XCD and sequence
    int r;
    if (CAUSAL) {
      qb = nqb - 1 - slot / (hpx * B);
      r = slot % (hpx * B);
    } else {
      qb = slot % nqb;
      r = slot / nqb;
    }
    b = r / hpx;
    const int hh = r % hpx;
    if (Hkv % kXcd == 0) {
      const int G = Hq / Hkv;  // query heads per KV group; groups x, x + 8, ... live on XCD x
      h = (x + kXcd * (hh / G)) * G + hh % G;
    } else {
      h = x + kXcd * hh;
    }
  } else {
    const int logical = xcd_remap(wg, nqb * Hq * B);
    qb = logical % nqb;
    const int bh = logical / nqb;
    h = bh % Hq;
    b = bh / Hq;
    if (CAUSAL) qb = nqb - 1 - qb;
  }
}

}  // namespace attn
