// Tile order of the grouped GEMM launches, shared by every GEMM kernel.
#pragma once
#include <hip/hip_runtime.h>

#include "gemm.hpp"

namespace so2 {

// linear block id -> position in a virtual tile order such that the blocks one
// XCD receives (round-robin dispatch over 8 XCDs) cover a contiguous range
__device__ inline int xcd_remap(int bid, int total) {
  const int q = total / 8, r = total % 8;
  const int x = bid % 8, i = bid / 8;
  return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// Virtual order: eight slots, slot s holding the s-th eighth of every problem's
// tiles (problems in order, tiles contiguous inside each share). Combined with
// xcd_remap, every XCD gets an equal share of each problem -- problems of one
// launch differ in K, so handing whole problems to XCDs would leave the XCDs
// with the heavy problem running long -- while tiles that share a row panel
// stay on one XCD.
__device__ inline void decode_tile(const GemmBatch& b, int v, int* pi, int* local) {
  int acc = 0;
#pragma unroll 1
  for (int s = 0; s < 8; ++s) {
    int slot = 0;
#pragma unroll 1
    for (int p = 0; p < b.nprob; ++p) {
      const int T = (p + 1 < b.nprob ? b.p[p + 1].tile_begin : b.total_tiles) - b.p[p].tile_begin;
      slot += ((s + 1) * T) / 8 - (s * T) / 8;
    }
    if (v < acc + slot) {
      int off = v - acc;
#pragma unroll 1
      for (int p = 0; p < b.nprob; ++p) {
        const int T = (p + 1 < b.nprob ? b.p[p + 1].tile_begin : b.total_tiles) - b.p[p].tile_begin;
        const int lo = (s * T) / 8, cnt = ((s + 1) * T) / 8 - lo;
        if (off < cnt) {
          *pi = p;
          *local = lo + off;
          return;
        }
        off -= cnt;
      }
    }
    acc += slot;
  }
  *pi = 0;
  *local = 0;
}

}  // namespace so2
