// Direct-to-LDS staging of float32 operand tiles (16 k per tile), shared by
// the float32 GEMM kernels.
#pragma once
#include <hip/hip_runtime.h>

namespace so2 {

typedef float f32x4_dma __attribute__((ext_vector_type(4)));

// gfx950's global_load_lds_dwordx4 moves 16 bytes per lane from global memory
// straight into LDS: lane l writes bytes [16 l, 16 l + 16) of a 1 KB block
// with a wave-uniform base, from any per-lane address. The float32 kernels
// build their 16-k operand tiles from such blocks in a ring of stages: the
// loads of later k tiles are in flight while a tile is multiplied, with no
// register staging and no LDS store instructions (measured on MI355X at the
// per-order shapes, 725k rows: 5-6% faster than register-staged kernels, which
// remain for operands without 16-byte alignment).
//
// The lane -> element map of a block is free, which gives the tile layouts:
//   k-contiguous tile (R rows x 16 k): block b holds rows 16b .. 16b+15; lane
//     l = 4r + s carries row 16b + r, k chunk q = (s - r/4) mod 4 (four k), so
//     chunk q of row r sits at 16-byte unit 4r + (q + r/4) mod 4. A
//     quarter-wave (16 lanes) then loads four whole 64-byte row segments, and
//     a fragment read (16 rows, one chunk) still falls on 16 distinct groups
//     of four banks (the rotation by r/4 separates rows r, r+4, r+8, r+12).
//   k-major tile (16 k x R columns): block b holds k rows b KPB .. b KPB +
//     KPB-1 (KPB = 256/R) at R floats apart, and blocks sit BLK = 256 + 1024/R
//     floats apart, so k and k + 8 (the two lane halves of a read) are 32
//     banks apart ((8/KPB) BLK = 32 mod 64).
// Every wave issues three loads per stage, so a wave's vmcnt tells when its
// part of a stage has landed, and a barrier after that wait publishes the
// stage. A tile that runs past the end of K (the last of a split) is staged
// through registers, zero-filled, into the same positions. Rows (columns)
// past the operand's edge load the last valid row (column chunk) instead:
// they only reach outputs that are not stored.
constexpr int DNS = 3;       // stages
template <bool KCONTIG, int R>
struct DT {
  static constexpr int NB = R / 16;                     // 1 KB blocks per tile
  static constexpr int KPB = 256 / R;                   // k-major: k rows per block
  static constexpr int BLK = KCONTIG ? 256 : 256 + 1024 / R;
  static constexpr int FL = NB * BLK;                   // floats per tile
};
struct DSlot {
  const float* src;   // this lane's 16 bytes in the split's first k tile
  long step;          // elements between consecutive k tiles
  int dst;            // block offset within a stage (floats)
  int kofs;           // k of this lane's data within a tile (first of four if k-contiguous)
  int kc;             // k-contiguous data
};
template <bool KCONTIG, int R>
__device__ inline DSlot dslot(int b, const float* P, int ld, int r0, int rlim, int kbeg, int lane, int base) {
  DSlot d;
  if (KCONTIG) {
    const int rr = lane / 4, q = (lane % 4 - rr / 4) & 3;
    const int row = min(r0 + 16 * b + rr, rlim - 1);
    d.src = P + (size_t)row * ld + kbeg + 4 * q;
    d.step = 16;
    d.kofs = 4 * q;
    d.kc = 1;
    d.dst = base + b * 256;
  } else {
    constexpr int LPR = R / 4;
    const int k = b * DT<false, R>::KPB + lane / LPR, col = min(r0 + 4 * (lane % LPR), rlim - 4);
    d.src = P + (size_t)(kbeg + k) * ld + col;
    d.step = 16L * ld;
    d.kofs = k;
    d.kc = 0;
    d.dst = base + b * DT<false, R>::BLK;
  }
  return d;
}
__device__ __forceinline__ void dma16(const float* src, float* dst) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}
// stage k tile t (of a split holding nkk k values) into st
template <int SL>
__device__ inline void dstage(const DSlot (&sl)[SL], float* st, int t, int nkk, int lane) {
  const int k0 = 16 * t;
  if (k0 + 16 <= nkk) {
#pragma unroll
    for (int j = 0; j < SL; ++j) dma16(sl[j].src + t * sl[j].step, st + sl[j].dst);
  } else {
#pragma unroll
    for (int j = 0; j < SL; ++j) {
      const float* q = sl[j].src + t * sl[j].step;
      f32x4_dma x = {0.f, 0.f, 0.f, 0.f};
      if (sl[j].kc) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (k0 + sl[j].kofs + c < nkk) x[c] = q[c];
      } else if (k0 + sl[j].kofs < nkk) {
        x = *reinterpret_cast<const f32x4_dma*>(q);
      }
      *reinterpret_cast<f32x4_dma*>(st + sl[j].dst + 4 * lane) = x;
    }
  }
}
// wait until this wave's loads of tile t have landed (the SL loads of tile
// t + 1, if issued, may still be in flight) and publish the stage to the block
template <int SL>
__device__ __forceinline__ void dsync(bool next_in_flight) {
  static_assert(SL == 2 || SL == 3 || SL == 5, "loads per wave and stage");
  if (!next_in_flight) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  else if (SL == 2) asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)" ::: "memory");
  else if (SL == 3) asm volatile("s_waitcnt vmcnt(3) lgkmcnt(0)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(5) lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// MFMA operands of one staged tile for lane half lk: row `row`, k = 8 lk + s
template <bool KCONTIG, int R>
__device__ __forceinline__ void dfrag(const float* T, int row, int lk, float (&f)[8]) {
  if (KCONTIG) {
    const int r = row % 16;
    const float* q = T + (row / 16) * 256 + 16 * r;
    const f32x4_dma u = *reinterpret_cast<const f32x4_dma*>(q + 4 * ((2 * lk + r / 4) & 3));
    const f32x4_dma w = *reinterpret_cast<const f32x4_dma*>(q + 4 * ((2 * lk + 1 + r / 4) & 3));
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      f[c] = u[c];
      f[4 + c] = w[c];
    }
  } else {
    using D = DT<false, R>;
    const float* q = T + lk * (8 / D::KPB) * D::BLK + row;
#pragma unroll
    for (int s = 0; s < 8; ++s) f[s] = q[(s / D::KPB) * D::BLK + (s % D::KPB) * R];
  }
}

}  // namespace so2
