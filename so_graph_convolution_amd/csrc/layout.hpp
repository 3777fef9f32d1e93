// Index arithmetic shared by host and device code of the SO(2) convolution library.
//
// Notation (TrimSO(2) page, Section 2 and Appendix A.2): L = lmax, M = mmax,
// C = node channels, Ci = 2C message input channels ([source | target]),
// degree-major node rows (l, m) at l*l + l + m, retained orders |m| <= min(l, M).
//
// "m-major" edge layouts (the GEMM layouts of Appendix B.1/B.3): one row per
// edge, blocks for |m| = 0..M. With channel width W:
//   block 0 : columns (l = 0..L, c)                               width (L+1) W
//   block m : columns [ +m : (l = m..L, c) | -m : (l = m..L, c) ] width 2 (L-m+1) W
// Total width q_{L,M} W. With the gated activation the first linear's output
// adds L*C gate columns (l = 1..L, c) to block 0; with the spherical-grid
// SwiGLU activation it has width 2C per row (value channels, then gate
// channels) and no extra columns.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace so2 {

constexpr int kMaxL = 6;

__host__ __device__ constexpr inline int imin(int a, int b) { return a < b ? a : b; }
__host__ __device__ constexpr inline int iabs(int a) { return a < 0 ? -a : a; }

// retained half-width of degree l
__host__ __device__ constexpr inline int qhalf(int l, int M) { return imin(l, M); }

// q_{L,M} = sum_l (2 min(l,M) + 1)
__host__ __device__ constexpr inline int q_count(int L, int M) {
  return (L + 1) * (2 * M + 1) - M * (M + 1);
}

// offset of the compact rotation rows of degree l; entry (l, m, n) lives at
// rot_off(l) + (m + qhalf(l)) * (2l+1) + (n + l)
__host__ __device__ constexpr inline int rot_off(int l, int M) {
  int o = 0;
  for (int k = 0; k < l; ++k) o += (2 * qhalf(k, M) + 1) * (2 * k + 1);
  return o;
}
__host__ __device__ constexpr inline int k_count(int L, int M) { return rot_off(L + 1, M); }

// first column of block |m| = a in an m-major layout of channel width W
__host__ __device__ constexpr inline int mm_block(int a, int L, int W) {
  // (L+1) + sum_{m'=1}^{a-1} 2 (L - m' + 1)
  return a == 0 ? 0 : W * ((L + 1) + 2 * ((a - 1) * (L + 1) - (a - 1) * a / 2));
}
// width of block |m| = a
__host__ __device__ constexpr inline int mm_width(int a, int L, int W) {
  return a == 0 ? (L + 1) * W : 2 * (L - a + 1) * W;
}
// column of (l, m, c) in an m-major layout of channel width W
__host__ __device__ constexpr inline int mm_col(int l, int m, int c, int L, int W) {
  const int a = iabs(m);
  return a == 0 ? l * W + c : mm_block(a, L, W) + (m < 0 ? (L - a + 1) * W : 0) + (l - a) * W + c;
}

// The so(3) generators in the real harmonic basis have at most two nonzeros
// per row: G_x couples order m to orders -(m+1) and -(m-1), G_y to m-1 and
// m+1, G_z to -m. gen_cand gives the candidate orders of row m (ascending; a
// candidate outside -l..l, or c1 == c0, is not used).
__host__ __device__ constexpr inline void gen_cand(int k, int m, int* c0, int* c1) {
  const int a = k == 0 ? -(m + 1) : (k == 1 ? m - 1 : -m);
  const int b = k == 0 ? -(m - 1) : (k == 1 ? m + 1 : -m);
  *c0 = a < b ? a : b;
  *c1 = a < b ? b : a;
}

// so(3) generator table: degree l block at gen_off(l), (2l+1)^2 entries
__host__ __device__ constexpr inline int gen_off(int l) { return l == 0 ? 0 : gen_off(l - 1) + (2 * l - 1) * (2 * l - 1); }
constexpr int kGenSize = gen_off(kMaxL + 1);   // 455 per generator

constexpr int kMaxHeads = 16;   // heads of the per-edge message weights (C / heads >= 16)

struct Dims {
  int L, M, C;
  int H = 1;    // heads of the per-edge message weights: channel c belongs to head c / (C / H)
  int s2 = 0;   // Edge -> Edge activation: 0 gate, 1 spherical-grid SwiGLU
  __host__ __device__ int Ci() const { return 2 * C; }
  __host__ __device__ int hs() const { return C / H; }                // channels per head
  __host__ __device__ int d() const { return (L + 1) * (L + 1); }
  __host__ __device__ int q() const { return q_count(L, M); }
  __host__ __device__ int K() const { return k_count(L, M); }
  __host__ __device__ int wT() const { return q() * 2 * C; }        // rotated input row
  __host__ __device__ int wZ() const { return q() * C; }            // hidden / message row
  __host__ __device__ int hw() const { return s2 ? 2 * C : C; }     // first-linear output width per row
  __host__ __device__ int wU() const { return s2 ? q() * 2 * C : q() * C + L * C; }   // first-linear output row
  // column of block a in the first-linear output (with the gate, block 0 carries the gate columns)
  __host__ __device__ int u_block(int a) const {
    return s2 ? mm_block(a, L, 2 * C) : (a == 0 ? 0 : mm_block(a, L, C) + L * C);
  }
  __host__ __device__ int u_width(int a) const {
    return s2 ? mm_width(a, L, 2 * C) : (a == 0 ? (2 * L + 1) * C : mm_width(a, L, C));
  }
  __host__ __device__ int gate_col(int l, int c) const { return (L + 1) * C + (l - 1) * C + c; }
  // U column of (l, m, c)
  __host__ __device__ int u_col(int l, int m, int c) const {
    return m == 0 ? l * C + c : mm_col(l, m, c, L, C) + L * C;
  }
};

// Launch shape of the elementwise gate kernels: one thread per (edge, degree,
// four channels), block (C/4, L+1, edges per block) with whole waves per
// block; blocks stride over the edges. Needs C % 4 == 0 (C is a multiple of 16).
inline void gate_dims(const Dims& d, long E, dim3* grid, dim3* block) {
  const int tpe = (d.C / 4) * (d.L + 1);
  int g = tpe, b = 64;
  while (b) {
    const int t = g % b;
    g = b;
    b = t;
  }
  int epb = 64 / g;
  while (epb > 1 && epb * tpe > 1024) epb /= 2;
  *block = dim3(d.C / 4, d.L + 1, epb);
  long nb = (E + epb - 1) / epb;
  if (nb > 65536) nb = 65536;
  *grid = dim3((unsigned)(nb > 0 ? nb : 1));
}

}  // namespace so2
