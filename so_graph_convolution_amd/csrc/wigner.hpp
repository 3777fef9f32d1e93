// Edge frame and real Wigner-D rows, generated on the fly.
//
// The rotation law of node features (TrimSO(2) page, Appendix A.1) uses real
// Wigner-D blocks D^(l)(R) with Y(R u) = D(R) Y(u) for real orthonormal
// spherical harmonics without the Condon-Shortley phase, orders m = -l..l
// (so Y_1 is proportional to (y, z, x)). The convolution only needs the rows
// of retained orders |m| <= min(l, M) (the compact rotation blocks of
// Appendix B.1).
//
// Here D^(l) is built from D^(1) by the recursion of Ivanic and Ruedenberg
// (J. Phys. Chem. 100, 6342 (1996), with the corrections of 102, 9099
// (1998)): every entry of D^(l) is a weighted sum of three terms U, V, W, each
// a product of one entry of D^(1) with entries of D^(l-1). Row m of D^(l)
// needs rows up to |m|+1 of D^(l-1), so degree l keeps rows
// |m| <= min(l, M + L - l) and only the top degree is trimmed to M.
#pragma once
#include "layout.hpp"

namespace so2 {

// Rows of the edge frame R_e with R_e rhat = +z (the edge-aligned frame of
// Appendix A.2; any roll about the edge axis gives the same operator output).
//   z >= 0, k = 1/(1+z): (1-x^2 k, -xyk, -x), (-xyk, 1-y^2 k, -y), (x, y, z)
//   z <  0, k = 1/(1-z): (1-x^2 k, -xyk,  x), ( xyk, y^2 k-1, -y), (x, y, z)
template <typename T>
__host__ __device__ inline void edge_frame(T x, T y, T z, T R[9]) {
  const bool up = z >= T(0);
  const T k = up ? T(1) / (T(1) + z) : T(1) / (T(1) - z);
  const T s = up ? T(1) : T(-1);
  R[0] = T(1) - x * x * k; R[1] = -x * y * k;          R[2] = -s * x;
  R[3] = -s * x * y * k;    R[4] = s * (T(1) - y * y * k); R[5] = -y;
  R[6] = x;                 R[7] = y;                   R[8] = z;
}

// D^(1) in the (y, z, x) component order: D1[(i+1)*3 + (j+1)] = R[p(i)][p(j)],
// p(-1) = y, p(0) = z, p(1) = x.
template <typename T>
__host__ __device__ inline void wigner_l1(const T R[9], T D1[9]) {
  const int p[3] = {1, 2, 0};
#pragma unroll
  for (int a = 0; a < 3; ++a)
#pragma unroll
    for (int b = 0; b < 3; ++b) D1[a * 3 + b] = R[p[a] * 3 + p[b]];
}

// half-width of the rows kept at degree l when the top degree L keeps |m| <= M
__host__ __device__ constexpr inline int rows_kept(int l, int L, int M) { return imin(l, M + L - l); }

// one P term of the recursion; prev holds D^(l-1) rows -rp..rp, columns -(l-1)..(l-1)
template <typename T>
__host__ __device__ inline T wig_P(int i, int a, int b, int l, const T* D1, const T* prev, int rp) {
  const int w = 2 * l - 1;
  const T* row = prev + (a + rp) * w + (l - 1);
  const T* r1 = D1 + (i + 1) * 3;
  if (b == l) return r1[2] * row[l - 1] - r1[0] * row[-(l - 1)];
  if (b == -l) return r1[2] * row[-(l - 1)] + r1[0] * row[l - 1];
  return r1[1] * row[b];
}

// entry (m, n) of D^(l) from D^(1) and D^(l-1), l >= 2
template <typename T>
__host__ __device__ inline T wig_entry(int l, int m, int n, const T* D1, const T* prev, int rp) {
  const int am = iabs(m);
  const T den = (n > -l && n < l) ? T((l + n) * (l - n)) : T((2 * l) * (2 * l - 1));
  T out = T(0);
  if (am < l) {  // U term
    const T u = sqrt(T((l + m) * (l - m)) / den);
    out += u * wig_P(0, m, n, l, D1, prev, rp);
  }
  {  // V term
    const T v = (m == 0 ? T(-0.5) : T(0.5)) * sqrt(T((m == 0 ? 2 : 1) * (l + am - 1) * (l + am)) / den);
    T V;
    if (m == 0) {
      V = wig_P(1, 1, n, l, D1, prev, rp) + wig_P(-1, -1, n, l, D1, prev, rp);
    } else if (m > 0) {
      V = (m == 1) ? T(1.4142135623730951) * wig_P(1, 0, n, l, D1, prev, rp)
                   : wig_P(1, m - 1, n, l, D1, prev, rp) - wig_P(-1, -m + 1, n, l, D1, prev, rp);
    } else {
      V = (m == -1) ? T(1.4142135623730951) * wig_P(-1, 0, n, l, D1, prev, rp)
                    : wig_P(1, m + 1, n, l, D1, prev, rp) + wig_P(-1, -m - 1, n, l, D1, prev, rp);
    }
    out += v * V;
  }
  if (m != 0 && am <= l - 2) {  // W term
    const T w = T(-0.5) * sqrt(T((l - am - 1) * (l - am)) / den);
    const T W = (m > 0) ? wig_P(1, m + 1, n, l, D1, prev, rp) + wig_P(-1, -m - 1, n, l, D1, prev, rp)
                        : wig_P(1, m - 1, n, l, D1, prev, rp) - wig_P(-1, -m + 1, n, l, D1, prev, rp);
    out += w * W;
  }
  return out;
}

// LDS floats per edge used by the level scratch of wigner_rows_block
__host__ __device__ inline int wig_level_stride(int L, int M) {
  int s = 9;
  for (int l = 2; l < L; ++l) {
    const int r = rows_kept(l, L, M);
    const int w = (2 * r + 1) * (2 * l + 1);
    s = s > w ? s : w;
  }
  return s;
}

// Cooperative generation of the compact rotation rows of `ne` edges.
//   D1   [ne][9]   degree-1 blocks (input)
//   out  [ne][ldo] compact rows, entry (l, m, n) at rot_off(l) + (m+q_l)(2l+1) + n + l
//   bufA, bufB [ne][stride] level scratch, stride >= wig_level_stride(L, M)
// All threads of the block must call it; it ends with a barrier.
__device__ inline void wigner_rows_block(int L, int M, int ne, const float* D1, float* out, int ldo,
                                         float* bufA, float* bufB, int stride) {
  const int tid = threadIdx.x, nt = blockDim.x;
  for (int e = tid; e < ne; e += nt) {
    out[e * ldo] = 1.f;
    if (L >= 1) {
      const int q1 = qhalf(1, M);
      for (int m = -q1; m <= q1; ++m)
        for (int n = -1; n <= 1; ++n) out[e * ldo + 1 + (m + q1) * 3 + n + 1] = D1[e * 9 + (m + 1) * 3 + n + 1];
      for (int k = 0; k < 9; ++k) bufA[e * stride + k] = D1[e * 9 + k];
    }
  }
  __syncthreads();
  float* prev = bufA;
  float* cur = bufB;
  int rp = 1;
  for (int l = 2; l <= L; ++l) {
    const int rl = rows_kept(l, L, M);
    const int cols = 2 * l + 1;
    const int per = (2 * rl + 1) * cols;
    const int ql = qhalf(l, M);
    const int ro = rot_off(l, M);
    for (int idx = tid; idx < ne * per; idx += nt) {
      const int e = idx / per, rem = idx - e * per;
      const int m = rem / cols - rl, n = rem % cols - l;
      const float v = wig_entry<float>(l, m, n, D1 + e * 9, prev + e * stride, rp);
      if (l < L) cur[e * stride + rem] = v;
      if (iabs(m) <= ql) out[e * ldo + ro + (m + ql) * cols + n + l] = v;
    }
    __syncthreads();
    float* t = prev; prev = cur; cur = t;
    rp = rl;
  }
}

}  // namespace so2
