// Spherical-grid SwiGLU activation on edges (SwiGLU-S2): TrimSO(2) page,
// Table 2 (EquiformerV3's activation), Appendix C.1 "Implementation" (its Edge -> Edge
// spherical-grid activation) and Appendix B.4 (G_l evaluates the degree-l
// basis at n_g grid points; the nonlinearity acts on grid values).
//
// Per edge e and channel c, with q coefficient rows of a value half u_v
// (channels 0..C-1) and a gate half u_g (channels C..2C-1):
//   v = G u_v,  a = G u_g,  s = SiLU(a) v,  z = P s
// G [n_g, q] and P [q, n_g] are caller-supplied constants.
//
// Every (edge, channel) pair is one column of two small dense products that
// share their left factor: V = G U_v (M = grid points, K = rows) and
// Z = P S (M = rows, K = grid points). A wave takes 16 columns and runs both
// on v_mfma_f32_16x16x4_f32, one tile of 16 grid points at a time:
//   phase 1  V_t, A_t += G_t U   (K steps over rows 4kk .. 4kk+3)
//   SwiGLU   on the accumulators (lane (h, j) holds grid points 16t + 4h + i
//            of column j, i = 0..3)
//   phase 2  Z += P_t S_t, where K step i takes grid point 16t + 4k + i from
//            the lanes of group k: exactly the accumulator element i those
//            lanes hold, so S_t feeds the next product without a transpose.
// Grid values are never stored; the backward and double backward recompute
// V and A the same way. The constant operands are staged once per block in
// LDS in fragment order (a float4 per lane feeds 4 consecutive MFMA steps),
// zero-padded to whole tiles, which also makes padded rows and grid points
// contribute nothing.
#include "ops.hpp"

namespace so2 {

namespace {

typedef float s2f4 __attribute__((ext_vector_type(4)));

constexpr int kS2Threads = 512;        // 8 waves
constexpr int kS2Waves = kS2Threads / 64;
constexpr int kS2MaxBlocks = 2048;

__device__ __forceinline__ s2f4 s2_mma(float a, float b, s2f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float s2_sigm(float a) { return __builtin_amdgcn_rcpf(1.f + __expf(-a)); }

// Left operand with K over coefficient rows (phase 1): A[i][k] = M(gp, r) with
// gp = 16t + i, r = 4kk + k; float4 index (t * QR + kk / 4) * 64 + lane,
// component kk % 4 (lane = 16k + i). M(gp, r) = src[gp * sg + r * sr].
template <int QR>
__device__ void s2_build_rows(s2f4* dst, const float* __restrict__ src, int sg, int sr, int q, int ng, int NT) {
  float* d = reinterpret_cast<float*>(dst);
  const int n = NT * QR * 256;
  for (int idx = threadIdx.x; idx < n; idx += blockDim.x) {
    const int c = idx & 3, lane = (idx >> 2) & 63, kq = (idx >> 8) % QR, t = (idx >> 8) / QR;
    const int gp = 16 * t + (lane & 15), r = 4 * (4 * kq + c) + (lane >> 4);
    d[idx] = (gp < ng && r < q) ? src[(size_t)gp * sg + (size_t)r * sr] : 0.f;
  }
}

// Left operand with K over grid points (phase 2): A[i][k] = M(gp, r) with
// r = 16m + i, gp = 16t + 4k + c for component c; float4 index
// (m * NT + t) * 64 + lane.
template <int QR>
__device__ void s2_build_grid(s2f4* dst, const float* __restrict__ src, int sg, int sr, int q, int ng, int NT) {
  float* d = reinterpret_cast<float*>(dst);
  const int n = NT * QR * 256;
  for (int idx = threadIdx.x; idx < n; idx += blockDim.x) {
    const int c = idx & 3, lane = (idx >> 2) & 63, t = (idx >> 8) % NT, m = (idx >> 8) / NT;
    const int r = 16 * m + (lane & 15), gp = 16 * t + 4 * (lane >> 4) + c;
    d[idx] = (gp < ng && r < q) ? src[(size_t)gp * sg + (size_t)r * sr] : 0.f;
  }
}

// This lane's column (edge, channel) of column block cb: base offsets into
// the [E][q][2C] and [E][q][C] arrays; ok = false past the last column.
struct S2Col {
  size_t o2, o1;
  bool ok;
};
__device__ __forceinline__ S2Col s2_col(long cb, long ncol, int C, int q) {
  const long n = cb * 16 + (threadIdx.x & 15);
  S2Col s;
  s.ok = n < ncol;
  const long e = s.ok ? n / C : 0;
  const long c = s.ok ? n - e * C : 0;
  s.o2 = (size_t)e * q * 2 * C + c;
  s.o1 = (size_t)e * q * C + c;
  return s;
}

// B-operand rows of this lane: r = 4kk + lane / 16, zero past q
template <int QR>
__device__ __forceinline__ void s2_load(const float* __restrict__ p, size_t stride, int q, bool ok,
                                        float (&x)[4 * QR]) {
  const int h = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int kk = 0; kk < 4 * QR; ++kk) {
    const int r = 4 * kk + h;
    x[kk] = (ok && r < q) ? p[(size_t)r * stride] : 0.f;
  }
}

// accumulator rows of this lane: r = 16m + 4 (lane / 16) + i
template <int QR, typename OT>
__device__ __forceinline__ void s2_store(OT* __restrict__ p, size_t stride, int q, bool ok, const s2f4 (&x)[QR]) {
  if (!ok) return;
  const int h = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int m = 0; m < QR; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * m + 4 * h + i;
      if (r < q) st(p + (size_t)r * stride, x[m][i]);
    }
}

// acc += T_t x over the rows (phase 1)
template <int QR>
__device__ __forceinline__ s2f4 s2_rows(const s2f4* __restrict__ tab, int t, const float (&x)[4 * QR], s2f4 acc) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int kq = 0; kq < QR; ++kq) {
    const s2f4 g = tab[(t * QR + kq) * 64 + lane];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc = s2_mma(g[c], x[4 * kq + c], acc);
  }
  return acc;
}

// acc[m] += T_t w over the tile's grid points (phase 2)
template <int QR>
__device__ __forceinline__ void s2_grid(const s2f4* __restrict__ tab, int t, int NT, const s2f4& w, s2f4 (&acc)[QR]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int m = 0; m < QR; ++m) {
    const s2f4 g = tab[(m * NT + t) * 64 + lane];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[m] = s2_mma(g[c], w[c], acc[m]);
  }
}

template <int QR, typename OT>
__global__ __launch_bounds__(kS2Threads) void s2_fwd_kernel(long ncol, int q, int C, int ng, int NT,
                                                           const float* __restrict__ U, const float* __restrict__ G,
                                                           const float* __restrict__ P, OT* __restrict__ Z) {
  extern __shared__ s2f4 s2_lds[];
  s2f4* sGa = s2_lds;
  s2f4* sPb = s2_lds + NT * QR * 64;
  s2_build_rows<QR>(sGa, G, q, 1, q, ng, NT);
  s2_build_grid<QR>(sPb, P, 1, ng, q, ng, NT);
  __syncthreads();
  const long ncb = (ncol + 15) / 16;
  for (long cb = (long)blockIdx.x * kS2Waves + threadIdx.x / 64; cb < ncb; cb += (long)gridDim.x * kS2Waves) {
    const S2Col col = s2_col(cb, ncol, C, q);
    float uv[4 * QR], ug[4 * QR];
    s2_load<QR>(U + col.o2, 2 * C, q, col.ok, uv);
    s2_load<QR>(U + col.o2 + C, 2 * C, q, col.ok, ug);
    s2f4 z[QR];
#pragma unroll
    for (int m = 0; m < QR; ++m) z[m] = s2f4{0.f, 0.f, 0.f, 0.f};
    for (int t = 0; t < NT; ++t) {
      const s2f4 v = s2_rows<QR>(sGa, t, uv, s2f4{0.f, 0.f, 0.f, 0.f});
      const s2f4 a = s2_rows<QR>(sGa, t, ug, s2f4{0.f, 0.f, 0.f, 0.f});
      s2f4 s;
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = a[i] * s2_sigm(a[i]) * v[i];
      s2_grid<QR>(sPb, t, NT, s, z);
    }
    s2_store<QR>(Z + col.o1, C, q, col.ok, z);
  }
}

// gU = [G^T (sb SiLU(a)) ; G^T (sb v SiLU'(a))], sb = P^T gZ
template <int QR, typename OT>
__global__ __launch_bounds__(kS2Threads) void s2_bwd_kernel(long ncol, int q, int C, int ng, int NT,
                                                           const float* __restrict__ U, const float* __restrict__ G,
                                                           const float* __restrict__ P, const float* __restrict__ gZ,
                                                           OT* __restrict__ gU) {
  extern __shared__ s2f4 s2_lds[];
  s2f4* sGa = s2_lds;
  s2f4* sPa = s2_lds + NT * QR * 64;
  s2f4* sGb = s2_lds + 2 * NT * QR * 64;
  s2_build_rows<QR>(sGa, G, q, 1, q, ng, NT);
  s2_build_rows<QR>(sPa, P, 1, ng, q, ng, NT);
  s2_build_grid<QR>(sGb, G, q, 1, q, ng, NT);
  __syncthreads();
  const long ncb = (ncol + 15) / 16;
  for (long cb = (long)blockIdx.x * kS2Waves + threadIdx.x / 64; cb < ncb; cb += (long)gridDim.x * kS2Waves) {
    const S2Col col = s2_col(cb, ncol, C, q);
    float uv[4 * QR], ug[4 * QR], gz[4 * QR];
    s2_load<QR>(U + col.o2, 2 * C, q, col.ok, uv);
    s2_load<QR>(U + col.o2 + C, 2 * C, q, col.ok, ug);
    s2_load<QR>(gZ + col.o1, C, q, col.ok, gz);
    s2f4 bv[QR], bg[QR];
#pragma unroll
    for (int m = 0; m < QR; ++m) bv[m] = bg[m] = s2f4{0.f, 0.f, 0.f, 0.f};
    for (int t = 0; t < NT; ++t) {
      const s2f4 v = s2_rows<QR>(sGa, t, uv, s2f4{0.f, 0.f, 0.f, 0.f});
      const s2f4 a = s2_rows<QR>(sGa, t, ug, s2f4{0.f, 0.f, 0.f, 0.f});
      const s2f4 sb = s2_rows<QR>(sPa, t, gz, s2f4{0.f, 0.f, 0.f, 0.f});
      s2f4 wv, wg;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sg = s2_sigm(a[i]);
        wv[i] = sb[i] * (a[i] * sg);
        wg[i] = sb[i] * v[i] * (sg * (1.f + a[i] * (1.f - sg)));   // SiLU'(a)
      }
      s2_grid<QR>(sGb, t, NT, wv, bv);
      s2_grid<QR>(sGb, t, NT, wg, bg);
    }
    s2_store<QR>(gU + col.o2, 2 * C, q, col.ok, bv);
    s2_store<QR>(gU + col.o2 + C, 2 * C, q, col.ok, bg);
  }
}

// L = <pU, gU>: ggZ = P (SiLU'(a) ad v + SiLU(a) vd), gU2 = G^T [sb ad SiLU'(a) ;
// sb (vd SiLU'(a) + ad v SiLU''(a))] with vd = G pU_v, ad = G pU_g, sb = P^T gZ
template <int QR, typename OT>
__global__ __launch_bounds__(kS2Threads) void s2_dbwd_kernel(long ncol, int q, int C, int ng, int NT,
                                                            const float* __restrict__ U, const float* __restrict__ G,
                                                            const float* __restrict__ P, const float* __restrict__ gZ,
                                                            const float* __restrict__ pU, OT* __restrict__ ggZ,
                                                            OT* __restrict__ gU2) {
  extern __shared__ s2f4 s2_lds[];
  s2f4* sGa = s2_lds;
  s2f4* sPa = s2_lds + NT * QR * 64;
  s2f4* sGb = s2_lds + 2 * NT * QR * 64;
  s2f4* sPb = s2_lds + 3 * NT * QR * 64;
  s2_build_rows<QR>(sGa, G, q, 1, q, ng, NT);
  s2_build_rows<QR>(sPa, P, 1, ng, q, ng, NT);
  s2_build_grid<QR>(sGb, G, q, 1, q, ng, NT);
  s2_build_grid<QR>(sPb, P, 1, ng, q, ng, NT);
  __syncthreads();
  const bool wz = ggZ != nullptr, wu = gU2 != nullptr;
  const long ncb = (ncol + 15) / 16;
  for (long cb = (long)blockIdx.x * kS2Waves + threadIdx.x / 64; cb < ncb; cb += (long)gridDim.x * kS2Waves) {
    const S2Col col = s2_col(cb, ncol, C, q);
    float uv[4 * QR], ug[4 * QR], pv[4 * QR], pg[4 * QR], gz[4 * QR];
    s2_load<QR>(U + col.o2, 2 * C, q, col.ok, uv);
    s2_load<QR>(U + col.o2 + C, 2 * C, q, col.ok, ug);
    s2_load<QR>(pU + col.o2, 2 * C, q, col.ok, pv);
    s2_load<QR>(pU + col.o2 + C, 2 * C, q, col.ok, pg);
    s2_load<QR>(gZ + col.o1, C, q, col.ok && wu, gz);
    s2f4 oz[QR], ov[QR], og[QR];
#pragma unroll
    for (int m = 0; m < QR; ++m) oz[m] = ov[m] = og[m] = s2f4{0.f, 0.f, 0.f, 0.f};
    for (int t = 0; t < NT; ++t) {
      const s2f4 v = s2_rows<QR>(sGa, t, uv, s2f4{0.f, 0.f, 0.f, 0.f});
      const s2f4 a = s2_rows<QR>(sGa, t, ug, s2f4{0.f, 0.f, 0.f, 0.f});
      const s2f4 vd = s2_rows<QR>(sGa, t, pv, s2f4{0.f, 0.f, 0.f, 0.f});
      const s2f4 ad = s2_rows<QR>(sGa, t, pg, s2f4{0.f, 0.f, 0.f, 0.f});
      s2f4 sg, ds;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sg[i] = s2_sigm(a[i]);
        ds[i] = sg[i] * (1.f + a[i] * (1.f - sg[i]));   // SiLU'(a)
      }
      if (wz) {
        s2f4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = ds[i] * ad[i] * v[i] + a[i] * sg[i] * vd[i];
        s2_grid<QR>(sPb, t, NT, w, oz);
      }
      if (wu) {
        const s2f4 sb = s2_rows<QR>(sPa, t, gz, s2f4{0.f, 0.f, 0.f, 0.f});
        s2f4 w1, w2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float dds = sg[i] * (1.f - sg[i]) * (2.f + a[i] * (1.f - 2.f * sg[i]));   // SiLU''(a)
          w1[i] = sb[i] * ad[i] * ds[i];
          w2[i] = sb[i] * (vd[i] * ds[i] + ad[i] * v[i] * dds);
        }
        s2_grid<QR>(sGb, t, NT, w1, ov);
        s2_grid<QR>(sGb, t, NT, w2, og);
      }
    }
    if (wz) s2_store<QR>(ggZ + col.o1, C, q, col.ok, oz);
    if (wu) {
      s2_store<QR>(gU2 + col.o2, 2 * C, q, col.ok, ov);
      s2_store<QR>(gU2 + col.o2 + C, 2 * C, q, col.ok, og);
    }
  }
}

// Reverse pass of the convolution's double backward through the activation,
// with a = the cotangent of the tangent output Zdot and b = the cotangent of
// the primal output Z:
//   o2 = J(U)^T b + d/dU <a, J(U) Ud>     (Ud: the tangent of U)
//   o1 = J(U)^T a                         (optional)
// Per grid point, with v, g the value and gate grid values of U, vd, gd those
// of Ud, sa = P^T a and sb = P^T b:
//   o2 value half: G^T (sb SiLU(g) + sa gd SiLU'(g))
//   o2 gate half : G^T (sb v SiLU'(g) + sa (vd SiLU'(g) + gd v SiLU''(g)))
//   o1           : G^T [sa SiLU(g) ; sa v SiLU'(g)]
template <int QR, typename OT>
__global__ __launch_bounds__(kS2Threads) void s2_rev_kernel(long ncol, int q, int C, int ng, int NT,
                                                           const float* __restrict__ U, const float* __restrict__ G,
                                                           const float* __restrict__ P, const float* __restrict__ Ud,
                                                           const float* __restrict__ Za, const float* __restrict__ Zb,
                                                           OT* __restrict__ o1, OT* __restrict__ o2) {
  extern __shared__ s2f4 s2_lds[];
  s2f4* sGa = s2_lds;
  s2f4* sPa = s2_lds + NT * QR * 64;
  s2f4* sGb = s2_lds + 2 * NT * QR * 64;
  s2_build_rows<QR>(sGa, G, q, 1, q, ng, NT);
  s2_build_rows<QR>(sPa, P, 1, ng, q, ng, NT);
  s2_build_grid<QR>(sGb, G, q, 1, q, ng, NT);
  __syncthreads();
  const bool w1 = o1 != nullptr;
  const long ncb = (ncol + 15) / 16;
  for (long cb = (long)blockIdx.x * kS2Waves + threadIdx.x / 64; cb < ncb; cb += (long)gridDim.x * kS2Waves) {
    const S2Col col = s2_col(cb, ncol, C, q);
    float uv[4 * QR], ug[4 * QR], dv[4 * QR], dg[4 * QR], za[4 * QR], zb[4 * QR];
    s2_load<QR>(U + col.o2, 2 * C, q, col.ok, uv);
    s2_load<QR>(U + col.o2 + C, 2 * C, q, col.ok, ug);
    s2_load<QR>(Ud + col.o2, 2 * C, q, col.ok, dv);
    s2_load<QR>(Ud + col.o2 + C, 2 * C, q, col.ok, dg);
    s2_load<QR>(Za + col.o1, C, q, col.ok, za);
    s2_load<QR>(Zb + col.o1, C, q, col.ok, zb);
    s2f4 av[QR], ag[QR], bv[QR], bg[QR];
#pragma unroll
    for (int m = 0; m < QR; ++m) av[m] = ag[m] = bv[m] = bg[m] = s2f4{0.f, 0.f, 0.f, 0.f};
    for (int t = 0; t < NT; ++t) {
      const s2f4 v = s2_rows<QR>(sGa, t, uv, s2f4{0.f, 0.f, 0.f, 0.f});
      const s2f4 g = s2_rows<QR>(sGa, t, ug, s2f4{0.f, 0.f, 0.f, 0.f});
      const s2f4 vd = s2_rows<QR>(sGa, t, dv, s2f4{0.f, 0.f, 0.f, 0.f});
      const s2f4 gd = s2_rows<QR>(sGa, t, dg, s2f4{0.f, 0.f, 0.f, 0.f});
      const s2f4 sa = s2_rows<QR>(sPa, t, za, s2f4{0.f, 0.f, 0.f, 0.f});
      const s2f4 sb = s2_rows<QR>(sPa, t, zb, s2f4{0.f, 0.f, 0.f, 0.f});
      s2f4 wv, wg, xv, xg;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sg = s2_sigm(g[i]);
        const float si = g[i] * sg;                                               // SiLU(g)
        const float ds = sg * (1.f + g[i] * (1.f - sg));                          // SiLU'(g)
        const float dds = sg * (1.f - sg) * (2.f + g[i] * (1.f - 2.f * sg));      // SiLU''(g)
        wv[i] = sb[i] * si + sa[i] * gd[i] * ds;
        wg[i] = sb[i] * v[i] * ds + sa[i] * (vd[i] * ds + gd[i] * v[i] * dds);
        xv[i] = sa[i] * si;
        xg[i] = sa[i] * v[i] * ds;
      }
      s2_grid<QR>(sGb, t, NT, wv, bv);
      s2_grid<QR>(sGb, t, NT, wg, bg);
      if (w1) {
        s2_grid<QR>(sGb, t, NT, xv, av);
        s2_grid<QR>(sGb, t, NT, xg, ag);
      }
    }
    s2_store<QR>(o2 + col.o2, 2 * C, q, col.ok, bv);
    s2_store<QR>(o2 + col.o2 + C, 2 * C, q, col.ok, bg);
    if (w1) {
      s2_store<QR>(o1 + col.o2, 2 * C, q, col.ok, av);
      s2_store<QR>(o1 + col.o2 + C, 2 * C, q, col.ok, ag);
    }
  }
}

// Grid tables of the convolution's activation, from the caller's degree-major
// retained rows (l = 0..L, m = -min(l,M)..min(l,M)) to the m-major row order
// of the edge arrays: Gm[g][mm(l,m)] = G[g][dm(l,m)], Pm[mm(l,m)][g] = P[dm(l,m)][g].
__global__ void s2_mmajor_kernel(int L, int M, int ng, const float* __restrict__ G, const float* __restrict__ P,
                                 float* __restrict__ Gm, float* __restrict__ Pm) {
  const int q = q_count(L, M);
  for (int idx = blockIdx.x * blockDim.x + threadIdx.x; idx < ng * q; idx += gridDim.x * blockDim.x) {
    const int g = idx / q, rd = idx - g * q;
    int l = 0, base = 0;
    while (rd >= base + 2 * qhalf(l, M) + 1) {
      base += 2 * qhalf(l, M) + 1;
      ++l;
    }
    const int m = rd - base - qhalf(l, M);
    const int rm = mm_col(l, m, 0, L, 1);
    Gm[(size_t)g * q + rm] = G[(size_t)g * q + rd];
    Pm[(size_t)rm * ng + g] = P[(size_t)rd * ng + g];
  }
}

struct S2Launch {
  dim3 grid;
  size_t lds;
  int NT;
};
// tables: count of staged constant operands (fwd 2, bwd 3, dbwd 4)
S2Launch s2_launch(long ncol, int q, int ng, int tables) {
  const int QR = q <= 16 ? 1 : 2, NT = (ng + 15) / 16;
  const long ncb = (ncol + 15) / 16;
  long nb = (ncb + kS2Waves - 1) / kS2Waves;
  if (nb > kS2MaxBlocks) nb = kS2MaxBlocks;
  return {dim3((unsigned)(nb > 0 ? nb : 1)), (size_t)tables * NT * QR * 64 * sizeof(s2f4), NT};
}

// dynamic LDS beyond the default limit has to be requested per kernel
template <typename K>
hipError_t s2_allow_lds(K* kernel, size_t lds) {
  if (lds <= 32768) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)lds);
}

// ---------------------------------------------------------------- bfloat16 variant
// For bfloat16 calls of the convolution the grid products take bfloat16
// operands (the first linear's float32 output rows, the grid tables and the
// SwiGLU values rounded to nearest even) with float32 accumulation on
// v_mfma_f32_32x32x16_bf16, sixteen times the float32 matrix rate; the
// nonlinearity and its derivatives stay float32. A wave takes 32 columns:
//   phase 1  grid tile t of 32 points: V = G_t U over the rows in steps of
//            16 (lane (j, h) carries rows 16 s + 8 h + k of column j);
//   phase 2  Z += P_t S_t in two steps of 16 grid points; lane (j, h) holds
//            the accumulator elements 4 g + i = grid points 8 g + 4 h + i of
//            its column, and slot k of step u takes g = 2 u + k / 4,
//            i = k mod 4, so S_t feeds the next product without a transpose;
//            the tables are staged in LDS with the same slot order.
typedef __bf16 s2b8 __attribute__((ext_vector_type(8)));
typedef float s2f16 __attribute__((ext_vector_type(16)));
typedef unsigned s2u4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ s2f16 s2b_mma(const s2u4& a, const s2u4& b, const s2f16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(s2b8, a), __builtin_bit_cast(s2b8, b), c, 0, 0,
                                                  0);
}
__device__ __forceinline__ s2u4 s2b_pack(const float (&x)[8]) {
  s2u4 u;
#pragma unroll
  for (int q = 0; q < 4; ++q) u[q] = (unsigned)f32_to_bf16(x[2 * q]) | ((unsigned)f32_to_bf16(x[2 * q + 1]) << 16);
  return u;
}
__device__ __forceinline__ s2f16 s2b_zero() {
  s2f16 z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

// rows form (K over rows): fragment (t, s), lane (i, h): M(32 t + i, 16 s + 8 h + k), k < 8
template <int QS>
__device__ void s2b_build_rows(s2u4* dst, const float* __restrict__ src, int sg, int sr, int q, int ng, int NT) {
  const int n = NT * QS * 64;
  for (int idx = threadIdx.x; idx < n; idx += blockDim.x) {
    const int lane = idx & 63, f = idx >> 6, sq = f % QS, t = f / QS;
    const int gp = 32 * t + (lane & 31), h = lane >> 5;
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = 16 * sq + 8 * h + k;
      x[k] = (gp < ng && r < q) ? src[(size_t)gp * sg + (size_t)r * sr] : 0.f;
    }
    dst[idx] = s2b_pack(x);
  }
}
// grid form (K over grid points): fragment (t, u), lane (r, h): M(32 t + 16 u + 8 (k/4) + 4 h + k%4, r)
__device__ void s2b_build_grid(s2u4* dst, const float* __restrict__ src, int sg, int sr, int q, int ng, int NT) {
  const int n = NT * 2 * 64;
  for (int idx = threadIdx.x; idx < n; idx += blockDim.x) {
    const int lane = idx & 63, f = idx >> 6, u = f & 1, t = f >> 1;
    const int r = lane & 31, h = lane >> 5;
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int gp = 32 * t + 16 * u + 8 * (k / 4) + 4 * h + (k % 4);
      x[k] = (gp < ng && r < q) ? src[(size_t)gp * sg + (size_t)r * sr] : 0.f;
    }
    dst[idx] = s2b_pack(x);
  }
}

struct S2BCol {
  size_t o2, o1;
  bool ok;
};
__device__ __forceinline__ S2BCol s2b_col(long cb, long ncol, int C, int q) {
  const long n = cb * 32 + (threadIdx.x & 31);
  S2BCol s;
  s.ok = n < ncol;
  const long e = s.ok ? n / C : 0;
  const long c = s.ok ? n - e * C : 0;
  s.o2 = (size_t)e * q * 2 * C + c;
  s.o1 = (size_t)e * q * C + c;
  return s;
}
// rows 16 s + 8 h + k of this lane's column, packed per step
template <int QS>
__device__ __forceinline__ void s2b_load(const float* __restrict__ p, size_t stride, int q, bool ok, s2u4 (&x)[QS]) {
  const int h = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int sq = 0; sq < QS; ++sq) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = 16 * sq + 8 * h + k;
      v[k] = (ok && r < q) ? p[(size_t)r * stride] : 0.f;
    }
    x[sq] = s2b_pack(v);
  }
}
// accumulator rows 8 g + 4 h + i of this lane's column
template <typename OT>
__device__ __forceinline__ void s2b_store(OT* __restrict__ p, size_t stride, int q, bool ok, const s2f16& x) {
  if (!ok) return;
  const int h = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 8 * g + 4 * h + i;
      if (r < q) st(p + (size_t)r * stride, x[4 * g + i]);
    }
}
// phase 1: rows-form table fragments of grid tile t times the packed rows
template <int QS>
__device__ __forceinline__ s2f16 s2b_rows(const s2u4* __restrict__ tab, int t, const s2u4 (&x)[QS]) {
  const int lane = threadIdx.x & 63;
  s2f16 acc = s2b_zero();
#pragma unroll
  for (int sq = 0; sq < QS; ++sq) acc = s2b_mma(tab[(t * QS + sq) * 64 + lane], x[sq], acc);
  return acc;
}
// phase 2: acc += grid-form table fragments (t, 0..1) times the grid values w
__device__ __forceinline__ void s2b_grid(const s2u4* __restrict__ tab, int t, const s2f16& w, s2f16& acc) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = w[(2 * u + k / 4) * 4 + (k % 4)];
    acc = s2b_mma(tab[(t * 2 + u) * 64 + lane], s2b_pack(x), acc);
  }
}

template <int QS, typename OT>
__global__ __launch_bounds__(kS2Threads) void s2b_fwd_kernel(long ncol, int q, int C, int ng, int NT,
                                                            const float* __restrict__ U, const float* __restrict__ G,
                                                            const float* __restrict__ P, OT* __restrict__ Z) {
  extern __shared__ s2u4 s2b_lds[];
  s2u4* tG = s2b_lds;
  s2u4* tP = s2b_lds + NT * QS * 64;
  s2b_build_rows<QS>(tG, G, q, 1, q, ng, NT);
  s2b_build_grid(tP, P, 1, ng, q, ng, NT);
  __syncthreads();
  const long ncb = (ncol + 31) / 32;
  for (long cb = (long)blockIdx.x * kS2Waves + threadIdx.x / 64; cb < ncb; cb += (long)gridDim.x * kS2Waves) {
    const S2BCol col = s2b_col(cb, ncol, C, q);
    s2u4 uv[QS], ug[QS];
    s2b_load<QS>(U + col.o2, 2 * C, q, col.ok, uv);
    s2b_load<QS>(U + col.o2 + C, 2 * C, q, col.ok, ug);
    s2f16 z = s2b_zero();
    for (int t = 0; t < NT; ++t) {
      const s2f16 v = s2b_rows<QS>(tG, t, uv), a = s2b_rows<QS>(tG, t, ug);
      s2f16 w;
#pragma unroll
      for (int r = 0; r < 16; ++r) w[r] = a[r] * s2_sigm(a[r]) * v[r];
      s2b_grid(tP, t, w, z);
    }
    s2b_store(Z + col.o1, C, q, col.ok, z);
  }
}

template <int QS, typename OT>
__global__ __launch_bounds__(kS2Threads) void s2b_bwd_kernel(long ncol, int q, int C, int ng, int NT,
                                                            const float* __restrict__ U, const float* __restrict__ G,
                                                            const float* __restrict__ P, const float* __restrict__ gZ,
                                                            OT* __restrict__ gU) {
  extern __shared__ s2u4 s2b_lds[];
  s2u4* tG = s2b_lds;
  s2u4* tPt = s2b_lds + NT * QS * 64;
  s2u4* tGt = s2b_lds + 2 * NT * QS * 64;
  s2b_build_rows<QS>(tG, G, q, 1, q, ng, NT);
  s2b_build_rows<QS>(tPt, P, 1, ng, q, ng, NT);
  s2b_build_grid(tGt, G, q, 1, q, ng, NT);
  __syncthreads();
  const long ncb = (ncol + 31) / 32;
  for (long cb = (long)blockIdx.x * kS2Waves + threadIdx.x / 64; cb < ncb; cb += (long)gridDim.x * kS2Waves) {
    const S2BCol col = s2b_col(cb, ncol, C, q);
    s2u4 uv[QS], ug[QS], gz[QS];
    s2b_load<QS>(U + col.o2, 2 * C, q, col.ok, uv);
    s2b_load<QS>(U + col.o2 + C, 2 * C, q, col.ok, ug);
    s2b_load<QS>(gZ + col.o1, C, q, col.ok, gz);
    s2f16 bv = s2b_zero(), bg = s2b_zero();
    for (int t = 0; t < NT; ++t) {
      const s2f16 v = s2b_rows<QS>(tG, t, uv), a = s2b_rows<QS>(tG, t, ug), sb = s2b_rows<QS>(tPt, t, gz);
      s2f16 wv, wg;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float sg = s2_sigm(a[r]);
        wv[r] = sb[r] * (a[r] * sg);
        wg[r] = sb[r] * v[r] * (sg * (1.f + a[r] * (1.f - sg)));   // SiLU'(a)
      }
      s2b_grid(tGt, t, wv, bv);
      s2b_grid(tGt, t, wg, bg);
    }
    s2b_store(gU + col.o2, 2 * C, q, col.ok, bv);
    s2b_store(gU + col.o2 + C, 2 * C, q, col.ok, bg);
  }
}

// the forward's directional derivative along pU: ggZ = P (SiLU'(a) ad v + SiLU(a) vd)
template <int QS, typename OT>
__global__ __launch_bounds__(kS2Threads) void s2b_dual_kernel(long ncol, int q, int C, int ng, int NT,
                                                             const float* __restrict__ U, const float* __restrict__ G,
                                                             const float* __restrict__ P,
                                                             const float* __restrict__ pU, OT* __restrict__ ggZ) {
  extern __shared__ s2u4 s2b_lds[];
  s2u4* tG = s2b_lds;
  s2u4* tP = s2b_lds + NT * QS * 64;
  s2b_build_rows<QS>(tG, G, q, 1, q, ng, NT);
  s2b_build_grid(tP, P, 1, ng, q, ng, NT);
  __syncthreads();
  const long ncb = (ncol + 31) / 32;
  for (long cb = (long)blockIdx.x * kS2Waves + threadIdx.x / 64; cb < ncb; cb += (long)gridDim.x * kS2Waves) {
    const S2BCol col = s2b_col(cb, ncol, C, q);
    s2u4 uv[QS], ug[QS], pv[QS], pg[QS];
    s2b_load<QS>(U + col.o2, 2 * C, q, col.ok, uv);
    s2b_load<QS>(U + col.o2 + C, 2 * C, q, col.ok, ug);
    s2b_load<QS>(pU + col.o2, 2 * C, q, col.ok, pv);
    s2b_load<QS>(pU + col.o2 + C, 2 * C, q, col.ok, pg);
    s2f16 oz = s2b_zero();
    for (int t = 0; t < NT; ++t) {
      const s2f16 v = s2b_rows<QS>(tG, t, uv), a = s2b_rows<QS>(tG, t, ug);
      const s2f16 vd = s2b_rows<QS>(tG, t, pv), ad = s2b_rows<QS>(tG, t, pg);
      s2f16 w;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float sg = s2_sigm(a[r]);
        w[r] = sg * (1.f + a[r] * (1.f - sg)) * ad[r] * v[r] + a[r] * sg * vd[r];
      }
      s2b_grid(tP, t, w, oz);
    }
    s2b_store(ggZ + col.o1, C, q, col.ok, oz);
  }
}

// reverse pass of the double backward, o2 of s2_rev_kernel (J^T a, the
// other output, is the backward kernel's product with a as the cotangent)
template <int QS, typename OT>
__global__ __launch_bounds__(kS2Threads) void s2b_rev_kernel(long ncol, int q, int C, int ng, int NT,
                                                            const float* __restrict__ U, const float* __restrict__ G,
                                                            const float* __restrict__ P, const float* __restrict__ Ud,
                                                            const float* __restrict__ Za, const float* __restrict__ Zb,
                                                            OT* __restrict__ o2) {
  extern __shared__ s2u4 s2b_lds[];
  s2u4* tG = s2b_lds;
  s2u4* tPt = s2b_lds + NT * QS * 64;
  s2u4* tGt = s2b_lds + 2 * NT * QS * 64;
  s2b_build_rows<QS>(tG, G, q, 1, q, ng, NT);
  s2b_build_rows<QS>(tPt, P, 1, ng, q, ng, NT);
  s2b_build_grid(tGt, G, q, 1, q, ng, NT);
  __syncthreads();
  const long ncb = (ncol + 31) / 32;
  for (long cb = (long)blockIdx.x * kS2Waves + threadIdx.x / 64; cb < ncb; cb += (long)gridDim.x * kS2Waves) {
    const S2BCol col = s2b_col(cb, ncol, C, q);
    s2u4 uv[QS], ug[QS], dv[QS], dg[QS], za[QS], zb[QS];
    s2b_load<QS>(U + col.o2, 2 * C, q, col.ok, uv);
    s2b_load<QS>(U + col.o2 + C, 2 * C, q, col.ok, ug);
    s2b_load<QS>(Ud + col.o2, 2 * C, q, col.ok, dv);
    s2b_load<QS>(Ud + col.o2 + C, 2 * C, q, col.ok, dg);
    s2b_load<QS>(Za + col.o1, C, q, col.ok, za);
    s2b_load<QS>(Zb + col.o1, C, q, col.ok, zb);
    s2f16 bv = s2b_zero(), bg = s2b_zero();
    for (int t = 0; t < NT; ++t) {
      const s2f16 v = s2b_rows<QS>(tG, t, uv), g = s2b_rows<QS>(tG, t, ug);
      const s2f16 vd = s2b_rows<QS>(tG, t, dv), gd = s2b_rows<QS>(tG, t, dg);
      const s2f16 sa = s2b_rows<QS>(tPt, t, za), sb = s2b_rows<QS>(tPt, t, zb);
      s2f16 wv, wg;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float sg = s2_sigm(g[r]);
        const float ds = sg * (1.f + g[r] * (1.f - sg));
        const float dds = sg * (1.f - sg) * (2.f + g[r] * (1.f - 2.f * sg));
        wv[r] = sb[r] * (g[r] * sg) + sa[r] * gd[r] * ds;
        wg[r] = sb[r] * v[r] * ds + sa[r] * (vd[r] * ds + gd[r] * v[r] * dds);
      }
      s2b_grid(tGt, t, wv, bv);
      s2b_grid(tGt, t, wg, bg);
    }
    s2b_store(o2 + col.o2, 2 * C, q, col.ok, bv);
    s2b_store(o2 + col.o2 + C, 2 * C, q, col.ok, bg);
  }
}

// launch shape of the bfloat16 variant: rows-form tables NT QS KB each, grid-form NT 2 KB each
S2Launch s2b_launch(long ncol, int q, int ng, int rows_tables, int grid_tables) {
  const int QS = q <= 16 ? 1 : 2, NT = (ng + 31) / 32;
  const long ncb = (ncol + 31) / 32;
  long nb = (ncb + kS2Waves - 1) / kS2Waves;
  if (nb > kS2MaxBlocks) nb = kS2MaxBlocks;
  return {dim3((unsigned)(nb > 0 ? nb : 1)), (size_t)(rows_tables * QS + 2 * grid_tables) * NT * 64 * sizeof(s2u4),
          NT};
}

}  // namespace

#define SO2_S2_LAUNCH_T(KERNEL, OT, TABLES, ...)                                                       \
  do {                                                                                                  \
    const long ncol_ = E * (long)C;                                                                     \
    const S2Launch L_ = s2_launch(ncol_, q, ng, TABLES);                                                \
    hipError_t st_;                                                                                     \
    if (q <= 16) {                                                                                      \
      if ((st_ = s2_allow_lds(KERNEL<1, OT>, L_.lds)) != hipSuccess) return st_;                        \
      hipLaunchKernelGGL((KERNEL<1, OT>), L_.grid, dim3(kS2Threads), L_.lds, s, ncol_, q, C, ng, L_.NT, \
                         __VA_ARGS__);                                                                  \
    } else {                                                                                            \
      if ((st_ = s2_allow_lds(KERNEL<2, OT>, L_.lds)) != hipSuccess) return st_;                        \
      hipLaunchKernelGGL((KERNEL<2, OT>), L_.grid, dim3(kS2Threads), L_.lds, s, ncol_, q, C, ng, L_.NT, \
                         __VA_ARGS__);                                                                  \
    }                                                                                                   \
  } while (0)

// outputs of the operand type: float32, or bfloat16 (bf16 != 0)
#define SO2_S2B_LAUNCH(KERNEL, RT, GT, ...)                                                            \
  do {                                                                                                  \
    const long ncol_ = E * (long)C;                                                                     \
    const S2Launch L_ = s2b_launch(ncol_, q, ng, RT, GT);                                               \
    hipError_t st_;                                                                                     \
    if (q <= 16) {                                                                                      \
      if ((st_ = s2_allow_lds(KERNEL<1, bf16s>, L_.lds)) != hipSuccess) return st_;                     \
      hipLaunchKernelGGL((KERNEL<1, bf16s>), L_.grid, dim3(kS2Threads), L_.lds, s, ncol_, q, C, ng, L_.NT, \
                         __VA_ARGS__);                                                                  \
    } else {                                                                                            \
      if ((st_ = s2_allow_lds(KERNEL<2, bf16s>, L_.lds)) != hipSuccess) return st_;                     \
      hipLaunchKernelGGL((KERNEL<2, bf16s>), L_.grid, dim3(kS2Threads), L_.lds, s, ncol_, q, C, ng, L_.NT, \
                         __VA_ARGS__);                                                                  \
    }                                                                                                   \
  } while (0)

int launch_s2_fwd(long E, int q, int C, int ng, const float* U, const float* G, const float* P, void* Z, int bf16,
                  hipStream_t s) {
  if (E == 0) return hipSuccess;
  if (bf16) SO2_S2B_LAUNCH(s2b_fwd_kernel, 1, 1, U, G, P, static_cast<bf16s*>(Z));
  else SO2_S2_LAUNCH_T(s2_fwd_kernel, float, 2, U, G, P, static_cast<float*>(Z));
  return hipGetLastError();
}

int launch_s2_bwd(long E, int q, int C, int ng, const float* U, const float* G, const float* P, const float* gZ,
                  void* gU, int bf16, hipStream_t s) {
  if (E == 0) return hipSuccess;
  if (bf16) SO2_S2B_LAUNCH(s2b_bwd_kernel, 2, 1, U, G, P, gZ, static_cast<bf16s*>(gU));
  else SO2_S2_LAUNCH_T(s2_bwd_kernel, float, 3, U, G, P, gZ, static_cast<float*>(gU));
  return hipGetLastError();
}

int launch_s2_dbwd(long E, int q, int C, int ng, const float* U, const float* G, const float* P, const float* gZ,
                   const float* pU, void* ggZ, void* gU2, int bf16, hipStream_t s) {
  if (E == 0) return hipSuccess;
  if (bf16 && !gU2)   // the tangent of the convolution's double backward
    SO2_S2B_LAUNCH(s2b_dual_kernel, 1, 1, U, G, P, pU, static_cast<bf16s*>(ggZ));
  else if (bf16)
    SO2_S2_LAUNCH_T(s2_dbwd_kernel, bf16s, 4, U, G, P, gZ, pU, static_cast<bf16s*>(ggZ), static_cast<bf16s*>(gU2));
  else
    SO2_S2_LAUNCH_T(s2_dbwd_kernel, float, 4, U, G, P, gZ, pU, static_cast<float*>(ggZ), static_cast<float*>(gU2));
  return hipGetLastError();
}

int launch_s2_rev(long E, int q, int C, int ng, const float* U, const float* G, const float* P, const float* Ud,
                  const float* Za, const float* Zb, void* o1, void* o2, int bf16, hipStream_t s) {
  if (E == 0) return hipSuccess;
  if (bf16) {
    if (o1) SO2_S2B_LAUNCH(s2b_bwd_kernel, 2, 1, U, G, P, Za, static_cast<bf16s*>(o1));
    SO2_S2B_LAUNCH(s2b_rev_kernel, 2, 1, U, G, P, Ud, Za, Zb, static_cast<bf16s*>(o2));
  }
  else
    SO2_S2_LAUNCH_T(s2_rev_kernel, float, 3, U, G, P, Ud, Za, Zb, static_cast<float*>(o1), static_cast<float*>(o2));
  return hipGetLastError();
}

int launch_s2_mmajor(int L, int M, int ng, const float* G, const float* P, float* Gm, float* Pm, hipStream_t s) {
  const int n = ng * q_count(L, M);
  hipLaunchKernelGGL(s2_mmajor_kernel, dim3((n + 255) / 256), dim3(256), 0, s, L, M, ng, G, P, Gm, Pm);
  return hipGetLastError();
}

}  // namespace so2
