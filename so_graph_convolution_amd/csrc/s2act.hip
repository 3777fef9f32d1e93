// Spherical-grid SwiGLU activation on edges (SwiGLU-S2): TrimSO(2) page,
// Table 5 (EquiformerV3's activation), Section 5.1 (its Edge -> Edge
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
template <int QR>
__device__ __forceinline__ void s2_store(float* __restrict__ p, size_t stride, int q, bool ok, const s2f4 (&x)[QR]) {
  if (!ok) return;
  const int h = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int m = 0; m < QR; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * m + 4 * h + i;
      if (r < q) p[(size_t)r * stride] = x[m][i];
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

template <int QR>
__global__ __launch_bounds__(kS2Threads) void s2_fwd_kernel(long ncol, int q, int C, int ng, int NT,
                                                           const float* __restrict__ U, const float* __restrict__ G,
                                                           const float* __restrict__ P, float* __restrict__ Z) {
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
template <int QR>
__global__ __launch_bounds__(kS2Threads) void s2_bwd_kernel(long ncol, int q, int C, int ng, int NT,
                                                           const float* __restrict__ U, const float* __restrict__ G,
                                                           const float* __restrict__ P, const float* __restrict__ gZ,
                                                           float* __restrict__ gU) {
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
template <int QR>
__global__ __launch_bounds__(kS2Threads) void s2_dbwd_kernel(long ncol, int q, int C, int ng, int NT,
                                                            const float* __restrict__ U, const float* __restrict__ G,
                                                            const float* __restrict__ P, const float* __restrict__ gZ,
                                                            const float* __restrict__ pU, float* __restrict__ ggZ,
                                                            float* __restrict__ gU2) {
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

}  // namespace

#define SO2_S2_LAUNCH(KERNEL, TABLES, ...)                                                              \
  do {                                                                                                  \
    const long ncol_ = E * (long)C;                                                                     \
    const S2Launch L_ = s2_launch(ncol_, q, ng, TABLES);                                                \
    hipError_t st_;                                                                                     \
    if (q <= 16) {                                                                                      \
      if ((st_ = s2_allow_lds(KERNEL<1>, L_.lds)) != hipSuccess) return st_;                            \
      hipLaunchKernelGGL((KERNEL<1>), L_.grid, dim3(kS2Threads), L_.lds, s, ncol_, q, C, ng, L_.NT,     \
                         __VA_ARGS__);                                                                  \
    } else {                                                                                            \
      if ((st_ = s2_allow_lds(KERNEL<2>, L_.lds)) != hipSuccess) return st_;                            \
      hipLaunchKernelGGL((KERNEL<2>), L_.grid, dim3(kS2Threads), L_.lds, s, ncol_, q, C, ng, L_.NT,     \
                         __VA_ARGS__);                                                                  \
    }                                                                                                   \
  } while (0)

int launch_s2_fwd(long E, int q, int C, int ng, const float* U, const float* G, const float* P, float* Z,
                  hipStream_t s) {
  if (E == 0) return hipSuccess;
  SO2_S2_LAUNCH(s2_fwd_kernel, 2, U, G, P, Z);
  return hipGetLastError();
}

int launch_s2_bwd(long E, int q, int C, int ng, const float* U, const float* G, const float* P, const float* gZ,
                  float* gU, hipStream_t s) {
  if (E == 0) return hipSuccess;
  SO2_S2_LAUNCH(s2_bwd_kernel, 3, U, G, P, gZ, gU);
  return hipGetLastError();
}

int launch_s2_dbwd(long E, int q, int C, int ng, const float* U, const float* G, const float* P, const float* gZ,
                   const float* pU, float* ggZ, float* gU2, hipStream_t s) {
  if (E == 0) return hipSuccess;
  SO2_S2_LAUNCH(s2_dbwd_kernel, 4, U, G, P, gZ, pU, ggZ, gU2);
  return hipGetLastError();
}

}  // namespace so2
