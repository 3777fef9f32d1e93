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
// One thread per (edge, channel): its q values of each half stay in registers
// (QM >= q, compile-time), G and P^T are staged in LDS and read as broadcasts,
// and the grid points are visited one at a time, so no grid value is stored.
// The backward and double backward recompute v and a the same way.
#include "ops.hpp"

namespace so2 {

namespace {

constexpr int kS2Threads = 256;

__device__ __forceinline__ float s2_sigm(float a) { return 1.f / (1.f + __expf(-a)); }

// G and P^T into LDS (both [n_g][q])
__device__ inline void s2_stage(const float* __restrict__ G, const float* __restrict__ P, int q, int ng, float* sG,
                                float* sPT) {
  for (int i = threadIdx.x; i < ng * q; i += blockDim.x) {
    const int gp = i / q, r = i - gp * q;
    sG[i] = G[i];
    sPT[i] = P[r * ng + gp];
  }
  __syncthreads();
}

template <int QM>
__device__ __forceinline__ float s2_dot(const float* row, const float (&x)[QM], int q) {
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < QM; ++r)
    if (r < q) s += row[r] * x[r];
  return s;
}

template <int QM>
__device__ __forceinline__ void s2_axpy(const float* row, float w, float (&y)[QM], int q) {
#pragma unroll
  for (int r = 0; r < QM; ++r)
    if (r < q) y[r] += row[r] * w;
}

template <int QM>
__device__ __forceinline__ void s2_load(const float* p, int stride, int q, float (&x)[QM]) {
#pragma unroll
  for (int r = 0; r < QM; ++r) x[r] = r < q ? p[(size_t)r * stride] : 0.f;
}

template <int QM>
__device__ __forceinline__ void s2_store(float* p, int stride, int q, const float (&x)[QM]) {
#pragma unroll
  for (int r = 0; r < QM; ++r)
    if (r < q) p[(size_t)r * stride] = x[r];
}

// thread -> (edge slot, channel); EPB edges per block and step
struct S2Map {
  int c, slot, epb;
  bool act;
};
__device__ inline S2Map s2_map(int C) {
  S2Map m;
  m.epb = C >= kS2Threads ? 1 : kS2Threads / C;
  m.c = threadIdx.x % C;
  m.slot = threadIdx.x / C;
  m.act = m.slot < m.epb && m.c < C;
  return m;
}

template <int QM>
__global__ __launch_bounds__(kS2Threads) void s2_fwd_kernel(long E, int q, int C, int ng, const float* __restrict__ U,
                                                           const float* __restrict__ G, const float* __restrict__ P,
                                                           float* __restrict__ Z) {
  extern __shared__ float s2_lds[];
  float* sG = s2_lds;
  float* sPT = s2_lds + ng * q;
  s2_stage(G, P, q, ng, sG, sPT);
  const S2Map mp = s2_map(C);
  if (!mp.act) return;
  for (long e = (long)blockIdx.x * mp.epb + mp.slot; e < E; e += (long)gridDim.x * mp.epb) {
    const float* u = U + (size_t)e * q * 2 * C + mp.c;
    float uv[QM], ug[QM], z[QM];
    s2_load<QM>(u, 2 * C, q, uv);
    s2_load<QM>(u + C, 2 * C, q, ug);
#pragma unroll
    for (int r = 0; r < QM; ++r) z[r] = 0.f;
    for (int gp = 0; gp < ng; ++gp) {
      const float* grow = sG + gp * q;
      const float v = s2_dot<QM>(grow, uv, q), a = s2_dot<QM>(grow, ug, q);
      s2_axpy<QM>(sPT + gp * q, a * s2_sigm(a) * v, z, q);
    }
    s2_store<QM>(Z + (size_t)e * q * C + mp.c, C, q, z);
  }
}

template <int QM>
__global__ __launch_bounds__(kS2Threads) void s2_bwd_kernel(long E, int q, int C, int ng, const float* __restrict__ U,
                                                           const float* __restrict__ G, const float* __restrict__ P,
                                                           const float* __restrict__ gZ, float* __restrict__ gU) {
  extern __shared__ float s2_lds[];
  float* sG = s2_lds;
  float* sPT = s2_lds + ng * q;
  s2_stage(G, P, q, ng, sG, sPT);
  const S2Map mp = s2_map(C);
  if (!mp.act) return;
  for (long e = (long)blockIdx.x * mp.epb + mp.slot; e < E; e += (long)gridDim.x * mp.epb) {
    const float* u = U + (size_t)e * q * 2 * C + mp.c;
    float uv[QM], ug[QM], gz[QM], bv[QM], bg[QM];
    s2_load<QM>(u, 2 * C, q, uv);
    s2_load<QM>(u + C, 2 * C, q, ug);
    s2_load<QM>(gZ + (size_t)e * q * C + mp.c, C, q, gz);
#pragma unroll
    for (int r = 0; r < QM; ++r) bv[r] = bg[r] = 0.f;
    for (int gp = 0; gp < ng; ++gp) {
      const float* grow = sG + gp * q;
      const float v = s2_dot<QM>(grow, uv, q), a = s2_dot<QM>(grow, ug, q);
      const float sb = s2_dot<QM>(sPT + gp * q, gz, q);   // (P^T gz) at this grid point
      const float sg = s2_sigm(a);
      const float ds = sg * (1.f + a * (1.f - sg));      // SiLU'(a)
      s2_axpy<QM>(grow, sb * (a * sg), bv, q);
      s2_axpy<QM>(grow, sb * v * ds, bg, q);
    }
    float* g = gU + (size_t)e * q * 2 * C + mp.c;
    s2_store<QM>(g, 2 * C, q, bv);
    s2_store<QM>(g + C, 2 * C, q, bg);
  }
}

// L = <pU, gU>: ggZ = P (SiLU'(a) ad v + SiLU(a) vd), gU2 = G^T [sb ad SiLU'(a) ;
// sb (vd SiLU'(a) + ad v SiLU''(a))] with vd = G pU_v, ad = G pU_g, sb = P^T gZ
template <int QM>
__global__ __launch_bounds__(kS2Threads) void s2_dbwd_kernel(long E, int q, int C, int ng, const float* __restrict__ U,
                                                            const float* __restrict__ G, const float* __restrict__ P,
                                                            const float* __restrict__ gZ, const float* __restrict__ pU,
                                                            float* __restrict__ ggZ, float* __restrict__ gU2) {
  extern __shared__ float s2_lds[];
  float* sG = s2_lds;
  float* sPT = s2_lds + ng * q;
  s2_stage(G, P, q, ng, sG, sPT);
  const S2Map mp = s2_map(C);
  if (!mp.act) return;
  for (long e = (long)blockIdx.x * mp.epb + mp.slot; e < E; e += (long)gridDim.x * mp.epb) {
    const size_t o2 = (size_t)e * q * 2 * C + mp.c, o1 = (size_t)e * q * C + mp.c;
    float uv[QM], ug[QM], pv[QM], pg[QM], gz[QM], oz[QM], ov[QM], og[QM];
    s2_load<QM>(U + o2, 2 * C, q, uv);
    s2_load<QM>(U + o2 + C, 2 * C, q, ug);
    s2_load<QM>(pU + o2, 2 * C, q, pv);
    s2_load<QM>(pU + o2 + C, 2 * C, q, pg);
    if (gU2) s2_load<QM>(gZ + o1, C, q, gz);
#pragma unroll
    for (int r = 0; r < QM; ++r) oz[r] = ov[r] = og[r] = 0.f;
    for (int gp = 0; gp < ng; ++gp) {
      const float* grow = sG + gp * q;
      const float v = s2_dot<QM>(grow, uv, q), a = s2_dot<QM>(grow, ug, q);
      const float vd = s2_dot<QM>(grow, pv, q), ad = s2_dot<QM>(grow, pg, q);
      const float sg = s2_sigm(a);
      const float ds = sg * (1.f + a * (1.f - sg));                       // SiLU'(a)
      if (ggZ) s2_axpy<QM>(sPT + gp * q, ds * ad * v + a * sg * vd, oz, q);
      if (gU2) {
        const float sb = s2_dot<QM>(sPT + gp * q, gz, q);
        const float dds = sg * (1.f - sg) * (2.f + a * (1.f - 2.f * sg));  // SiLU''(a)
        s2_axpy<QM>(grow, sb * ad * ds, ov, q);
        s2_axpy<QM>(grow, sb * (vd * ds + ad * v * dds), og, q);
      }
    }
    if (ggZ) s2_store<QM>(ggZ + o1, C, q, oz);
    if (gU2) {
      s2_store<QM>(gU2 + o2, 2 * C, q, ov);
      s2_store<QM>(gU2 + o2 + C, 2 * C, q, og);
    }
  }
}

struct S2Launch {
  dim3 grid, block;
  size_t lds;
};
S2Launch s2_launch(long E, int q, int C, int ng) {
  const int epb = C >= kS2Threads ? 1 : kS2Threads / C;
  long nb = (E + epb - 1) / epb;
  if (nb > 8192) nb = 8192;
  return {dim3((unsigned)(nb > 0 ? nb : 1)), dim3(kS2Threads), sizeof(float) * 2 * (size_t)ng * q};
}

}  // namespace

#define SO2_S2_DISPATCH(KERNEL, ...)                                                              \
  do {                                                                                            \
    const S2Launch L_ = s2_launch(E, q, C, ng);                                                   \
    if (q <= 8) hipLaunchKernelGGL((KERNEL<8>), L_.grid, L_.block, L_.lds, s, E, q, C, ng, __VA_ARGS__);    \
    else if (q <= 16) hipLaunchKernelGGL((KERNEL<16>), L_.grid, L_.block, L_.lds, s, E, q, C, ng, __VA_ARGS__); \
    else if (q <= 24) hipLaunchKernelGGL((KERNEL<24>), L_.grid, L_.block, L_.lds, s, E, q, C, ng, __VA_ARGS__); \
    else hipLaunchKernelGGL((KERNEL<32>), L_.grid, L_.block, L_.lds, s, E, q, C, ng, __VA_ARGS__);           \
  } while (0)

int launch_s2_fwd(long E, int q, int C, int ng, const float* U, const float* G, const float* P, float* Z,
                  hipStream_t s) {
  if (E == 0) return hipSuccess;
  SO2_S2_DISPATCH(s2_fwd_kernel, U, G, P, Z);
  return hipGetLastError();
}

int launch_s2_bwd(long E, int q, int C, int ng, const float* U, const float* G, const float* P, const float* gZ,
                  float* gU, hipStream_t s) {
  if (E == 0) return hipSuccess;
  SO2_S2_DISPATCH(s2_bwd_kernel, U, G, P, gZ, gU);
  return hipGetLastError();
}

int launch_s2_dbwd(long E, int q, int C, int ng, const float* U, const float* G, const float* P, const float* gZ,
                   const float* pU, float* ggZ, float* gU2, hipStream_t s) {
  if (E == 0) return hipSuccess;
  SO2_S2_DISPATCH(s2_dbwd_kernel, U, G, P, gZ, pU, ggZ, gU2);
  return hipGetLastError();
}

}  // namespace so2
