// Node-to-node spherical projection (TrimSO(2) page, Appendix B.4, spherical
// activations): per node, U = G Y with G the n_g x (L+1)^2 basis-at-grid
// matrix and Y = [X^(l) B_l]_l the node's coefficient rows after the fused
// channel map; and the transposed application Z = G^T Ubar of the backward.
// The back-projection from the grid applies H ((L+1)^2 x n_g) the same way,
// given as the transposed basis (BT: element (g, j) at j * n_g + g).
// Both stream one node array in and one out (HBM-bound); the basis is staged
// in LDS 32 grid rows at a time and read as a broadcast, one thread per
// channel, several nodes per block.
#include "ops.hpp"

namespace so2 {

namespace {

constexpr int kGridRows = 32;

// 32 grid rows of the basis from row g0 (gn rows) into sG [gn][D]
template <int D, bool BT>
__device__ inline void stage_basis(float* sG, const float* __restrict__ G, int ng, int g0, int gn) {
  for (int idx = threadIdx.x; idx < gn * D; idx += blockDim.x)
    sG[idx] = BT ? G[(size_t)(idx % D) * ng + g0 + idx / D] : G[(size_t)g0 * D + idx];
}

template <int D, bool BT>
__global__ __launch_bounds__(1024) void grid_apply_kernel(int N, int ng, int C, const float* __restrict__ G,
                                                          const float* __restrict__ Y, float* __restrict__ U) {
  __shared__ float sG[kGridRows * D];
  const int CP = ((C + 63) / 64) * 64, npb = blockDim.x / CP;
  const int lnode = threadIdx.x / CP, c = threadIdx.x - lnode * CP;
  const long node = (long)blockIdx.x * npb + lnode;
  const bool act = c < C && node < N;
  float y[D];
#pragma unroll
  for (int j = 0; j < D; ++j) y[j] = act ? Y[((size_t)node * D + j) * C + c] : 0.f;
  for (int g0 = 0; g0 < ng; g0 += kGridRows) {
    const int gn = min(kGridRows, ng - g0);
    __syncthreads();
    stage_basis<D, BT>(sG, G, ng, g0, gn);
    __syncthreads();
    if (act) {
      float* u = U + ((size_t)node * ng + g0) * C + c;
      for (int g = 0; g < gn; ++g) {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < D; ++j) s += sG[g * D + j] * y[j];
        u[(size_t)g * C] = s;
      }
    }
  }
}

template <int D, bool BT>
__global__ __launch_bounds__(1024) void grid_apply_t_kernel(int N, int ng, int C, const float* __restrict__ G,
                                                            const float* __restrict__ U, float* __restrict__ Z) {
  __shared__ float sG[kGridRows * D];
  const int CP = ((C + 63) / 64) * 64, npb = blockDim.x / CP;
  const int lnode = threadIdx.x / CP, c = threadIdx.x - lnode * CP;
  const long node = (long)blockIdx.x * npb + lnode;
  const bool act = c < C && node < N;
  float z[D];
#pragma unroll
  for (int j = 0; j < D; ++j) z[j] = 0.f;
  for (int g0 = 0; g0 < ng; g0 += kGridRows) {
    const int gn = min(kGridRows, ng - g0);
    __syncthreads();
    stage_basis<D, BT>(sG, G, ng, g0, gn);
    __syncthreads();
    if (act) {
      const float* u = U + ((size_t)node * ng + g0) * C + c;
      for (int g = 0; g < gn; ++g) {
        const float v = u[(size_t)g * C];
#pragma unroll
        for (int j = 0; j < D; ++j) z[j] += sG[g * D + j] * v;
      }
    }
  }
  if (act) {
#pragma unroll
    for (int j = 0; j < D; ++j) Z[((size_t)node * D + j) * C + c] = z[j];
  }
}

template <int D, bool T, bool BT>
int grid_launch_d(int N, int ng, int C, const float* G, const float* in, float* out, hipStream_t s) {
  if (N == 0) return hipSuccess;
  const int CP = ((C + 63) / 64) * 64, npb = CP >= 256 ? 1 : 256 / CP;
  const long blocks = ((long)N + npb - 1) / npb;
  if (T)
    hipLaunchKernelGGL((grid_apply_t_kernel<D, BT>), dim3((unsigned)blocks), dim3(CP * npb), 0, s, N, ng, C, G, in,
                       out);
  else
    hipLaunchKernelGGL((grid_apply_kernel<D, BT>), dim3((unsigned)blocks), dim3(CP * npb), 0, s, N, ng, C, G, in, out);
  return hipGetLastError();
}

template <bool T, bool BT>
int grid_launch(int L, int N, int ng, int C, const float* G, const float* in, float* out, hipStream_t s) {
  switch (L) {
    case 0: return grid_launch_d<1, T, BT>(N, ng, C, G, in, out, s);
    case 1: return grid_launch_d<4, T, BT>(N, ng, C, G, in, out, s);
    case 2: return grid_launch_d<9, T, BT>(N, ng, C, G, in, out, s);
    case 3: return grid_launch_d<16, T, BT>(N, ng, C, G, in, out, s);
    case 4: return grid_launch_d<25, T, BT>(N, ng, C, G, in, out, s);
    case 5: return grid_launch_d<36, T, BT>(N, ng, C, G, in, out, s);
    case 6: return grid_launch_d<49, T, BT>(N, ng, C, G, in, out, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int launch_grid_apply(int L, int N, int ng, int C, const float* G, const float* Y, float* U, hipStream_t s,
                      int basis_t) {
  return basis_t ? grid_launch<false, true>(L, N, ng, C, G, Y, U, s) : grid_launch<false, false>(L, N, ng, C, G, Y, U, s);
}

int launch_grid_apply_t(int L, int N, int ng, int C, const float* G, const float* U, float* Z, hipStream_t s,
                        int basis_t) {
  return basis_t ? grid_launch<true, true>(L, N, ng, C, G, U, Z, s) : grid_launch<true, false>(L, N, ng, C, G, U, Z, s);
}

}  // namespace so2
