// Forward kernels of the fused SO(2) convolution.
//
//   edge_fwd  : rotation on gather (TrimSO(2) page, Section 3.2 and Appendix
//               B.1): per edge tile, build the frame and compact Wigner rows in
//               LDS, gather [x_src | x_dst] rows (coalesced over channels),
//               rotate, apply the radial scale and write the m-major input of
//               the first SO(2) linear.
//   gate_fwd  : gated activation on the first linear's output (Appendix B.2):
//               SiLU on l = 0, sigmoid(gate_l) on every retained order of l >= 1.
//   node_fwd  : inverse rotation on reduction (Appendix B.3): one block per
//               target node walks its incoming-edge range (edges sorted by
//               target), regenerates each edge's rotation rows, accumulates
//               R^T t in registers and writes the node row once. No atomics.
#include "ops.hpp"
#include "dispatch.hpp"
#include "rotation.hpp"

namespace so2 {

int upload_generators_fwd(const float* host) { return upload_generators_here(host); }

namespace {

constexpr int kTileE = 32;   // edges per LDS tile

// ------------------------------------------------------------------ edge_fwd
template <int L, int M, typename OT>
__global__ __launch_bounds__(256) void edge_fwd_kernel(Dims d, GraphDev g, const float* __restrict__ x,
                                                       const float* __restrict__ pos, const float* __restrict__ S,
                                                       OT* __restrict__ T) {
  constexpr int D = (L + 1) * (L + 1), Q = q_count(L, M), K = k_count(L, M), ST = wig_stride_c(L, M);
  __shared__ float sD1[kTileE * 9];
  __shared__ float sR[kTileE * K];
  __shared__ float sA[kTileE * ST], sB[kTileE * ST];
  __shared__ int sNode[2][kTileE];

  const long e0 = g.e0 + (long)blockIdx.x * kTileE;
  const int ne = (int)min((long)kTileE, g.e1 - e0);
  for (int t = threadIdx.x; t < ne; t += blockDim.x) {
    const long e = e0 + t;
    const int j = g.src[e], i = g.dst[e];
    sNode[0][t] = j;
    sNode[1][t] = i;
    edge_geometry(pos, g.shift, j, i, e, sD1 + 9 * t);
  }
  __syncthreads();
  wigner_rows_block(L, M, ne, sD1, sR, K, sA, sB, ST);

  const int C = d.C, Ci = 2 * C, wT = d.wT();
  const int ldS = (L + 1) * Ci;
  for (int c = threadIdx.x; c < Ci; c += blockDim.x) {
    const int half = c >= C, cc = c - half * C;
    for (int t = 0; t < ne; ++t) {
      const long e = e0 + t - g.e0;   // chunk-relative row
      const float* xr = x + (size_t)sNode[half][t] * D * C + cc;
      float a[D];
#pragma unroll
      for (int r = 0; r < D; ++r) a[r] = xr[(size_t)r * C];
      const float* sr = S + (size_t)e * ldS + c;
      float scv[L + 1];   // every load of the edge before the rotation and its stores
#pragma unroll
      for (int l = 0; l <= L; ++l) scv[l] = sr[l * Ci];
      float o[Q];
      rot_fwd<L, M>(sR + t * K, a, o);
      OT* tr = T + (size_t)e * wT;
#pragma unroll
      for (int l = 0; l <= L; ++l) {
        const float sc = scv[l];
        const int q = qhalf(l, M);
#pragma unroll
        for (int m = -q; m <= q; ++m) st(tr + mm_col(l, m, c, L, Ci), sc * o[ridx(l, m, M)]);
      }
    }
  }
}

template <int L, int M>
struct EdgeFwd {
  static int run(const Dims& d, const GraphDev& g, const float* x, const float* pos, const float* S, void* T,
                 int bf16, hipStream_t s) {
    const long nb = (g.e1 - g.e0 + kTileE - 1) / kTileE;
    if (nb <= 0) return hipSuccess;
    const int threads = min(256, ((2 * d.C + 63) / 64) * 64);
    if (bf16)
      hipLaunchKernelGGL((edge_fwd_kernel<L, M, bf16s>), dim3(nb), dim3(threads), 0, s, d, g, x, pos, S,
                         static_cast<bf16s*>(T));
    else
      hipLaunchKernelGGL((edge_fwd_kernel<L, M, float>), dim3(nb), dim3(threads), 0, s, d, g, x, pos, S,
                         static_cast<float*>(T));
    return hipGetLastError();
  }
};

// ------------------------------------------------------------------ node_fwd
template <int L, int M>
__global__ __launch_bounds__(512) void node_fwd_kernel(Dims d, GraphDev g, const float* __restrict__ pos,
                                                       const float* __restrict__ V, const float* __restrict__ env,
                                                       float* __restrict__ y, int accumulate) {
  constexpr int D = (L + 1) * (L + 1), Q = q_count(L, M), K = k_count(L, M), ST = wig_stride_c(L, M);
  __shared__ float sD1[kTileE * 9];
  __shared__ float sR[kTileE * K];
  __shared__ float sA[kTileE * ST], sB[kTileE * ST];
  __shared__ float sComb[kCombFallback];

  const int node = blockIdx.x;
  int beg, end;
  in_range(g, node, &beg, &end);
  if (accumulate && beg == end) return;
  const int C = d.C, wZ = d.wZ();
  const int CW = blockDim.x / 2;
  const int c = threadIdx.x % CW, grp = threadIdx.x / CW;   // channel, edge parity
  const bool act = c < C;
  float acc[D];
#pragma unroll
  for (int r = 0; r < D; ++r) acc[r] = 0.f;

  for (int t0 = beg; t0 < end; t0 += kTileE) {
    const int ne = min(kTileE, end - t0);
    for (int t = threadIdx.x; t < ne; t += blockDim.x) {
      const long e = t0 + t;
      edge_geometry(pos, g.shift, g.src[e], node, e, sD1 + 9 * t);
    }
    __syncthreads();
    wigner_rows_block(L, M, ne, sD1, sR, K, sA, sB, ST);
    if (act) {
      for (int t = grp; t < ne; t += 2) {
        const float* vr = V + (size_t)(t0 + t - g.e0) * wZ + c;
        const float ev = env ? env[(size_t)(t0 + t) * d.H + c / d.hs()] : 1.f;   // message weight of c's head
        float tv[Q];
#pragma unroll
        for (int l = 0; l <= L; ++l) {
          const int q = qhalf(l, M);
#pragma unroll
          for (int m = -q; m <= q; ++m) tv[ridx(l, m, M)] = ev * vr[mm_col(l, m, 0, L, C)];
        }
        rot_bwd_acc<L, M>(sR + t * K, tv, acc);
      }
    }
    __syncthreads();
  }
  int cap;
  float* cb = comb_buffer(sR, kTileE * K, sComb, CW, &cap);
  combine_groups<D>(acc, cb, cap, c, grp, CW, act, y + (size_t)node * D * C, C, accumulate);
}

template <int L, int M>
struct NodeFwd {
  static int run(const Dims& d, const GraphDev& g, const float* pos, const float* V, const float* env, float* y,
                 int accumulate, hipStream_t s) {
    if (g.N == 0) return hipSuccess;
    const int threads = 2 * ((d.C + 63) / 64) * 64;
    hipLaunchKernelGGL((node_fwd_kernel<L, M>), dim3(g.N), dim3(threads), 0, s, d, g, pos, V, env, y, accumulate);
    return hipGetLastError();
  }
};

// ------------------------------------------------------------------ gate_fwd
__device__ __forceinline__ float sigm(float v) { return 1.f / (1.f + __expf(-v)); }

// one thread per (edge, l, four channels; launch shape gate_dims): reads the
// gate once, scales every retained order of l
template <typename OT>
__global__ void gate_fwd_kernel(Dims d, long E, const float* __restrict__ U, OT* __restrict__ Z) {
  const int L = d.L, M = d.M, C = d.C;
  const int c = 4 * threadIdx.x, l = threadIdx.y;
  const int wU = d.wU(), wZ = d.wZ();
  for (long e = (long)blockIdx.x * blockDim.z + threadIdx.z; e < E; e += (long)gridDim.x * blockDim.z) {
    const float* ur = U + e * wU;
    OT* zr = Z + e * wZ;
    float u[4], z[4];
    if (l == 0) {
      ld4(ur + c, u);
#pragma unroll
      for (int i = 0; i < 4; ++i) z[i] = u[i] * sigm(u[i]);
      st4(zr + c, z);
    } else {
      float gs[4];
      ld4(ur + d.gate_col(l, c), gs);
#pragma unroll
      for (int i = 0; i < 4; ++i) gs[i] = sigm(gs[i]);
      const int q = qhalf(l, M);
      for (int m = -q; m <= q; ++m) {
        ld4(ur + d.u_col(l, m, c), u);
#pragma unroll
        for (int i = 0; i < 4; ++i) z[i] = gs[i] * u[i];
        st4(zr + mm_col(l, m, c, L, C), z);
      }
    }
  }
}

// ------------------------------------------------------------------ weights
// block of w: [k][2h] = [W0 | W1] (plain: [k][h2] copied as is);
// realified: [2k][2h] = [[W0, W1], [-W1, W0]]; transposed output: [2h][2k]
template <typename IT, typename OT, bool TRANS>
__global__ void realify_kernel(const IT* __restrict__ w, int k, int h, int plain, OT* __restrict__ wr) {
  const int rows = plain ? k : 2 * k, cols = plain ? h : 2 * h;
  const long n = (long)rows * cols;
  for (long idx = (long)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (long)gridDim.x * blockDim.x) {
    int r, col;
    if (TRANS) {
      col = (int)(idx / rows);
      r = (int)(idx - (long)col * rows);
    } else {
      r = (int)(idx / cols);
      col = (int)(idx - (long)r * cols);
    }
    float v;
    if (plain) {
      v = ld(w + (long)r * cols + col);
    } else {
      const int rr = r % k, lower = r >= k, right = col >= h, cc = col % h;
      if (!lower) v = ld(w + (long)rr * 2 * h + col);
      else v = right ? ld(w + (long)rr * 2 * h + cc) : -ld(w + (long)rr * 2 * h + h + cc);
    }
    st(wr + idx, v);
  }
}

template <typename OT>
__global__ void fold_kernel(const float* __restrict__ gr, int k, int h, OT* __restrict__ gw) {
  // gw[k][2h]: [G00 + G11 | G01 - G10]
  const long n = (long)k * 2 * h;
  for (long idx = (long)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (long)gridDim.x * blockDim.x) {
    const int r = (int)(idx / (2 * h)), col = (int)(idx - (long)r * 2 * h);
    const int cc = col % h;
    const long top = (long)r * 2 * h, bot = (long)(r + k) * 2 * h;
    st(gw + idx, col < h ? gr[top + cc] + gr[bot + h + cc] : gr[top + h + cc] - gr[bot + cc]);
  }
}

template <typename IT, typename OT>
__global__ void convert_kernel(const IT* __restrict__ in, OT* __restrict__ out, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    st(out + i, ld(in + i));
}

inline int grid_for(long n) {
  long b = (n + 255) / 256;
  if (b > 16384) b = 16384;
  if (b < 1) b = 1;
  return (int)b;
}

}  // namespace

int launch_edge_fwd(const Dims& d, const GraphDev& g, const float* x, const float* pos, const float* S, void* T,
                    int bf16, hipStream_t s) {
  return dispatch_lm<EdgeFwd>(d.L, d.M, d, g, x, pos, S, T, bf16, s);
}

int launch_node_fwd(const Dims& d, const GraphDev& g, const float* pos, const float* V, const float* env, float* y,
                    int accumulate, hipStream_t s) {
  return dispatch_lm<NodeFwd>(d.L, d.M, d, g, pos, V, env, y, accumulate, s);
}

int launch_gate_fwd(const Dims& d, long E, const float* U, void* Z, int bf16, hipStream_t s) {
  if (E == 0) return hipSuccess;
  dim3 grid, block;
  gate_dims(d, E, &grid, &block);
  if (bf16)
    hipLaunchKernelGGL(gate_fwd_kernel<bf16s>, grid, block, 0, s, d, E, U, static_cast<bf16s*>(Z));
  else
    hipLaunchKernelGGL(gate_fwd_kernel<float>, grid, block, 0, s, d, E, U, static_cast<float*>(Z));
  return hipGetLastError();
}

void realified_shape(const Dims& d, int second, int a, int* rows, int* cols, long* off) {
  const int win = second ? d.C : 2 * d.C;
  long o = 0;
  for (int b = 0; b <= d.M; ++b) {
    int r, c;
    const int hout = second ? d.C : d.hw();
    if (b == 0) {
      r = (d.L + 1) * win;
      c = second || d.s2 ? (d.L + 1) * hout : (2 * d.L + 1) * d.C;
    } else {
      r = 2 * (d.L - b + 1) * win;
      c = 2 * (d.L - b + 1) * hout;
    }
    if (b == a) {
      *rows = r;
      *cols = c;
      *off = o;
      return;
    }
    o += (long)r * c;
  }
}

long realified_size(const Dims& d, int second) {
  int r, c;
  long off;
  realified_shape(d, second, d.M, &r, &c, &off);
  return off + (long)r * c;
}

template <typename IT, typename OT, bool TRANS>
int realify_block(const void* w, int k, int h, int plain, void* out, hipStream_t s) {
  const long n = (long)(plain ? k : 2 * k) * (plain ? h : 2 * h);
  hipLaunchKernelGGL((realify_kernel<IT, OT, TRANS>), dim3(grid_for(n)), dim3(256), 0, s, static_cast<const IT*>(w), k,
                     h, plain, static_cast<OT*>(out));
  return hipGetLastError();
}

int launch_realify(const Dims& d, int second, const void* const* w, void* wr, void* wrt, int bf16, hipStream_t s,
                   int in_f32) {
  for (int a = 0; a <= d.M; ++a) {
    int r, c;
    long off;
    realified_shape(d, second, a, &r, &c, &off);
    const int plain = a == 0;
    const int k = plain ? r : r / 2, h = plain ? c : c / 2;
    int e;
    if (bf16 && in_f32) {
      e = realify_block<float, bf16s, false>(w[a], k, h, plain, static_cast<bf16s*>(wr) + off, s);
      if (e == hipSuccess && wrt)
        e = realify_block<float, bf16s, true>(w[a], k, h, plain, static_cast<bf16s*>(wrt) + off, s);
    } else if (!bf16) {
      if (plain) {
        e = hipMemcpyAsync(static_cast<float*>(wr) + off, w[0], sizeof(float) * (size_t)r * c,
                           hipMemcpyDeviceToDevice, s);
        if (e == hipSuccess && wrt)
          e = realify_block<float, float, true>(w[0], k, h, 1, static_cast<float*>(wrt) + off, s);
      } else {
        e = realify_block<float, float, false>(w[a], k, h, 0, static_cast<float*>(wr) + off, s);
      }
    } else {
      e = realify_block<bf16s, bf16s, false>(w[a], k, h, plain, static_cast<bf16s*>(wr) + off, s);
      if (e == hipSuccess && wrt)
        e = realify_block<bf16s, bf16s, true>(w[a], k, h, plain, static_cast<bf16s*>(wrt) + off, s);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

int launch_fold_grad(const Dims& d, int second, const float* gr, void* const* gw, int bf16, hipStream_t s,
                     int user_layout) {
  for (int a = 0; a <= d.M; ++a) {
    if (!gw[a]) continue;
    int r, c;
    long off;
    realified_shape(d, second, a, &r, &c, &off);
    hipError_t e;
    if (a > 0 && user_layout && !bf16) {   // already [k][2h] at the block's offset
      e = hipMemcpyAsync(gw[a], gr + off, sizeof(float) * (size_t)(r / 2) * c, hipMemcpyDeviceToDevice, s);
    } else if (a == 0) {
      if (bf16) e = (hipError_t)launch_to_bf16(gr + off, static_cast<bf16s*>(gw[0]), (size_t)r * c, s);
      else e = hipMemcpyAsync(gw[0], gr + off, sizeof(float) * (size_t)r * c, hipMemcpyDeviceToDevice, s);
    } else {
      const int k = r / 2, h = c / 2;
      if (bf16)
        hipLaunchKernelGGL(fold_kernel<bf16s>, dim3(grid_for((long)k * c)), dim3(256), 0, s, gr + off, k, h,
                           static_cast<bf16s*>(gw[a]));
      else
        hipLaunchKernelGGL(fold_kernel<float>, dim3(grid_for((long)k * c)), dim3(256), 0, s, gr + off, k, h,
                           static_cast<float*>(gw[a]));
      e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

int launch_to_f32(const bf16s* in, float* out, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL((convert_kernel<bf16s, float>), dim3(grid_for((long)n)), dim3(256), 0, s, in, out, n);
  return hipGetLastError();
}

int launch_to_bf16(const float* in, bf16s* out, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL((convert_kernel<float, bf16s>), dim3(grid_for((long)n)), dim3(256), 0, s, in, out, n);
  return hipGetLastError();
}

bool lm_supported(int L, int M) { return lm_pair_compiled(L, M); }

}  // namespace so2
