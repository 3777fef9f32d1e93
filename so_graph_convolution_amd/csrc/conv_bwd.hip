// Backward kernels of the fused SO(2) convolution (TrimSO(2) page, Section
// 3.3 Eq.(4) and Appendix B.1-B.3 derivative formulas).
//
//   edge_bwd  : the transpose of the reduction: tbar_e = R_e gy[dst] (gather from
//               the receiver and rotate, coalesced because edges are grouped
//               by receiver) and the rotation torque of the reduction,
//               tau_k = <V_e, (R_e G_k) gy[dst]>  (Rbar = t gy^T, B.3).
//   gate_bwd  : ubar = sigmoid(gate) zbar, gatebar = sigmoid'(gate) sum_m zbar u (B.2);
//               SiLU' on l = 0.
//   node_bwd  : the transpose of rotation on gather (Eq.(4)): one block per node
//               walks its incoming edges (target half of the message input)
//               and its outgoing edges through the source permutation (source
//               half), accumulating R^T (s * Tbar) in registers; it also writes
//               the radial-scale gradient sbar = sum_m Tbar * (R a) and the
//               rotation torque <s * Tbar, (R G_k) a> (Rbar = xtilde_bar a^T, B.1).
//   pos_grad  : vbar_e = rhat x tau / rho (the frame depends on the edge
//               direction only; the operator is invariant to the frame's roll)
//               and gpos[n] = sum_{src=n} vbar - sum_{dst=n} vbar, per node.
#include "ops.hpp"
#include "dispatch.hpp"
#include "rotation.hpp"

namespace so2 {

int upload_generators_bwd(const float* host) { return upload_generators_here(host); }

namespace {

// edges per LDS tile so that the tile state stays below 48 KB
template <int L, int M, int EXTRA, int BYTES = 48 * 1024>
constexpr int tile_edges() {
  constexpr int per = 9 + k_count(L, M) + 2 * wig_stride_c(L, M) + EXTRA + 16;
  return (32 * per * 4 <= BYTES) ? 32 : (16 * per * 4 <= BYTES) ? 16 : (8 * per * 4 <= BYTES) ? 8 : 4;
}
// LDS budget of an edge kernel's tile. Its blocks hold one tile each, and
// LDS bounds how many run per CU: smaller tiles, more blocks in flight to
// hide the per-edge gathers. Measured on MI355X at lmax 4, C 128 (725k edges):
// edge_bwd 9.6 -> 5.7 ms with 24 KB instead of 48 KB.
constexpr int kEdgeTileBytes = 24 * 1024;

__device__ __forceinline__ float sigm(float v) { return 1.f / (1.f + __expf(-v)); }

// ------------------------------------------------------------------ edge_bwd
// With per-edge message weights (env [E, H]: a cutoff envelope, H = 1, or
// attention weights per head, channel c in head c / (C / H)) the message is
// env_{e,h(c)} V_e[:, c]: tbar and the torque scale per channel, and
// genv_{e,h} = <V_e, R_e gy[dst]> over the channels of head h.
template <int L, int M, typename OT>
__global__ __launch_bounds__(256) void edge_bwd_kernel(Dims d, GraphDev g, const float* __restrict__ pos,
                                                       const float* __restrict__ gy, const float* __restrict__ V,
                                                       const float* __restrict__ env, OT* __restrict__ tbar,
                                                       float* __restrict__ tau, float* __restrict__ genv) {
  constexpr int D = (L + 1) * (L + 1), Q = q_count(L, M), K = k_count(L, M), ST = wig_stride_c(L, M);
  constexpr int TE = tile_edges<L, M, 0, kEdgeTileBytes>();
  __shared__ float sD1[TE * 9];
  __shared__ float sR[TE * K];
  __shared__ float sA[TE * ST], sB[TE * ST];
  __shared__ float sRed[TE * 4 * 4];
  __shared__ float sHead[TE * kMaxHeads];
  __shared__ int sDst[TE];

  const long e0 = g.e0 + (long)blockIdx.x * TE;
  const int ne = (int)min((long)TE, g.e1 - e0);
  for (int t = threadIdx.x; t < ne; t += blockDim.x) {
    const long e = e0 + t;
    const int i = g.dst[e];
    sDst[t] = i;
    edge_geometry(pos, g.shift, g.src[e], i, e, sD1 + 9 * t);
  }
  __syncthreads();
  wigner_rows_block(L, M, ne, sD1, sR, K, sA, sB, ST);
  __syncthreads();
  const int H = d.H, head = c_head(d, threadIdx.x);

  const int C = d.C, wZ = d.wZ();
  const int c = threadIdx.x;
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const bool act = c < C;
  for (int t = 0; t < ne; ++t) {
    const long e = e0 + t - g.e0;   // chunk-relative row
    const float ev = env ? env[(e0 + t) * H + head] : 1.f;
    float tk[4] = {0.f, 0.f, 0.f, 0.f};
    if (act) {
      float gv[D];
      const float* gr = gy + (size_t)sDst[t] * D * C + c;
#pragma unroll
      for (int r = 0; r < D; ++r) gv[r] = gr[(size_t)r * C];
      const float* vr = V + (size_t)e * wZ + c;
      float vv[Q];   // the message row's loads in flight during the rotation
#pragma unroll
      for (int l = 0; l <= L; ++l) {
        const int q = qhalf(l, M);
#pragma unroll
        for (int m = -q; m <= q; ++m) vv[ridx(l, m, M)] = vr[mm_col(l, m, 0, L, C)];
      }
      float o[Q];
      rot_fwd<L, M>(sR + t * K, gv, o);
      OT* tr = tbar + (size_t)e * wZ + c;
#pragma unroll
      for (int l = 0; l <= L; ++l) {
        const int q = qhalf(l, M);
#pragma unroll
        for (int m = -q; m <= q; ++m) st(tr + mm_col(l, m, 0, L, C), ev * o[ridx(l, m, M)]);
      }
      // torque: <v, (R G_k) gy> taken as <G_k^T u, gy> with u = R^T v
      float u[D];
#pragma unroll
      for (int r = 0; r < D; ++r) u[r] = 0.f;
      rot_bwd_acc<L, M>(sR + t * K, vv, u);
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        float s = 0.f;
#pragma unroll
        for (int l = 1; l <= L; ++l) s += gen_form<L>(k, l, u + l * l, gv + l * l);
        tk[k] = ev * s;
      }
#pragma unroll
      for (int j = 0; j < Q; ++j) tk[3] += vv[j] * o[j];
    }
    for (int k = 0; k < 3; ++k) {
      const float s = wave_sum(tk[k]);
      if (lane == 0) sRed[(t * 4 + wave) * 4 + k] = s;
    }
    if (genv) head_partial(tk[3], d, c, t, sRed, 4, 3, sHead);
  }
  __syncthreads();
  const int nw = blockDim.x / 64;
  for (int idx = threadIdx.x; idx < ne * 3; idx += blockDim.x) {
    const int t = idx / 3, k = idx - t * 3;
    float s = 0.f;
    for (int w = 0; w < nw; ++w) s += sRed[(t * 4 + w) * 4 + k];
    tau[(e0 + t - g.e0) * 3 + k] = s;
  }
  if (genv)
    for (int idx = threadIdx.x; idx < ne * H; idx += blockDim.x) {
      const int t = idx / H, h = idx - t * H;
      genv[(e0 + t) * H + h] = head_total(d, t, h, sRed, 4, 3, sHead);
    }
}

template <int L, int M>
struct EdgeBwd {
  static int run(const Dims& d, const GraphDev& g, const float* pos, const float* gy, const float* V,
                 const float* env, void* tbar, float* tau, float* genv, int bf16, hipStream_t s) {
    constexpr int TE = tile_edges<L, M, 0, kEdgeTileBytes>();
    const long nb = (g.e1 - g.e0 + TE - 1) / TE;
    if (nb <= 0) return hipSuccess;
    const int threads = ((d.C + 63) / 64) * 64;
    if (bf16)
      hipLaunchKernelGGL((edge_bwd_kernel<L, M, bf16s>), dim3(nb), dim3(threads), 0, s, d, g, pos, gy, V, env,
                         static_cast<bf16s*>(tbar), tau, genv);
    else
      hipLaunchKernelGGL((edge_bwd_kernel<L, M, float>), dim3(nb), dim3(threads), 0, s, d, g, pos, gy, V, env,
                         static_cast<float*>(tbar), tau, genv);
    return hipGetLastError();
  }
};

// ------------------------------------------------------------------ node_bwd
// The torque terms sum_rows xb <(R G_k)_row, x_n> of a degree are taken as
// <G_k^T y, x_n> with y = R^T xb, the edge's contribution to acc.
template <int L, int M>
__device__ __forceinline__ void node_bwd_edge_half(const Dims& d, RotPtr sRt,
                                                   const float (&xn)[(L + 1) * (L + 1)],
                                                   const float* __restrict__ S, const float* __restrict__ Tbar,
                                                   float* __restrict__ Sbar, long e, int cin,
                                                   float (&acc)[(L + 1) * (L + 1)], float (&tk)[3]) {
  const int Ci = 2 * d.C, wT = d.wT(), wS = (L + 1) * Ci;
  const float* tb = Tbar + (size_t)e * wT + cin;
  const float* sr = S + (size_t)e * wS + cin;
  float* sb = Sbar + (size_t)e * wS + cin;
  // one pass over the rows of R and R G_k: radial cotangent, transposed
  // product into acc and the torque. The global loads of a degree are issued
  // together before its rows (one memory latency per degree, not per row);
  // its radial cotangent store closes it.
#pragma unroll
  for (int l = 0; l <= L; ++l) {
    const int q = qhalf(l, M), n = 2 * l + 1;
    float tv[2 * M + 1];
#pragma unroll
    for (int m = -q; m <= q; ++m) tv[m + q] = tb[mm_col(l, m, 0, L, Ci)];
    const float sc = sr[l * Ci];
    float sacc = 0.f, y[2 * L + 1];
#pragma unroll
    for (int i = 0; i < 2 * L + 1; ++i) y[i] = 0.f;
#pragma unroll
    for (int m = -q; m <= q; ++m) {
      const int off = rot_off(l, M) + (m + q) * n;
      const float v = tv[m + q];
      const float xb = sc * v;
      float r[2 * L + 1];
      load_row<L>(sRt, off, n, r);
      sacc += v * row_dot<L>(r, xn + l * l, n);
      row_axpy<L>(r, xb, y, n);
    }
#pragma unroll
    for (int i = 0; i < 2 * L + 1; ++i)
      if (i < n) acc[l * l + i] += y[i];
    if (l > 0)
#pragma unroll
      for (int k = 0; k < 3; ++k) tk[k] += gen_form<L>(k, l, y, xn + l * l);
    sb[l * Ci] = sacc;
  }
}

template <int L, int M>
__global__ __launch_bounds__(512) void node_bwd_kernel(Dims d, GraphDev g, const float* __restrict__ x,
                                                       const float* __restrict__ pos, const float* __restrict__ S,
                                                       const float* __restrict__ Tbar, float* __restrict__ gx,
                                                       float* __restrict__ Sbar, float* __restrict__ tau_dst,
                                                       float* __restrict__ tau_src, int accumulate) {
  constexpr int D = (L + 1) * (L + 1), K = k_count(L, M), ST = wig_stride_c(L, M);
  constexpr int TE = tile_edges<L, M, 0>();
  __shared__ float sD1[TE * 9];
  __shared__ float sR[TE * K];
  __shared__ float sA[TE * ST], sB[TE * ST];
  __shared__ float sRed[TE * 8 * 3];
  __shared__ int sE[TE];
  __shared__ float sComb[kCombFallback];

  const int node = blockIdx.x;
  const int C = d.C;
  const int CW = blockDim.x / 2;
  const int c = threadIdx.x % CW, grp = threadIdx.x / CW;   // channel, edge parity
  const bool act = c < C;
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64, wpg = CW / 64;
  float xn[D], acc[D];
#pragma unroll
  for (int r = 0; r < D; ++r) {
    xn[r] = act ? x[((size_t)node * D + r) * C + c] : 0.f;
    acc[r] = 0.f;
  }

  for (int pass = 0; pass < 2; ++pass) {
    // pass 0: incoming edges (this node is the receiver, target half of the input)
    // pass 1: outgoing edges via the source permutation (source half)
    int beg, end;
    if (pass == 0) in_range(g, node, &beg, &end);
    else out_range(g, node, &beg, &end);
    float* tau_out = pass == 0 ? tau_dst : tau_src;
    for (int t0 = beg; t0 < end; t0 += TE) {
      const int ne = min(TE, end - t0);
      for (int t = threadIdx.x; t < ne; t += blockDim.x) {
        const long e = pass == 0 ? (long)(t0 + t) : (long)g.src_perm[t0 + t];
        sE[t] = (int)(e - g.e0);   // chunk-relative row
        const int j = pass == 0 ? g.src[e] : node;
        const int i = pass == 0 ? node : g.dst[e];
        edge_geometry(pos, g.shift, j, i, e, sD1 + 9 * t);
      }
      __syncthreads();
      wigner_rows_block(L, M, ne, sD1, sR, K, sA, sB, ST);
      __syncthreads();
      for (int t = grp; t < ne; t += 2) {
        float tk[3] = {0.f, 0.f, 0.f};
        if (act) {
          const int cin = pass == 0 ? C + c : c;
          node_bwd_edge_half<L, M>(d, sR + t * K, xn, S, Tbar, Sbar, sE[t], cin, acc, tk);
        }
#pragma unroll
        for (int k = 0; k < 3; ++k) {
          const float s = wave_sum(tk[k]);
          if (lane == 0) sRed[(t * 8 + wave) * 3 + k] = s;
        }
      }
      __syncthreads();
      for (int idx = threadIdx.x; idx < ne * 3; idx += blockDim.x) {
        const int t = idx / 3, k = idx - t * 3;
        const int w0 = (t % 2) * wpg;   // waves of the group that handled edge t
        float s = 0.f;
        for (int w = w0; w < w0 + wpg; ++w) s += sRed[(t * 8 + w) * 3 + k];
        tau_out[(size_t)sE[t] * 3 + k] = s;
      }
      __syncthreads();
    }
  }
  if (gx) {
    int cap;
    float* cb = comb_buffer(sR, TE * K, sComb, CW, &cap);
    combine_groups<D>(acc, cb, cap, c, grp, CW, act, gx + (size_t)node * D * C, C, accumulate);
  }
}

// ------------------------------------------------------------------ node_bwd, degree split
// At lmax 6 a whole node row and its accumulator per thread hold 222
// registers (two waves per SIMD); there the two thread groups of a node's
// block own degrees [0, LS) and [LS, L] (deg_split, halves within 3% of each
// other at mmax 2) instead of alternate edges. Measured on MI355X at lmax 6
// (1.05M edges): 20.0 -> 17.4 ms per call; at lmax 4, where the halves are
// 70 : 45, the edge-parity kernel above stays faster (7.95 vs 10.0 ms).
// The torque terms sum_rows xb <(R G_k)_row, x_n> of a degree are taken as
// <G_k^T y, x_n> with y = R^T xb, the edge's contribution to acc.
// Degrees [LA, LB) of one edge side; xn and acc hold rows LA^2 .. LB^2 - 1.
// Every load of the edge (T-bar rows, then the radial scales, into `v` of
// capacity VN, the larger group's count) is issued before its first row is
// used and before its radial cotangents are stored: one memory latency per
// edge, not one per degree.
template <int L, int M, int LA, int LB, int VN>
__device__ __forceinline__ void node_bwd_load(const Dims& d, const float* __restrict__ S,
                                              const float* __restrict__ Tbar, long e, int cin, float (&v)[VN]) {
  constexpr int R0 = ridx(LA, -qhalf(LA, M), M), QR = q_range(LA, LB, M);
  const int Ci = 2 * d.C;
  const float* tb = Tbar + (size_t)e * d.wT() + cin;
  const float* sr = S + (size_t)e * ((L + 1) * Ci) + cin;
#pragma unroll
  for (int l = LA; l < LB; ++l) {
    const int q = qhalf(l, M);
#pragma unroll
    for (int m = -q; m <= q; ++m) v[ridx(l, m, M) - R0] = tb[mm_col(l, m, 0, L, Ci)];
    v[QR + l - LA] = sr[l * Ci];
  }
}

template <int L, int M, int LA, int LB, int DH, int VN>
__device__ __forceinline__ void node_bwd_edge_degs(const Dims& d, RotPtr sRt, const float (&xn)[DH],
                                                   const float (&v)[VN], float* __restrict__ Sbar, long e, int cin,
                                                   float (&acc)[DH], float (&tk)[3]) {
  constexpr int B = LA * LA, R0 = ridx(LA, -qhalf(LA, M), M), QR = q_range(LA, LB, M);
  const int Ci = 2 * d.C;
  float* sb = Sbar + (size_t)e * ((L + 1) * Ci) + cin;
  // one pass over the rows of R and R G_k: radial cotangent, transposed
  // product into acc and the torque
#pragma unroll
  for (int l = LA; l < LB; ++l) {
    const int q = qhalf(l, M), n = 2 * l + 1;
    const float scl = v[QR + l - LA];
    float sacc = 0.f, y[2 * L + 1];
#pragma unroll
    for (int i = 0; i < 2 * L + 1; ++i) y[i] = 0.f;
#pragma unroll
    for (int m = -q; m <= q; ++m) {
      const int off = rot_off(l, M) + (m + q) * n;
      const float tv = v[ridx(l, m, M) - R0];
      const float xb = scl * tv;
      float r[2 * L + 1];
      load_row<L>(sRt, off, n, r);
      sacc += tv * row_dot<L>(r, xn + l * l - B, n);
      row_axpy<L>(r, xb, y, n);
    }
#pragma unroll
    for (int i = 0; i < 2 * L + 1; ++i)
      if (i < n) acc[l * l - B + i] += y[i];
    if (l > 0)
#pragma unroll
      for (int k = 0; k < 3; ++k) tk[k] += gen_form<L>(k, l, y, xn + l * l - B);
    sb[l * Ci] = sacc;
  }
}

template <int L, int M>
__global__ __launch_bounds__(512) void node_bwd_split_kernel(Dims d, GraphDev g, const float* __restrict__ x,
                                                       const float* __restrict__ pos, const float* __restrict__ S,
                                                       const float* __restrict__ Tbar, float* __restrict__ gx,
                                                       float* __restrict__ Sbar, float* __restrict__ tau_dst,
                                                       float* __restrict__ tau_src, int accumulate) {
  constexpr int D = (L + 1) * (L + 1), K = k_count(L, M), ST = wig_stride_c(L, M);
  constexpr int LS = deg_split(L, M), DH = half_rows(L, M);
  // values loaded per edge: retained T-bar rows and radial scales of a group's degrees
  constexpr int VN0 = q_range(0, LS, M) + LS, VN1 = q_range(LS, L + 1, M) + L + 1 - LS;
  constexpr int VN = VN0 > VN1 ? VN0 : VN1;
  constexpr int TE = tile_edges<L, M, 0>();
  __shared__ float sD1[TE * 9];
  __shared__ float sR[TE * K];
  __shared__ float sA[TE * ST], sB[TE * ST];
  __shared__ float sRed[TE * 8 * 3];
  __shared__ int sE[TE];

  const int node = blockIdx.x;
  const int C = d.C;
  const int CW = blockDim.x / 2;
  const int c = threadIdx.x % CW, grp = threadIdx.x / CW;   // channel, degree half
  const bool act = c < C;
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64, nw = blockDim.x / 64;
  const int r0 = grp == 0 ? 0 : LS * LS, nr = grp == 0 ? LS * LS : D - LS * LS;
  float xn[DH], acc[DH];
#pragma unroll
  for (int r = 0; r < DH; ++r) {
    xn[r] = (act && r < nr) ? x[((size_t)node * D + r0 + r) * C + c] : 0.f;
    acc[r] = 0.f;
  }

  for (int pass = 0; pass < 2; ++pass) {
    // pass 0: incoming edges (this node is the receiver, target half of the input)
    // pass 1: outgoing edges via the source permutation (source half)
    int beg, end;
    if (pass == 0) in_range(g, node, &beg, &end);
    else out_range(g, node, &beg, &end);
    float* tau_out = pass == 0 ? tau_dst : tau_src;
    for (int t0 = beg; t0 < end; t0 += TE) {
      const int ne = min(TE, end - t0);
      for (int t = threadIdx.x; t < ne; t += blockDim.x) {
        const long e = pass == 0 ? (long)(t0 + t) : (long)g.src_perm[t0 + t];
        sE[t] = (int)(e - g.e0);   // chunk-relative row
        const int j = pass == 0 ? g.src[e] : node;
        const int i = pass == 0 ? node : g.dst[e];
        edge_geometry(pos, g.shift, j, i, e, sD1 + 9 * t);
      }
      __syncthreads();
      wigner_rows_block(L, M, ne, sD1, sR, K, sA, sB, ST);
      __syncthreads();
      const int cin = pass == 0 ? C + c : c;
      for (int t = 0; t < ne; ++t) {
        float tk[3] = {0.f, 0.f, 0.f};
        if (act) {
          float v[VN];
          if (grp == 0) {
            node_bwd_load<L, M, 0, LS, VN>(d, S, Tbar, sE[t], cin, v);
            node_bwd_edge_degs<L, M, 0, LS, DH, VN>(d, sR + t * K, xn, v, Sbar, sE[t], cin, acc, tk);
          } else {
            node_bwd_load<L, M, LS, L + 1, VN>(d, S, Tbar, sE[t], cin, v);
            node_bwd_edge_degs<L, M, LS, L + 1, DH, VN>(d, sR + t * K, xn, v, Sbar, sE[t], cin, acc, tk);
          }
        }
#pragma unroll
        for (int k = 0; k < 3; ++k) {
          const float s = wave_sum(tk[k]);
          if (lane == 0) sRed[(t * 8 + wave) * 3 + k] = s;
        }
      }
      __syncthreads();
      for (int idx = threadIdx.x; idx < ne * 3; idx += blockDim.x) {
        const int t = idx / 3, k = idx - t * 3;
        float s = 0.f;
        for (int w = 0; w < nw; ++w) s += sRed[(t * 8 + w) * 3 + k];
        tau_out[(size_t)sE[t] * 3 + k] = s;
      }
      __syncthreads();
    }
  }
  if (gx && act) {
    float* o = gx + ((size_t)node * D + r0) * C + c;
#pragma unroll
    for (int r = 0; r < DH; ++r)
      if (r < nr) o[(size_t)r * C] = accumulate ? o[(size_t)r * C] + acc[r] : acc[r];
  }
}

template <int L, int M>
struct NodeBwd {
  static int run(const Dims& d, const GraphDev& g, const float* x, const float* pos, const float* S,
                 const float* Tbar, float* gx, float* Sbar, float* tau_dst, float* tau_src, int accumulate,
                 hipStream_t s) {
    if (g.N == 0) return hipSuccess;
    const int threads = 2 * ((d.C + 63) / 64) * 64;
    if constexpr (L >= 6)
      hipLaunchKernelGGL((node_bwd_split_kernel<L, M>), dim3(g.N), dim3(threads), 0, s, d, g, x, pos, S, Tbar, gx,
                         Sbar, tau_dst, tau_src, accumulate);
    else
      hipLaunchKernelGGL((node_bwd_kernel<L, M>), dim3(g.N), dim3(threads), 0, s, d, g, x, pos, S, Tbar, gx, Sbar,
                         tau_dst, tau_src, accumulate);
    return hipGetLastError();
  }
};

// ------------------------------------------------------------------ gate_bwd
// one thread per (edge, l, four channels; launch shape gate_dims)
template <typename OT>
__global__ void gate_bwd_kernel(Dims d, long E, const float* __restrict__ U, const float* __restrict__ Zb,
                                OT* __restrict__ Ub) {
  const int L = d.L, M = d.M, C = d.C;
  const int c = 4 * threadIdx.x, l = threadIdx.y;
  const int wU = d.wU(), wZ = d.wZ();
  for (long e = (long)blockIdx.x * blockDim.z + threadIdx.z; e < E; e += (long)gridDim.x * blockDim.z) {
    const float* ur = U + e * wU;
    const float* zb = Zb + e * wZ;
    OT* ub = Ub + e * wU;
    float u[4], z[4], o[4];
    if (l == 0) {
      ld4(ur + c, u);
      ld4(zb + c, z);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s = sigm(u[i]);
        o[i] = z[i] * s * (1.f + u[i] * (1.f - s));
      }
      st4(ub + c, o);
    } else {
      float s[4], gsum[4] = {0.f, 0.f, 0.f, 0.f};
      ld4(ur + d.gate_col(l, c), s);
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = sigm(s[i]);
      const int q = qhalf(l, M);
      for (int m = -q; m <= q; ++m) {
        ld4(zb + mm_col(l, m, c, L, C), z);
        const int uc = d.u_col(l, m, c);
        ld4(ur + uc, u);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          gsum[i] += z[i] * u[i];
          o[i] = s[i] * z[i];
        }
        st4(ub + uc, o);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = s[i] * (1.f - s[i]) * gsum[i];
      st4(ub + d.gate_col(l, c), o);
    }
  }
}

// ------------------------------------------------------------------ position gradient
// With `roll` the frame's turn about the edge axis counts (a grid activation
// is not invariant to it): the torque's axial part adds
// -(tau . v) s (vy, -vx, 0) / (rho^2 (rho + s vz)), s the sign of vz (the
// branch of edge_frame), from the roll rate -s (vy dvx - vx dvy) / (rho (rho + s vz)).
__global__ void vbar_kernel(GraphDev g, const float* __restrict__ pos, const float* __restrict__ t1,
                            const float* __restrict__ t2, const float* __restrict__ t3, float* __restrict__ vbar,
                            int roll) {
  for (long e = g.e0 + (long)blockIdx.x * blockDim.x + threadIdx.x; e < g.e1; e += (long)gridDim.x * blockDim.x) {
    const long le = e - g.e0;
    const int j = g.src[e], i = g.dst[e];
    float vx = pos[3 * j] - pos[3 * i], vy = pos[3 * j + 1] - pos[3 * i + 1], vz = pos[3 * j + 2] - pos[3 * i + 2];
    if (g.shift) {
      vx += g.shift[3 * e];
      vy += g.shift[3 * e + 1];
      vz += g.shift[3 * e + 2];
    }
    const float rho = sqrtf(vx * vx + vy * vy + vz * vz), inv = 1.f / rho;
    const float rx = vx * inv, ry = vy * inv, rz = vz * inv;
    const float tx = t1[3 * le] + t2[3 * le] + t3[3 * le];
    const float ty = t1[3 * le + 1] + t2[3 * le + 1] + t3[3 * le + 1];
    const float tz = t1[3 * le + 2] + t2[3 * le + 2] + t3[3 * le + 2];
    float o0 = (ry * tz - rz * ty) * inv, o1 = (rz * tx - rx * tz) * inv;
    const float o2 = (rx * ty - ry * tx) * inv;
    if (roll) {
      const float sg = vz >= 0.f ? 1.f : -1.f;
      const float f = -sg * (tx * vx + ty * vy + tz * vz) * inv * inv / (rho + sg * vz);
      o0 += f * vy;
      o1 -= f * vx;
    }
    vbar[3 * e] = o0;
    vbar[3 * e + 1] = o1;
    vbar[3 * e + 2] = o2;
  }
}

__global__ void node_pos_kernel(GraphDev g, const float* __restrict__ vbar, float* __restrict__ gpos) {
  for (long n = (long)blockIdx.x * blockDim.x + threadIdx.x; n < g.N; n += (long)gridDim.x * blockDim.x) {
    float a0 = 0.f, a1 = 0.f, a2 = 0.f;
    for (int k = g.src_ptr[n]; k < g.src_ptr[n + 1]; ++k) {
      const long e = g.src_perm[k];
      a0 += vbar[3 * e];
      a1 += vbar[3 * e + 1];
      a2 += vbar[3 * e + 2];
    }
    for (int e = g.dst_ptr[n]; e < g.dst_ptr[n + 1]; ++e) {
      a0 -= vbar[3 * (long)e];
      a1 -= vbar[3 * (long)e + 1];
      a2 -= vbar[3 * (long)e + 2];
    }
    gpos[3 * n] = a0;
    gpos[3 * n + 1] = a1;
    gpos[3 * n + 2] = a2;
  }
}

inline int grid_for(long n) {
  long b = (n + 255) / 256;
  if (b > 16384) b = 16384;
  if (b < 1) b = 1;
  return (int)b;
}

}  // namespace

int launch_edge_bwd(const Dims& d, const GraphDev& g, const float* pos, const float* gy, const float* V,
                    const float* env, void* tbar, float* tau, float* genv, int bf16, hipStream_t s) {
  return dispatch_lm<EdgeBwd>(d.L, d.M, d, g, pos, gy, V, env, tbar, tau, genv, bf16, s);
}

int launch_gate_bwd(const Dims& d, long E, const float* U, const float* Zbar, void* Ubar, int bf16, hipStream_t s) {
  if (E == 0) return hipSuccess;
  dim3 grid, block;
  gate_dims(d, E, &grid, &block);
  if (bf16)
    hipLaunchKernelGGL(gate_bwd_kernel<bf16s>, grid, block, 0, s, d, E, U, Zbar, static_cast<bf16s*>(Ubar));
  else
    hipLaunchKernelGGL(gate_bwd_kernel<float>, grid, block, 0, s, d, E, U, Zbar, static_cast<float*>(Ubar));
  return hipGetLastError();
}

int launch_node_bwd(const Dims& d, const GraphDev& g, const float* x, const float* pos, const float* S,
                    const float* Tbar, float* gx, float* Sbar, float* tau_dst, float* tau_src, int accumulate,
                    hipStream_t s) {
  return dispatch_lm<NodeBwd>(d.L, d.M, d, g, x, pos, S, Tbar, gx, Sbar, tau_dst, tau_src, accumulate, s);
}

int launch_vbar(const GraphDev& g, const float* pos, const float* tau1, const float* tau2, const float* tau3,
                float* vbar, int roll, hipStream_t s) {
  const long n = g.e1 - g.e0;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(vbar_kernel, dim3(grid_for(n)), dim3(256), 0, s, g, pos, tau1, tau2, tau3, vbar, roll);
  return hipGetLastError();
}

int launch_node_pos(const GraphDev& g, const float* vbar, float* gpos, hipStream_t s) {
  if (g.N == 0) return hipSuccess;
  hipLaunchKernelGGL(node_pos_kernel, dim3(grid_for(g.N)), dim3(256), 0, s, g, vbar, gpos);
  return hipGetLastError();
}

}  // namespace so2
