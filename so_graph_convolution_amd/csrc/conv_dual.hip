// Double-backward kernels of the fused SO(2) convolution.
//
// The double backward differentiates L = <p, backward(gy)> (TrimSO(2) page,
// Appendix A.3 Eq.(3): the force term of the training loss) with respect to
// the inputs and gy. Since the backward is linear in gy, dL/dgy is the
// forward's directional derivative along p (Eq.(5)), and the remaining
// derivatives are the reverse of that directional derivative with cotangent
// gy. Both run here as forward-over-reverse: a tangent ("dual") forward,
// then its reverse. A position direction moves each edge direction and so
// rotates its frame: Rdot_e = R_e Omega_e, Omega_e = sum_k w_k G_k with
// w = drhat x rhat, drhat = (I - rhat rhat^T) dv / rho.
//
//   edge_dual     : Tdot = sdot * (R a) + s * (Rdot a + R adot)
//   gate_dual     : zdot = sigmoid(g) udot + sigmoid'(g) gdot u  (SiLU'(u) udot on l = 0)
//   node_dual     : ydot_i = sum_e Rdot^T V + R^T Vdot          (= dL/dgy)
//   edge_bwd_dual : [R gy[dst]; Rdot gy[dst]]   (cotangents of Vdot and V)
//   gate_dbwd     : cotangents of (udot, u) from those of (zdot, z)
//   node_bwd_dual : dL/dx = R^T (s Tbar + sdot Tdotbar) + Rdot^T (s Tdotbar) on both
//                   halves, and the radial-scale cotangents sbar, sdotbar.
#include "ops.hpp"
#include "dispatch.hpp"
#include "rotation.hpp"

namespace so2 {

int upload_generators_dual(const float* host) { return upload_generators_here(host); }

namespace {

template <int L, int M, int EXTRA, int BYTES = 48 * 1024>
constexpr int tile_edges() {
  constexpr int per = 9 + k_count(L, M) + 2 * wig_stride_c(L, M) + EXTRA + 8;
  return (32 * per * 4 <= BYTES) ? 32 : (16 * per * 4 <= BYTES) ? 16 : (8 * per * 4 <= BYTES) ? 8 : 4;
}
// LDS budget of an edge kernel's tile. Its blocks hold one tile each, and
// LDS bounds how many run per CU: smaller tiles, more blocks in flight to
// hide the per-edge gathers. Measured on MI355X at lmax 4, C 128 (725k edges):
// edge_dual and edge_bwd_dual 8.1 -> 7.7 and 6.8 -> 3.3 ms with 16 KB instead of 48 KB.
constexpr int kEdgeTileBytes = 16 * 1024;

__device__ __forceinline__ float sigm(float v) { return 1.f / (1.f + __expf(-v)); }

// direction of the edge frame's rotation for an edge-vector direction dv.
// With `roll` it includes the frame's turn about the edge axis: the frame of
// edge_frame rolls at rate beta = -s (ry dx - rx dy) / (rho (1 + s rz)),
// s = sign of rz (the branch the frame takes), which the gated operator
// does not see (it is invariant to the roll) but a grid activation does.
__device__ inline void frame_rate(const EdgeGeo& gg, float dx, float dy, float dz, float* w, bool roll) {
  const float inv = 1.f / gg.rho;
  const float pr = gg.rx * dx + gg.ry * dy + gg.rz * dz;
  const float ax = (dx - gg.rx * pr) * inv, ay = (dy - gg.ry * pr) * inv, az = (dz - gg.rz * pr) * inv;
  // w = drhat x rhat
  w[0] = ay * gg.rz - az * gg.ry;
  w[1] = az * gg.rx - ax * gg.rz;
  w[2] = ax * gg.ry - ay * gg.rx;
  if (roll) {
    const float sg = gg.rz >= 0.f ? 1.f : -1.f;
    const float beta = -sg * (gg.ry * dx - gg.rx * dy) * inv / (1.f + sg * gg.rz);
    w[0] += beta * gg.rx;
    w[1] += beta * gg.ry;
    w[2] += beta * gg.rz;
  }
}

// ------------------------------------------------------------------ edge_dual
template <int L, int M, typename OT>
__global__ __launch_bounds__(256) void edge_dual_kernel(Dims d, GraphDev g, const float* __restrict__ x,
                                                        const float* __restrict__ px, const float* __restrict__ pos,
                                                        const float* __restrict__ ppos,
                                                        const float* __restrict__ pedge, const float* __restrict__ S,
                                                        const float* __restrict__ Sdot, OT* __restrict__ Tdot,
                                                        float* __restrict__ omega) {
  constexpr int D = (L + 1) * (L + 1), Q = q_count(L, M), K = k_count(L, M), ST = wig_stride_c(L, M);
  constexpr int TE = tile_edges<L, M, 3, kEdgeTileBytes>();
  __shared__ float sD1[TE * 9];
  __shared__ float sR[TE * K];
  __shared__ float sA[TE * ST], sB[TE * ST];
  __shared__ float sW[TE * 3];
  __shared__ int sNode[2][TE];

  const long e0 = g.e0 + (long)blockIdx.x * TE;
  const int ne = (int)min((long)TE, g.e1 - e0);
  for (int t = threadIdx.x; t < ne; t += blockDim.x) {
    const long e = e0 + t;
    const int j = g.src[e], i = g.dst[e];
    sNode[0][t] = j;
    sNode[1][t] = i;
    const EdgeGeo gg = edge_geometry(pos, g.shift, j, i, e, sD1 + 9 * t);
    float dx = 0.f, dy = 0.f, dz = 0.f;
    if (ppos) {
      dx = ppos[3 * j] - ppos[3 * i];
      dy = ppos[3 * j + 1] - ppos[3 * i + 1];
      dz = ppos[3 * j + 2] - ppos[3 * i + 2];
    }
    if (pedge) {
      dx += pedge[3 * e];
      dy += pedge[3 * e + 1];
      dz += pedge[3 * e + 2];
    }
    float w[3];
    frame_rate(gg, dx, dy, dz, w, d.s2 != 0);
    for (int k = 0; k < 3; ++k) {
      sW[t * 3 + k] = w[k];
      omega[(e - g.e0) * 3 + k] = w[k];
    }
  }
  __syncthreads();
  wigner_rows_block(L, M, ne, sD1, sR, K, sA, sB, ST);
  __syncthreads();

  const int C = d.C, Ci = 2 * C, wT = d.wT(), wS = (L + 1) * Ci;
  for (int c = threadIdx.x; c < Ci; c += blockDim.x) {
    const int half = c >= C, cc = c - half * C;
    for (int t = 0; t < ne; ++t) {
      const long e = e0 + t - g.e0;   // chunk-relative row
      const size_t nb = (size_t)sNode[half][t] * D * C + cc;
      float a[D], ad[D];
#pragma unroll
      for (int r = 0; r < D; ++r) {
        a[r] = x[nb + (size_t)r * C];
        ad[r] = px ? px[nb + (size_t)r * C] : 0.f;
      }
      const float* sr = S + (size_t)e * wS + c;
      const float* sd = Sdot + (size_t)e * wS + c;
      OT* tr = Tdot + (size_t)e * wT;
      float svv[L + 1], sdvv[L + 1];   // every load of the edge before its stores
#pragma unroll
      for (int l = 0; l <= L; ++l) {
        svv[l] = sr[l * Ci];
        sdvv[l] = sd[l * Ci];
      }
      const float w[3] = {sW[t * 3], sW[t * 3 + 1], sW[t * 3 + 2]};
#pragma unroll
      for (int l = 0; l <= L; ++l) {
        const float sv = svv[l], sdv = sdvv[l];
        const int q = qhalf(l, M), n = 2 * l + 1;
        float ga[2 * L + 1];   // G_w a: the rows of Rdot = R G_w applied as R (G_w a)
        gw_apply<L, false>(w, l, a + l * l, ga);
#pragma unroll
        for (int m = -q; m <= q; ++m) {
          const int off = rot_off(l, M) + (m + q) * n;
          float r[2 * L + 1];
          load_row<L>(sR + t * K, off, n, r);
          const float xt = row_dot<L>(r, a + l * l, n), y2 = row_dot<L>(r, ad + l * l, n);
          const float y1 = row_dot<L>(r, ga, n);
          st(tr + mm_col(l, m, c, L, Ci), sdv * xt + sv * (y1 + y2));
        }
      }
    }
  }
}

template <int L, int M>
struct EdgeDual {
  static int run(const Dims& d, const GraphDev& g, const float* x, const float* px, const float* pos,
                 const float* ppos, const float* pedge, const float* S, const float* Sdot, void* Tdot, float* omega,
                 int bf16, hipStream_t s) {
    constexpr int TE = tile_edges<L, M, 3, kEdgeTileBytes>();
    const long nb = (g.e1 - g.e0 + TE - 1) / TE;
    if (nb <= 0) return hipSuccess;
    const int threads = min(256, ((2 * d.C + 63) / 64) * 64);
    if (bf16)
      hipLaunchKernelGGL((edge_dual_kernel<L, M, bf16s>), dim3(nb), dim3(threads), 0, s, d, g, x, px, pos, ppos,
                         pedge, S, Sdot, static_cast<bf16s*>(Tdot), omega);
    else
      hipLaunchKernelGGL((edge_dual_kernel<L, M, float>), dim3(nb), dim3(threads), 0, s, d, g, x, px, pos, ppos,
                         pedge, S, Sdot, static_cast<float*>(Tdot), omega);
    return hipGetLastError();
  }
};

// ------------------------------------------------------------------ node_dual
template <int L, int M>
__global__ __launch_bounds__(512) void node_dual_kernel(Dims d, GraphDev g, const float* __restrict__ pos,
                                                        const float* __restrict__ omega, const float* __restrict__ V,
                                                        const float* __restrict__ Vdot, const float* __restrict__ env,
                                                        const float* __restrict__ penv, float* __restrict__ ydot,
                                                        int accumulate) {
  constexpr int D = (L + 1) * (L + 1), Q = q_count(L, M), K = k_count(L, M), ST = wig_stride_c(L, M);
  constexpr int TE = tile_edges<L, M, 3>();
  __shared__ float sD1[TE * 9];
  __shared__ float sR[TE * K];
  __shared__ float sA[TE * ST], sB[TE * ST];
  __shared__ float sW[TE * 3];
  __shared__ float sComb[kCombFallback];

  const int node = blockIdx.x;
  int beg, end;
  in_range(g, node, &beg, &end);
  if (accumulate && beg == end) return;
  const int C = d.C, wZ = d.wZ();
  const int CW = blockDim.x / 2;
  const int c = threadIdx.x % CW, grp = threadIdx.x / CW;   // channel, edge parity
  float acc[D];
#pragma unroll
  for (int r = 0; r < D; ++r) acc[r] = 0.f;
  for (int t0 = beg; t0 < end; t0 += TE) {
    const int ne = min(TE, end - t0);
    for (int t = threadIdx.x; t < ne; t += blockDim.x) {
      const long e = t0 + t;
      edge_geometry(pos, g.shift, g.src[e], node, e, sD1 + 9 * t);
      for (int k = 0; k < 3; ++k) sW[t * 3 + k] = omega[(e - g.e0) * 3 + k];
    }
    __syncthreads();
    wigner_rows_block(L, M, ne, sD1, sR, K, sA, sB, ST);
    __syncthreads();
    if (c < C) {
      for (int t = grp; t < ne; t += 2) {
        const float* vr = V + (size_t)(t0 + t - g.e0) * wZ + c;
        const float* vd = Vdot + (size_t)(t0 + t - g.e0) * wZ + c;
        // message env V (weights of c's head): tangent env (Rdot^T V + R^T Vdot) + penv R^T V
        const size_t wi = (size_t)(t0 + t) * d.H + c / d.hs();
        const float ev = env ? env[wi] : 1.f, pv = penv ? penv[wi] : 0.f;
        const float w[3] = {sW[t * 3], sW[t * 3 + 1], sW[t * 3 + 2]};
#pragma unroll
        for (int l = 0; l <= L; ++l) {
          const int q = qhalf(l, M), n = 2 * l + 1;
          float vv[2 * M + 1], vvd[2 * M + 1];   // the degree's loads together: one latency per degree
#pragma unroll
          for (int m = -q; m <= q; ++m) {
            vv[m + q] = vr[mm_col(l, m, 0, L, C)];
            vvd[m + q] = vd[mm_col(l, m, 0, L, C)];
          }
          // Rdot^T (ev v) = G_w^T (R^T ev v): z gathers R^T ev v over the rows
          float z[2 * L + 1], zw[2 * L + 1];
#pragma unroll
          for (int i = 0; i < 2 * L + 1; ++i) z[i] = 0.f;
#pragma unroll
          for (int m = -q; m <= q; ++m) {
            const int off = rot_off(l, M) + (m + q) * n;
            const float v = vv[m + q], vdv = vvd[m + q];
            float r[2 * L + 1];
            load_row<L>(sR + t * K, off, n, r);
            row_axpy<L>(r, ev * v, z, n);
            row_axpy<L>(r, ev * vdv + pv * v, acc + l * l, n);
          }
          gw_apply<L, true>(w, l, z, zw);
#pragma unroll
          for (int i = 0; i < 2 * L + 1; ++i)
            if (i < n) acc[l * l + i] += zw[i];
        }
      }
    }
    __syncthreads();
  }
  int cap;
  float* cb = comb_buffer(sR, TE * K, sComb, CW, &cap);
  combine_groups<D>(acc, cb, cap, c, grp, CW, c < C, ydot + (size_t)node * D * C, C, accumulate);
}

template <int L, int M>
struct NodeDual {
  static int run(const Dims& d, const GraphDev& g, const float* pos, const float* omega, const float* V,
                 const float* Vdot, const float* env, const float* penv, float* ydot, int accumulate, hipStream_t s) {
    if (g.N == 0) return hipSuccess;
    const int threads = 2 * ((d.C + 63) / 64) * 64;
    hipLaunchKernelGGL((node_dual_kernel<L, M>), dim3(g.N), dim3(threads), 0, s, d, g, pos, omega, V, Vdot, env,
                       penv, ydot, accumulate);
    return hipGetLastError();
  }
};

// ------------------------------------------------------------------ edge_bwd_dual
// G2 = [R gy; Rdot gy] per edge. With P2 (position derivatives of the double
// backward) it also writes, per edge, the rotation torque and rotation-rate
// cotangent of ydot = sum_e (Rdot^T V + R^T Vdot):
//   p2[e][k]     = Vdot^T (R G_k) gy + V^T (Rdot G_k) gy   (<Rbar, R G_k> + <Rdotbar, Rdot G_k>)
//   p2[e][3 + k] = V^T (R G_k) gy                           (<Rdotbar, R G_k>)
// With an envelope the tangent message is env (Rdot^T V + R^T Vdot) + penv R^T V:
// G2 = [env R gy; env Rdot gy + penv R gy], the torque terms scale alike, and
// genv2_e = <Rdot gy, V> + <R gy, Vdot> (per head of channels with weights [E, H]).
template <int L, int M, typename OT, bool P2>
__global__ __launch_bounds__(256) void edge_bwd_dual_kernel(Dims d, GraphDev g, const float* __restrict__ pos,
                                                            const float* __restrict__ omega,
                                                            const float* __restrict__ gy, OT* __restrict__ G2,
                                                            const float* __restrict__ V,
                                                            const float* __restrict__ Vdot,
                                                            const float* __restrict__ env,
                                                            const float* __restrict__ penv, float* __restrict__ p2,
                                                            float* __restrict__ genv2) {
  constexpr int D = (L + 1) * (L + 1), K = k_count(L, M), ST = wig_stride_c(L, M);
  constexpr int TE = tile_edges<L, M, 3 + 28, kEdgeTileBytes>();
  __shared__ float sD1[TE * 9];
  __shared__ float sR[TE * K];
  __shared__ float sA[TE * ST], sB[TE * ST];
  __shared__ float sW[TE * 3];
  __shared__ float sRed[TE * 4 * 7];
  __shared__ float sHead[TE * kMaxHeads];
  __shared__ int sDst[TE];

  const long e0 = g.e0 + (long)blockIdx.x * TE;
  const int ne = (int)min((long)TE, g.e1 - e0);
  for (int t = threadIdx.x; t < ne; t += blockDim.x) {
    const long e = e0 + t;
    const int i = g.dst[e];
    sDst[t] = i;
    edge_geometry(pos, g.shift, g.src[e], i, e, sD1 + 9 * t);
    for (int k = 0; k < 3; ++k) sW[t * 3 + k] = omega[(e - g.e0) * 3 + k];
  }
  __syncthreads();
  wigner_rows_block(L, M, ne, sD1, sR, K, sA, sB, ST);
  __syncthreads();
  const int C = d.C, wZ = d.wZ();
  const int c = threadIdx.x, lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const bool act = c < C;
  const int H = d.H, head = c_head(d, c);
  for (int t = 0; t < ne; ++t) {
    const long e = e0 + t - g.e0;   // chunk-relative row
    const float ev = env ? env[(e0 + t) * H + head] : 1.f, pv = penv ? penv[(e0 + t) * H + head] : 0.f;
    float tk[7] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (act) {
      float gv[D];
      const float* gr = gy + (size_t)sDst[t] * D * C + c;
#pragma unroll
      for (int r = 0; r < D; ++r) gv[r] = gr[(size_t)r * C];
      OT* r1 = G2 + (size_t)e * wZ + c;
      OT* r2 = G2 + ((size_t)(g.e1 - g.e0) + e) * wZ + c;
      const float* vr0 = V + (size_t)e * wZ + c;
      const float* vdr0 = Vdot + (size_t)e * wZ + c;
      const float w[3] = {sW[t * 3], sW[t * 3 + 1], sW[t * 3 + 2]};
#pragma unroll
      for (int l = 0; l <= L; ++l) {
        const int q = qhalf(l, M), n = 2 * l + 1;
        float gw[2 * L + 1];   // G_w gy: the rows of Rdot = R G_w applied as R (G_w gy)
        gw_apply<L, false>(w, l, gv + l * l, gw);
#pragma unroll
        for (int m = -q; m <= q; ++m) {
          const int off = rot_off(l, M) + (m + q) * n;
          float r[2 * L + 1];
          load_row<L>(sR + t * K, off, n, r);
          const float s1 = row_dot<L>(r, gv + l * l, n), s2 = row_dot<L>(r, gw, n);
          st(r1 + mm_col(l, m, 0, L, C), ev * s1);
          st(r2 + mm_col(l, m, 0, L, C), __builtin_fmaf(ev, s2, pv * s1));   // fused alike in every instantiation
          if (genv2) tk[6] += vr0[mm_col(l, m, 0, L, C)] * s2 + vdr0[mm_col(l, m, 0, L, C)] * s1;
        }
      }
      if (P2) {
        // sum over rows of vd (R G_k gy) and v (Rdot G_k gy) = v (R G_w G_k gy):
        // <G_k^T u1, gy> and <G_k^T G_w^T u0, gy> with u0 = R^T v, u1 = R^T vd
        const float* vr = V + (size_t)e * wZ + c;
        const float* vdr = Vdot + (size_t)e * wZ + c;
#pragma unroll
        for (int l = 1; l <= L; ++l) {
          const int q = qhalf(l, M), n = 2 * l + 1;
          float u0[2 * L + 1], u1[2 * L + 1], u0w[2 * L + 1];
#pragma unroll
          for (int i = 0; i < 2 * L + 1; ++i) u0[i] = u1[i] = 0.f;
#pragma unroll
          for (int m = -q; m <= q; ++m) {
            const int off = rot_off(l, M) + (m + q) * n;
            const float v = vr[mm_col(l, m, 0, L, C)], vd = vdr[mm_col(l, m, 0, L, C)];
            float r[2 * L + 1];
            load_row<L>(sR + t * K, off, n, r);
            row_axpy<L>(r, v, u0, n);
            row_axpy<L>(r, vd, u1, n);
          }
          gw_apply<L, true>(w, l, u0, u0w);
#pragma unroll
          for (int k = 0; k < 3; ++k) {
            const float a0 = gen_form<L>(k, l, u0, gv + l * l);
            const float a1 = gen_form<L>(k, l, u1, gv + l * l) + gen_form<L>(k, l, u0w, gv + l * l);
            tk[k] += ev * a1 + pv * a0;
            tk[3 + k] += ev * a0;
          }
        }
      }
    }
    if (P2) {
#pragma unroll
      for (int k = 0; k < 6; ++k) {
        const float sum = wave_sum(tk[k]);
        if (lane == 0) sRed[(t * 4 + wave) * 7 + k] = sum;
      }
    }
    if (genv2) head_partial(tk[6], d, c, t, sRed, 7, 6, sHead);
  }
  if (P2 || genv2) {
    __syncthreads();
    const int nw = blockDim.x / 64;
    if (P2)
      for (int idx = threadIdx.x; idx < ne * 6; idx += blockDim.x) {
        const int t = idx / 6, k = idx - t * 6;
        float sum = 0.f;
        for (int w = 0; w < nw; ++w) sum += sRed[(t * 4 + w) * 7 + k];
        p2[(e0 + t - g.e0) * 6 + k] = sum;
      }
    if (genv2)
      for (int idx = threadIdx.x; idx < ne * H; idx += blockDim.x) {
        const int t = idx / H, h = idx - t * H;
        genv2[(e0 + t) * H + h] = head_total(d, t, h, sRed, 7, 6, sHead);
      }
  }
}

template <int L, int M>
struct EdgeBwdDual {
  template <typename OT, bool P2>
  static void go(const Dims& d, const GraphDev& g, const float* pos, const float* omega, const float* gy, void* G2,
                 const float* V, const float* Vdot, const float* env, const float* penv, float* p2, float* genv2,
                 hipStream_t s) {
    constexpr int TE = tile_edges<L, M, 3 + 28, kEdgeTileBytes>();
    const long nb = (g.e1 - g.e0 + TE - 1) / TE;
    const int threads = ((d.C + 63) / 64) * 64;
    hipLaunchKernelGGL((edge_bwd_dual_kernel<L, M, OT, P2>), dim3(nb), dim3(threads), 0, s, d, g, pos, omega, gy,
                       static_cast<OT*>(G2), V, Vdot, env, penv, p2, genv2);
  }
  static int run(const Dims& d, const GraphDev& g, const float* pos, const float* omega, const float* gy, void* G2,
                 int bf16, const float* V, const float* Vdot, const float* env, const float* penv, float* p2,
                 float* genv2, hipStream_t s) {
    if (g.e1 <= g.e0) return hipSuccess;
    if (bf16) {
      if (p2) go<bf16s, true>(d, g, pos, omega, gy, G2, V, Vdot, env, penv, p2, genv2, s);
      else go<bf16s, false>(d, g, pos, omega, gy, G2, V, Vdot, env, penv, p2, genv2, s);
    } else {
      if (p2) go<float, true>(d, g, pos, omega, gy, G2, V, Vdot, env, penv, p2, genv2, s);
      else go<float, false>(d, g, pos, omega, gy, G2, V, Vdot, env, penv, p2, genv2, s);
    }
    return hipGetLastError();
  }
};

// ------------------------------------------------------------------ node_bwd_dual
// With P2 it also writes, per edge of each half, the torque and rotation-rate
// cotangent of the rotation on gather in the tangent forward (T = S (R a),
// Tdot = Sdot (R a) + S (Rdot a + R adot)), with Tbar, Tdotbar their cotangents:
//   p2[e][k]     = (S Tbar + Sdot Tdotbar)^T (R G_k) a + (S Tdotbar)^T ((R G_k) adot + (Rdot G_k) a)
//   p2[e][3 + k] = (S Tdotbar)^T (R G_k) a
template <int L, int M, bool P2>
__global__ __launch_bounds__(512) void node_bwd_dual_kernel(Dims d, GraphDev g, const float* __restrict__ x,
                                                            const float* __restrict__ px,
                                                            const float* __restrict__ pos,
                                                            const float* __restrict__ omega,
                                                            const float* __restrict__ S,
                                                            const float* __restrict__ Sdot,
                                                            const float* __restrict__ Tdb,
                                                            const float* __restrict__ Tb, float* __restrict__ gx2,
                                                            float* __restrict__ Sbar, float* __restrict__ Sdb,
                                                            float* __restrict__ p2_dst, float* __restrict__ p2_src,
                                                            int accumulate) {
  constexpr int D = (L + 1) * (L + 1), Q = q_count(L, M), K = k_count(L, M), ST = wig_stride_c(L, M);
  constexpr int TE = tile_edges<L, M, k_count(L, M) + 3 + (P2 ? 48 : 0)>();
  __shared__ float sD1[TE * 9];
  __shared__ float sR[TE * K];
  __shared__ float sA[TE * ST], sB[TE * ST];
  __shared__ float sRd[TE * K];
  __shared__ float sW[TE * 3];
  __shared__ float sRed[P2 ? TE * 8 * 6 : 1];
  __shared__ int sE[TE];
  __shared__ float sComb[kCombFallback];

  const int node = blockIdx.x;
  const int C = d.C, Ci = 2 * C, wT = d.wT(), wS = (L + 1) * Ci;
  const int CW = blockDim.x / 2;
  const int c = threadIdx.x % CW, grp = threadIdx.x / CW;   // channel, edge parity
  const bool act = c < C;
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64, wpg = CW / 64;
  float xn[D], xdn[D], acc[D];
#pragma unroll
  for (int r = 0; r < D; ++r) {
    const size_t o = ((size_t)node * D + r) * C + c;
    xn[r] = act ? x[o] : 0.f;
    xdn[r] = (act && px) ? px[o] : 0.f;
    acc[r] = 0.f;
  }
  for (int pass = 0; pass < 2; ++pass) {
    int beg, end;
    if (pass == 0) in_range(g, node, &beg, &end);
    else out_range(g, node, &beg, &end);
    float* p2_out = pass == 0 ? p2_dst : p2_src;
    for (int t0 = beg; t0 < end; t0 += TE) {
      const int ne = min(TE, end - t0);
      for (int t = threadIdx.x; t < ne; t += blockDim.x) {
        const long e = pass == 0 ? (long)(t0 + t) : (long)g.src_perm[t0 + t];
        sE[t] = (int)(e - g.e0);   // chunk-relative row
        const int j = pass == 0 ? g.src[e] : node;
        const int i = pass == 0 ? node : g.dst[e];
        edge_geometry(pos, g.shift, j, i, e, sD1 + 9 * t);
        for (int k = 0; k < 3; ++k) sW[t * 3 + k] = omega[(e - g.e0) * 3 + k];
      }
      __syncthreads();
      wigner_rows_block(L, M, ne, sD1, sR, K, sA, sB, ST);
      rot_directional(L, M, ne, sR, K, sW, 3, sRd, K);
      __syncthreads();
      const int cin = pass == 0 ? C + c : c;
      for (int t = grp; t < ne; t += 2) {
        float tk[6] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (act) {
          const long e = sE[t];
          const float* tdb = Tdb + (size_t)e * wT + cin;
          const float* tb = Tb + (size_t)e * wT + cin;
          const float* sr = S + (size_t)e * wS + cin;
          const float* sd = Sdot + (size_t)e * wS + cin;
          // one pass over the rows of R and Rdot: forward products for the
          // radial cotangents and the transposed products into acc. A
          // degree's global loads are issued together before its rows (one
          // memory latency per degree); its radial cotangent stores close it.
#pragma unroll
          for (int l = 0; l <= L; ++l) {
            const int q = qhalf(l, M), n = 2 * l + 1;
            float v1[2 * M + 1], v0[2 * M + 1];
#pragma unroll
            for (int m = -q; m <= q; ++m) {
              v1[m + q] = tdb[mm_col(l, m, 0, L, Ci)];
              v0[m + q] = tb[mm_col(l, m, 0, L, Ci)];
            }
            const float sv = sr[l * Ci], sdv = sd[l * Ci];
            float sb = 0.f, sdb = 0.f;
            // position terms: the row sums y = R^T u1, z = R^T u2, zw = Rdot^T u2
            float y[P2 ? 2 * L + 1 : 1], z[P2 ? 2 * L + 1 : 1], zw[P2 ? 2 * L + 1 : 1];
            if (P2)
#pragma unroll
              for (int i = 0; i < (P2 ? 2 * L + 1 : 1); ++i) y[i] = z[i] = zw[i] = 0.f;
#pragma unroll
            for (int m = -q; m <= q; ++m) {
              const int off = rot_off(l, M) + (m + q) * n;
              const float a1 = v1[m + q];
              const float a0 = v0[m + q];
              float r[2 * L + 1], rd[2 * L + 1];
              load_row<L>(sR + t * K, off, n, r);
              load_row<L>(sRd + t * K, off, n, rd);
              const float xt = row_dot<L>(r, xn + l * l, n), y2 = row_dot<L>(r, xdn + l * l, n);
              const float y1 = row_dot<L>(rd, xn + l * l, n);
              // explicit fused forms: every instantiation (with or without the
              // position derivatives) rounds alike
              sb = __builtin_fmaf(a0, xt, __builtin_fmaf(a1, y1 + y2, sb));
              sdb = __builtin_fmaf(a1, xt, sdb);
              const float u1 = __builtin_fmaf(sv, a0, sdv * a1), u2 = sv * a1;
              row_axpy<L>(r, u1, acc + l * l, n);
              row_axpy<L>(rd, u2, acc + l * l, n);
              if (P2)
#pragma unroll
                for (int i = 0; i < (P2 ? 2 * L + 1 : 1); ++i)
                  if (i < n) {
                    y[i] = __builtin_fmaf(r[i], u1, y[i]);
                    z[i] = __builtin_fmaf(r[i], u2, z[i]);
                    zw[i] = __builtin_fmaf(rd[i], u2, zw[i]);
                  }
            }
            if (P2 && l > 0) {
              // sum over rows of u1 (R G_k x) + u2 ((R G_k) xd + (Rdot G_k) x), u2 (R G_k x)
#pragma unroll
              for (int k = 0; k < 3; ++k) {
                const float ga = gen_form<L>(k, l, z, xn + l * l);
                tk[k] += gen_form<L>(k, l, y, xn + l * l) + gen_form<L>(k, l, z, xdn + l * l) +
                         gen_form<L>(k, l, zw, xn + l * l);
                tk[3 + k] += ga;
              }
            }
            Sbar[(size_t)e * wS + l * Ci + cin] = sb;
            Sdb[(size_t)e * wS + l * Ci + cin] = sdb;
          }
        }
        if (P2) {
#pragma unroll
          for (int k = 0; k < 6; ++k) {
            const float sum = wave_sum(tk[k]);
            if (lane == 0) sRed[(t * 8 + wave) * 6 + k] = sum;
          }
        }
      }
      if (P2) {
        __syncthreads();
        for (int idx = threadIdx.x; idx < ne * 6; idx += blockDim.x) {
          const int t = idx / 6, k = idx - t * 6;
          const int w0 = (t % 2) * wpg;   // waves of the group that handled edge t
          float sum = 0.f;
          for (int w = w0; w < w0 + wpg; ++w) sum += sRed[(t * 8 + w) * 6 + k];
          p2_out[(size_t)sE[t] * 6 + k] = sum;
        }
      }
      __syncthreads();
    }
  }
  if (gx2) {
    int cap;
    float* cb = comb_buffer(sRd, TE * K, sComb, CW, &cap);
    combine_groups<D>(acc, cb, cap, c, grp, CW, act, gx2 + (size_t)node * D * C, C, accumulate);
  }
}

// ------------------------------------------------------------------ node_bwd_dual, degree split
// The same outputs as node_bwd_dual_kernel, for lmax 6 (see
// node_bwd_split_kernel): 12.0 -> 10.6 ms per call at lmax 6, mmax 2 on
// MI355X without the position terms.
// The two thread groups of a node's block own degrees [0, LS) and [LS, L]
// (deg_split); each thread keeps x, xdot and the accumulator of its degrees.
//
// Every load of an edge's degrees (Tdotbar and Tbar rows, then S and Sdot)
// is issued before its first rotation row is used and before its radial
// cotangents are stored: one memory latency per edge, not one per degree.
template <int L, int M, int LA, int LB, int VN>
__device__ __forceinline__ void node_bwd_dual_load(const Dims& d, const float* __restrict__ S,
                                                   const float* __restrict__ Sdot, const float* __restrict__ Tdb,
                                                   const float* __restrict__ Tb, long e, int cin, float (&v)[VN]) {
  constexpr int R0 = ridx(LA, -qhalf(LA, M), M), QR = q_range(LA, LB, M), NL = LB - LA;
  const int Ci = 2 * d.C, wT = d.wT(), wS = (L + 1) * Ci;
  const float* tdb = Tdb + (size_t)e * wT + cin;
  const float* tb = Tb + (size_t)e * wT + cin;
  const float* sr = S + (size_t)e * wS + cin;
  const float* sd = Sdot + (size_t)e * wS + cin;
#pragma unroll
  for (int l = LA; l < LB; ++l) {
    const int q = qhalf(l, M);
#pragma unroll
    for (int m = -q; m <= q; ++m) {
      v[ridx(l, m, M) - R0] = tdb[mm_col(l, m, 0, L, Ci)];
      v[QR + ridx(l, m, M) - R0] = tb[mm_col(l, m, 0, L, Ci)];
    }
    v[2 * QR + l - LA] = sr[l * Ci];
    v[2 * QR + NL + l - LA] = sd[l * Ci];
  }
}

template <int L, int M, bool P2, int LA, int LB, int DH, int VN>
__device__ __forceinline__ void node_bwd_dual_degs(const Dims& d, RotPtr sRt, RotPtr sRdt,
                                                   const float (&xn)[DH], const float (&xdn)[DH],
                                                   const float (&v)[VN], float* __restrict__ Sbar,
                                                   float* __restrict__ Sdb, long e, int cin, float (&acc)[DH],
                                                   float (&tk)[6]) {
  constexpr int B = LA * LA, R0 = ridx(LA, -qhalf(LA, M), M), QR = q_range(LA, LB, M), NL = LB - LA;
  const int Ci = 2 * d.C, wS = (L + 1) * Ci;
  float* sbo = Sbar + (size_t)e * wS + cin;
  float* sdo = Sdb + (size_t)e * wS + cin;
  // one pass over the rows of R and Rdot: forward products for the radial
  // cotangents and the transposed products into acc
#pragma unroll
  for (int l = LA; l < LB; ++l) {
    const int q = qhalf(l, M), n = 2 * l + 1;
    const float sv = v[2 * QR + l - LA], sdv = v[2 * QR + NL + l - LA];
    float sb = 0.f, sdb = 0.f;
    // position terms: the row sums y = R^T u1, z = R^T u2, zw = Rdot^T u2
    float y[P2 ? 2 * L + 1 : 1], z[P2 ? 2 * L + 1 : 1], zw[P2 ? 2 * L + 1 : 1];
    if (P2)
#pragma unroll
      for (int i = 0; i < (P2 ? 2 * L + 1 : 1); ++i) y[i] = z[i] = zw[i] = 0.f;
#pragma unroll
    for (int m = -q; m <= q; ++m) {
      const int off = rot_off(l, M) + (m + q) * n;
      const float a1 = v[ridx(l, m, M) - R0];
      const float a0 = v[QR + ridx(l, m, M) - R0];
      float r[2 * L + 1], rd[2 * L + 1];
      load_row<L>(sRt, off, n, r);
      load_row<L>(sRdt, off, n, rd);
      const float xt = row_dot<L>(r, xn + l * l - B, n), y2 = row_dot<L>(r, xdn + l * l - B, n);
      const float y1 = row_dot<L>(rd, xn + l * l - B, n);
      // explicit fused forms: every instantiation (with or without the
      // position derivatives) rounds alike
      sb = __builtin_fmaf(a0, xt, __builtin_fmaf(a1, y1 + y2, sb));
      sdb = __builtin_fmaf(a1, xt, sdb);
      const float u1 = __builtin_fmaf(sv, a0, sdv * a1), u2 = sv * a1;
      row_axpy<L>(r, u1, acc + l * l - B, n);
      row_axpy<L>(rd, u2, acc + l * l - B, n);
      if (P2)
#pragma unroll
        for (int i = 0; i < (P2 ? 2 * L + 1 : 1); ++i)
          if (i < n) {
            y[i] = __builtin_fmaf(r[i], u1, y[i]);
            z[i] = __builtin_fmaf(r[i], u2, z[i]);
            zw[i] = __builtin_fmaf(rd[i], u2, zw[i]);
          }
    }
    if (P2 && l > 0) {
      // sum over rows of u1 (R G_k x) + u2 ((R G_k) xd + (Rdot G_k) x), u2 (R G_k x)
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const float ga = gen_form<L>(k, l, z, xn + l * l - B);
        tk[k] += gen_form<L>(k, l, y, xn + l * l - B) + gen_form<L>(k, l, z, xdn + l * l - B) +
                 gen_form<L>(k, l, zw, xn + l * l - B);
        tk[3 + k] += ga;
      }
    }
    sbo[l * Ci] = sb;
    sdo[l * Ci] = sdb;
  }
}

template <int L, int M, bool P2>
__global__ __launch_bounds__(512) void node_bwd_dual_split_kernel(
    Dims d, GraphDev g, const float* __restrict__ x, const float* __restrict__ px, const float* __restrict__ pos,
    const float* __restrict__ omega, const float* __restrict__ S, const float* __restrict__ Sdot,
    const float* __restrict__ Tdb, const float* __restrict__ Tb, float* __restrict__ gx2, float* __restrict__ Sbar,
    float* __restrict__ Sdb, float* __restrict__ p2_dst, float* __restrict__ p2_src, int accumulate) {
  constexpr int D = (L + 1) * (L + 1), K = k_count(L, M), ST = wig_stride_c(L, M);
  constexpr int LS = deg_split(L, M), DH = half_rows(L, M);
  // values loaded per edge: two rows per retained row, two scales per degree
  constexpr int VN0 = 2 * (q_range(0, LS, M) + LS), VN1 = 2 * (q_range(LS, L + 1, M) + L + 1 - LS);
  constexpr int VN = VN0 > VN1 ? VN0 : VN1;
  constexpr int TE = tile_edges<L, M, k_count(L, M) + 3 + (P2 ? 48 : 0)>();
  __shared__ float sD1[TE * 9];
  __shared__ float sR[TE * K];
  __shared__ float sA[TE * ST], sB[TE * ST];
  __shared__ float sRd[TE * K];
  __shared__ float sW[TE * 3];
  __shared__ float sRed[P2 ? TE * 8 * 6 : 1];
  __shared__ int sE[TE];

  const int node = blockIdx.x;
  const int C = d.C;
  const int CW = blockDim.x / 2;
  const int c = threadIdx.x % CW, grp = threadIdx.x / CW;   // channel, degree half
  const bool act = c < C;
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64, nw = blockDim.x / 64;
  const int r0 = grp == 0 ? 0 : LS * LS, nr = grp == 0 ? LS * LS : D - LS * LS;
  float xn[DH], xdn[DH], acc[DH];
#pragma unroll
  for (int r = 0; r < DH; ++r) {
    const size_t o = ((size_t)node * D + r0 + r) * C + c;
    xn[r] = (act && r < nr) ? x[o] : 0.f;
    xdn[r] = (act && r < nr && px) ? px[o] : 0.f;
    acc[r] = 0.f;
  }
  for (int pass = 0; pass < 2; ++pass) {
    int beg, end;
    if (pass == 0) in_range(g, node, &beg, &end);
    else out_range(g, node, &beg, &end);
    float* p2_out = pass == 0 ? p2_dst : p2_src;
    for (int t0 = beg; t0 < end; t0 += TE) {
      const int ne = min(TE, end - t0);
      for (int t = threadIdx.x; t < ne; t += blockDim.x) {
        const long e = pass == 0 ? (long)(t0 + t) : (long)g.src_perm[t0 + t];
        sE[t] = (int)(e - g.e0);   // chunk-relative row
        const int j = pass == 0 ? g.src[e] : node;
        const int i = pass == 0 ? node : g.dst[e];
        edge_geometry(pos, g.shift, j, i, e, sD1 + 9 * t);
        for (int k = 0; k < 3; ++k) sW[t * 3 + k] = omega[(e - g.e0) * 3 + k];
      }
      __syncthreads();
      wigner_rows_block(L, M, ne, sD1, sR, K, sA, sB, ST);
      rot_directional(L, M, ne, sR, K, sW, 3, sRd, K);
      __syncthreads();
      const int cin = pass == 0 ? C + c : c;
      for (int t = 0; t < ne; ++t) {
        float tk[6] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (act) {
          const long e = sE[t];
          float v[VN];
          if (grp == 0) {
            node_bwd_dual_load<L, M, 0, LS, VN>(d, S, Sdot, Tdb, Tb, e, cin, v);
            node_bwd_dual_degs<L, M, P2, 0, LS, DH, VN>(d, sR + t * K, sRd + t * K, xn, xdn, v, Sbar, Sdb, e,
                                                        cin, acc, tk);
          } else {
            node_bwd_dual_load<L, M, LS, L + 1, VN>(d, S, Sdot, Tdb, Tb, e, cin, v);
            node_bwd_dual_degs<L, M, P2, LS, L + 1, DH, VN>(d, sR + t * K, sRd + t * K, xn, xdn, v, Sbar, Sdb,
                                                            e, cin, acc, tk);
          }
        }
        if (P2) {
#pragma unroll
          for (int k = 0; k < 6; ++k) {
            const float sum = wave_sum(tk[k]);
            if (lane == 0) sRed[(t * 8 + wave) * 6 + k] = sum;
          }
        }
      }
      if (P2) {
        __syncthreads();
        for (int idx = threadIdx.x; idx < ne * 6; idx += blockDim.x) {
          const int t = idx / 6, k = idx - t * 6;
          float sum = 0.f;
          for (int w = 0; w < nw; ++w) sum += sRed[(t * 8 + w) * 6 + k];
          p2_out[(size_t)sE[t] * 6 + k] = sum;
        }
      }
      __syncthreads();
    }
  }
  if (gx2 && act) {
    float* o = gx2 + ((size_t)node * D + r0) * C + c;
#pragma unroll
    for (int r = 0; r < DH; ++r)
      if (r < nr) o[(size_t)r * C] = accumulate ? o[(size_t)r * C] + acc[r] : acc[r];
  }
}

template <int L, int M>
struct NodeBwdDual {
  static int run(const Dims& d, const GraphDev& g, const float* x, const float* px, const float* pos,
                 const float* omega, const float* S, const float* Sdot, const float* Tdb, const float* Tb,
                 float* gx2, float* Sbar,
                 float* Sdb, float* p2_dst, float* p2_src, int accumulate, hipStream_t s) {
    if (g.N == 0) return hipSuccess;
    const int threads = 2 * ((d.C + 63) / 64) * 64;
    // both variants on one schedule, so that asking for the position terms
    // leaves gx2, Sbar and Sdb bitwise unchanged (the position-term variant
    // of the split kernel spills 400 bytes per lane at lmax 6)
    if constexpr (L >= 6) {
      if (p2_dst)
        hipLaunchKernelGGL((node_bwd_dual_split_kernel<L, M, true>), dim3(g.N), dim3(threads), 0, s, d, g, x, px,
                           pos, omega, S, Sdot, Tdb, Tb, gx2, Sbar, Sdb, p2_dst, p2_src, accumulate);
      else
        hipLaunchKernelGGL((node_bwd_dual_split_kernel<L, M, false>), dim3(g.N), dim3(threads), 0, s, d, g, x, px,
                           pos, omega, S, Sdot, Tdb, Tb, gx2, Sbar, Sdb, p2_dst, p2_src, accumulate);
    } else if (p2_dst) {
      hipLaunchKernelGGL((node_bwd_dual_kernel<L, M, true>), dim3(g.N), dim3(threads), 0, s, d, g, x, px, pos, omega,
                         S, Sdot, Tdb, Tb, gx2, Sbar, Sdb, p2_dst, p2_src, accumulate);
    } else {
      hipLaunchKernelGGL((node_bwd_dual_kernel<L, M, false>), dim3(g.N), dim3(threads), 0, s, d, g, x, px, pos, omega,
                         S, Sdot, Tdb, Tb, gx2, Sbar, Sdb, p2_dst, p2_src, accumulate);
    }
    return hipGetLastError();
  }
};

// ------------------------------------------------------------------ position derivatives (double backward)
// Per edge: the frame depends on r = v/|v| (v = pos[src] - pos[dst] + shift)
// and the tangent rotation rate is w = (dv x v)/|v|^2 (dv = ppos[src] -
// ppos[dst] + pedge). With the torque tau of R (including Rdot = R W, whose
// R-dependence adds <Rdotbar, Rdot G_k> + (w x wbar)_k through the so(3)
// commutators) and the rate cotangent wbar:
//   vbar2 = r x tau / |v| + (wbar x dv)/|v|^2 - 2 (wbar . w) v/|v|^2
// With `roll` (the frame's turn about the edge axis counts, see frame_rate)
// the rate is w + beta r with beta = -s N / (|v| D), N = vy dvx - vx dvy,
// D = |v| + s vz, and two terms join: the torque's axial part through the
// roll, -(tau . r) s (vy, -vx, 0) / (|v| D), and the gradient of
// (wbar . r) beta, -s / (|v|^2 D) [(wbar . v)(-dvy, dvx, 0) + N wbar
// - N (wbar . v)(2 v / |v|^2 + (v / |v| + s z) / D)].
__global__ void pos2_kernel(GraphDev g, const float* __restrict__ pos, const float* __restrict__ ppos,
                            const float* __restrict__ pedge, const float* __restrict__ omega,
                            const float* __restrict__ pe, const float* __restrict__ pd, const float* __restrict__ ps,
                            float* __restrict__ vbar2, int roll) {
  for (long e = g.e0 + (long)blockIdx.x * blockDim.x + threadIdx.x; e < g.e1; e += (long)gridDim.x * blockDim.x) {
    const long le = e - g.e0;
    const int j = g.src[e], i = g.dst[e];
    float v[3], dv[3] = {0.f, 0.f, 0.f}, w[3], tau[3], wb[3];
    for (int k = 0; k < 3; ++k) {
      v[k] = pos[3 * j + k] - pos[3 * i + k] + (g.shift ? g.shift[3 * e + k] : 0.f);
      if (ppos) dv[k] = ppos[3 * j + k] - ppos[3 * i + k];
      if (pedge) dv[k] += pedge[3 * e + k];
      w[k] = omega[3 * le + k];
      tau[k] = pe[6 * le + k] + pd[6 * le + k] + ps[6 * le + k];
      wb[k] = pe[6 * le + 3 + k] + pd[6 * le + 3 + k] + ps[6 * le + 3 + k];
    }
    tau[0] += w[1] * wb[2] - w[2] * wb[1];
    tau[1] += w[2] * wb[0] - w[0] * wb[2];
    tau[2] += w[0] * wb[1] - w[1] * wb[0];
    const float rho2 = v[0] * v[0] + v[1] * v[1] + v[2] * v[2], inv2 = 1.f / rho2, inv = sqrtf(inv2);
    const float r[3] = {v[0] * inv, v[1] * inv, v[2] * inv};
    // the rate's part across the edge, (dv x v) / |v|^2: w without its axial part
    const float wr = w[0] * r[0] + w[1] * r[1] + w[2] * r[2];
    const float wbr = wb[0] * r[0] + wb[1] * r[1] + wb[2] * r[2];
    const float wbw = 2.f * (wb[0] * w[0] + wb[1] * w[1] + wb[2] * w[2] - (roll ? wr * wbr : 0.f));
    float o[3];
    o[0] = (r[1] * tau[2] - r[2] * tau[1]) * inv + (wb[1] * dv[2] - wb[2] * dv[1] - wbw * v[0]) * inv2;
    o[1] = (r[2] * tau[0] - r[0] * tau[2]) * inv + (wb[2] * dv[0] - wb[0] * dv[2] - wbw * v[1]) * inv2;
    o[2] = (r[0] * tau[1] - r[1] * tau[0]) * inv + (wb[0] * dv[1] - wb[1] * dv[0] - wbw * v[2]) * inv2;
    if (roll) {
      const float rho = rho2 * inv, sg = v[2] >= 0.f ? 1.f : -1.f, D = rho + sg * v[2];
      const float tv = tau[0] * v[0] + tau[1] * v[1] + tau[2] * v[2];
      const float N = v[1] * dv[0] - v[0] * dv[1];
      const float wv = wb[0] * v[0] + wb[1] * v[1] + wb[2] * v[2];
      const float a = -sg * inv2 / D, c = N * wv;
      const float h[3] = {2.f * v[0] * inv2 + v[0] * inv / D, 2.f * v[1] * inv2 + v[1] * inv / D,
                          2.f * v[2] * inv2 + (v[2] * inv + sg) / D};
      const float tr = -sg * tv * inv2 / D;   // -(tau . r) s / (|v| D)
      o[0] += tr * v[1] + a * (-wv * dv[1] + N * wb[0] - c * h[0]);
      o[1] += -tr * v[0] + a * (wv * dv[0] + N * wb[1] - c * h[1]);
      o[2] += a * (N * wb[2] - c * h[2]);
    }
    vbar2[3 * e] = o[0];
    vbar2[3 * e + 1] = o[1];
    vbar2[3 * e + 2] = o[2];
  }
}

// ------------------------------------------------------------------ gates
// one thread per (edge, l, four channels; launch shape gate_dims)
template <typename OT>
__global__ void gate_dual_kernel(Dims d, long E, const float* __restrict__ U, const float* __restrict__ Ud,
                                 OT* __restrict__ Zd) {
  const int L = d.L, M = d.M, C = d.C;
  const int c = 4 * threadIdx.x, l = threadIdx.y;
  const int wU = d.wU(), wZ = d.wZ();
  for (long e = (long)blockIdx.x * blockDim.z + threadIdx.z; e < E; e += (long)gridDim.x * blockDim.z) {
    const float* ur = U + e * wU;
    const float* udr = Ud + e * wU;
    OT* zr = Zd + e * wZ;
    float u[4], ud[4], o[4];
    if (l == 0) {
      ld4(ur + c, u);
      ld4(udr + c, ud);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s = sigm(u[i]);
        o[i] = s * (1.f + u[i] * (1.f - s)) * ud[i];
      }
      st4(zr + c, o);
    } else {
      const int gc = d.gate_col(l, c);
      float s[4], sp[4], gd[4];
      ld4(ur + gc, s);
      ld4(udr + gc, gd);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[i] = sigm(s[i]);
        sp[i] = s[i] * (1.f - s[i]);
      }
      const int q = qhalf(l, M);
      for (int m = -q; m <= q; ++m) {
        const int uc = d.u_col(l, m, c);
        ld4(udr + uc, ud);
        ld4(ur + uc, u);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = s[i] * ud[i] + sp[i] * gd[i] * u[i];
        st4(zr + mm_col(l, m, c, L, C), o);
      }
    }
  }
}

// (zdot_bar, zbar) -> (udot_bar, ubar), E rows each; with WD false udot_bar
// is not written (the caller already holds it: it is the backward's ubar)
template <typename OT, bool WD>
__global__ void gate_dbwd_kernel(Dims d, long E, const float* __restrict__ U, const float* __restrict__ Ud,
                                 const float* __restrict__ Zdb, const float* __restrict__ Zb,
                                 OT* __restrict__ Udb, OT* __restrict__ Ub) {
  const int L = d.L, M = d.M, C = d.C;
  const int c = 4 * threadIdx.x, l = threadIdx.y;
  const int wU = d.wU(), wZ = d.wZ();
  for (long e = (long)blockIdx.x * blockDim.z + threadIdx.z; e < E; e += (long)gridDim.x * blockDim.z) {
    const float* ur = U + e * wU;
    const float* udr = Ud + e * wU;
    const float* zdb = Zdb + e * wZ;
    const float* zb = Zb + e * wZ;
    OT* udb = WD ? Udb + e * wU : nullptr;
    OT* ub = Ub + e * wU;
    float u[4], ud[4], a[4], b[4], o1[4], o2[4];
    if (l == 0) {
      ld4(ur + c, u);
      ld4(udr + c, ud);
      ld4(zdb + c, a);
      ld4(zb + c, b);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s = sigm(u[i]);
        const float s1 = s * (1.f + u[i] * (1.f - s));
        const float s2 = s * (1.f - s) * (2.f + u[i] * (1.f - 2.f * s));
        o1[i] = s1 * a[i];
        o2[i] = s2 * ud[i] * a[i] + s1 * b[i];
      }
      if (WD) st4(udb + c, o1);
      st4(ub + c, o2);
    } else {
      const int gc = d.gate_col(l, c);
      float s[4], sp[4], spp[4], gd[4], gdb[4] = {0.f, 0.f, 0.f, 0.f}, gb[4] = {0.f, 0.f, 0.f, 0.f};
      ld4(ur + gc, s);
      ld4(udr + gc, gd);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[i] = sigm(s[i]);
        sp[i] = s[i] * (1.f - s[i]);
        spp[i] = sp[i] * (1.f - 2.f * s[i]);
      }
      const int q = qhalf(l, M);
      for (int m = -q; m <= q; ++m) {
        const int uc = d.u_col(l, m, c), zc = mm_col(l, m, c, L, C);
        ld4(zdb + zc, a);
        ld4(zb + zc, b);
        ld4(ur + uc, u);
        ld4(udr + uc, ud);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o1[i] = s[i] * a[i];
          o2[i] = sp[i] * gd[i] * a[i] + s[i] * b[i];
          gdb[i] += a[i] * u[i];
          gb[i] += spp[i] * gd[i] * u[i] * a[i] + sp[i] * ud[i] * a[i] + sp[i] * u[i] * b[i];
        }
        if (WD) st4(udb + uc, o1);
        st4(ub + uc, o2);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) o1[i] = sp[i] * gdb[i];
      if (WD) st4(udb + gc, o1);
      st4(ub + gc, gb);
    }
  }
}

inline int grid_for(long n) {
  long b = (n + 255) / 256;
  if (b > 16384) b = 16384;
  if (b < 1) b = 1;
  return (int)b;
}

}  // namespace

int launch_edge_dual(const Dims& d, const GraphDev& g, const float* x, const float* px, const float* pos,
                     const float* ppos, const float* pedge, const float* S, const float* Sdot, void* Tdot,
                     float* omega, int bf16, hipStream_t s) {
  return dispatch_lm<EdgeDual>(d.L, d.M, d, g, x, px, pos, ppos, pedge, S, Sdot, Tdot, omega, bf16, s);
}

int launch_gate_dual(const Dims& d, long E, const float* U, const float* Udot, void* Zdot, int bf16, hipStream_t s) {
  if (E == 0) return hipSuccess;
  dim3 grid, block;
  gate_dims(d, E, &grid, &block);
  if (bf16)
    hipLaunchKernelGGL(gate_dual_kernel<bf16s>, grid, block, 0, s, d, E, U, Udot, static_cast<bf16s*>(Zdot));
  else
    hipLaunchKernelGGL(gate_dual_kernel<float>, grid, block, 0, s, d, E, U, Udot, static_cast<float*>(Zdot));
  return hipGetLastError();
}

int launch_node_dual(const Dims& d, const GraphDev& g, const float* pos, const float* omega, const float* V,
                     const float* Vdot, const float* env, const float* penv, float* ydot, int accumulate,
                     hipStream_t s) {
  return dispatch_lm<NodeDual>(d.L, d.M, d, g, pos, omega, V, Vdot, env, penv, ydot, accumulate, s);
}

int launch_edge_bwd_dual(const Dims& d, const GraphDev& g, const float* pos, const float* omega, const float* gy,
                         void* G2, int bf16, const float* V, const float* Vdot, const float* env, const float* penv,
                         float* p2, float* genv2, hipStream_t s) {
  return dispatch_lm<EdgeBwdDual>(d.L, d.M, d, g, pos, omega, gy, G2, bf16, V, Vdot, env, penv, p2, genv2, s);
}

int launch_pos2(const GraphDev& g, const float* pos, const float* ppos, const float* pedge, const float* omega,
                const float* pe, const float* pd, const float* ps, float* vbar2, int roll, hipStream_t s) {
  const long n = g.e1 - g.e0;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(pos2_kernel, dim3(grid_for(n)), dim3(256), 0, s, g, pos, ppos, pedge, omega, pe, pd, ps, vbar2,
                     roll);
  return hipGetLastError();
}

int launch_gate_dbwd(const Dims& d, long E, const float* U, const float* Udot, const float* Zdb, const float* Zb,
                     void* Udb, void* Ub, int bf16, hipStream_t s) {
  if (E == 0) return hipSuccess;
  dim3 grid, block;
  gate_dims(d, E, &grid, &block);
  if (bf16) {
    bf16s *o1 = static_cast<bf16s*>(Udb), *o2 = static_cast<bf16s*>(Ub);
    if (Udb)
      hipLaunchKernelGGL((gate_dbwd_kernel<bf16s, true>), grid, block, 0, s, d, E, U, Udot, Zdb, Zb, o1, o2);
    else
      hipLaunchKernelGGL((gate_dbwd_kernel<bf16s, false>), grid, block, 0, s, d, E, U, Udot, Zdb, Zb, o1, o2);
  } else {
    float *o1 = static_cast<float*>(Udb), *o2 = static_cast<float*>(Ub);
    if (Udb)
      hipLaunchKernelGGL((gate_dbwd_kernel<float, true>), grid, block, 0, s, d, E, U, Udot, Zdb, Zb, o1, o2);
    else
      hipLaunchKernelGGL((gate_dbwd_kernel<float, false>), grid, block, 0, s, d, E, U, Udot, Zdb, Zb, o1, o2);
  }
  return hipGetLastError();
}

int launch_node_bwd_dual(const Dims& d, const GraphDev& g, const float* x, const float* px, const float* pos,
                         const float* omega, const float* S, const float* Sdot, const float* Tdb, const float* Tb,
                         float* gx2, float* Sbar, float* Sdot_bar, float* p2_dst, float* p2_src, int accumulate,
                         hipStream_t s) {
  return dispatch_lm<NodeBwdDual>(d.L, d.M, d, g, x, px, pos, omega, S, Sdot, Tdb, Tb, gx2, Sbar, Sdot_bar, p2_dst,
                                  p2_src, accumulate, s);
}

}  // namespace so2
