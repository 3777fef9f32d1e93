// Per-tile rotation state (edge frame, compact Wigner rows and their
// derivatives) built in LDS, and per-channel rotation products kept in
// registers. Used by every edge- and node-centric kernel.
#pragma once
#include "ops.hpp"
#include "wigner.hpp"
#include "so3_gen.hpp"

namespace so2 {

// so(3) generators in the real harmonic basis, G_k = d/dt D(exp(t [e_k]_x)) at
// t = 0, k = x, y, z; degree l block at gen_off(l), (2l+1)^2 row-major.
// Each translation unit holds its own copy; the host fills every copy once
// per device (library init) through that unit's upload function.
static __constant__ float c_gen[3 * kGenSize];

static inline int upload_generators_here(const float* host) {
  return (int)hipMemcpyToSymbol(HIP_SYMBOL(c_gen), host, sizeof(float) * 3 * kGenSize, 0, hipMemcpyHostToDevice);
}

// retained-row index of (l, m): rows ordered l = 0..L, m = -q_l..q_l
__host__ __device__ constexpr inline int ridx(int l, int m, int M) {
  int o = 0;
  for (int k = 0; k < l; ++k) o += 2 * qhalf(k, M) + 1;
  return o + m + qhalf(l, M);
}

__host__ __device__ constexpr inline int wig_stride_c(int L, int M) {
  int s = 9;
  for (int l = 2; l < L; ++l) {
    const int r = rows_kept(l, L, M);
    const int w = (2 * r + 1) * (2 * l + 1);
    s = s > w ? s : w;
  }
  return s;
}

struct EdgeGeo {
  float rx, ry, rz, rho;
};

// Edge vector v = pos[src] - pos[dst] + shift (TrimSO(2) page, Appendix A.1),
// its length and direction, and D^(1) of the edge frame.
__device__ inline EdgeGeo edge_geometry(const float* __restrict__ pos, const float* __restrict__ shift, int j, int i,
                                        long e, float* D1) {
  float vx = pos[3 * j] - pos[3 * i], vy = pos[3 * j + 1] - pos[3 * i + 1], vz = pos[3 * j + 2] - pos[3 * i + 2];
  if (shift) {
    vx += shift[3 * e];
    vy += shift[3 * e + 1];
    vz += shift[3 * e + 2];
  }
  const float rho = sqrtf(vx * vx + vy * vy + vz * vz);
  const float inv = 1.f / rho;
  EdgeGeo g{vx * inv, vy * inv, vz * inv, rho};
  float R[9];
  edge_frame<float>(g.rx, g.ry, g.rz, R);
  wigner_l1<float>(R, D1);
  return g;
}

// Rd[e][K] = R_e (sum_k w_k G_k) with per-edge weights w[e][3]; cooperative.
// Column col of G_k has its nonzeros at the rows gen_cand gives for col.
__device__ inline void rot_directional(int L, int M, int ne, const float* R, int ldr, const float* w, int ldw,
                                       float* Rd, int ldd) {
  const int K = k_count(L, M);
  for (int idx = threadIdx.x; idx < ne * K; idx += blockDim.x) {
    const int e = idx / K;
    const int rem = idx - e * K;
    int l = 0;
    while (rem >= rot_off(l + 1, M)) ++l;
    const int n = 2 * l + 1;
    const int loc = rem - rot_off(l, M);
    const int mi = loc / n, col = loc - mi * n;
    const float* Rrow = R + e * ldr + rot_off(l, M) + mi * n;
    float s = 0.f;
    for (int k = 0; k < 3; ++k) {
      const float* G = c_gen + k * kGenSize + gen_off(l);
      int p0, p1;
      gen_cand(k, col - l, &p0, &p1);
      float t = 0.f;
      if (p0 >= -l && p0 <= l) t = __builtin_fmaf(Rrow[p0 + l], G[(p0 + l) * n + col], t);
      if (p1 != p0 && p1 >= -l && p1 <= l) t = __builtin_fmaf(Rrow[p1 + l], G[(p1 + l) * n + col], t);
      s = __builtin_fmaf(w[e * ldw + k], t, s);
    }
    Rd[e * ldd + rem] = s;
  }
}

// Rotation entries live in LDS and are read with volatile LDS loads: each use
// is a broadcast LDS read instead of a register kept live across the unrolled
// loops (which would cost K_{L,M} registers per rotation table and occupancy).
typedef const float* RotPtr;
__device__ __forceinline__ float rot_ld(RotPtr p) {
  return *(const volatile __attribute__((address_space(3))) float*)(p);
}

// The generator blocks as compile-time constants (so3_gen.hpp): every product
// with a generator entry below has indices that are constants after
// unrolling, so the entry is a literal operand of its instruction.
constexpr GenTable kGenTab = make_gen_table();
__device__ __forceinline__ float gen_at(int k, int l, int idx) { return kGenTab.v[k * kGenSize + gen_off(l) + idx]; }

// <a, G_k^(l) b> for degree-l blocks a, b (k, l compile-time after
// unrolling), taken as <G_k^T a, b>: column c of G_k has its nonzeros at the
// rows gen_cand gives for order c (the generators are antisymmetric), so each
// entry of G_k^T a is two table products.
// (Explicit fused forms throughout: every kernel instantiation rounds alike.)
template <int L>
__device__ __forceinline__ float gen_form(int k, int l, const float* a, const float* b) {
  const int n = 2 * l + 1;
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 2 * L + 1; ++c) {
    if (c < n) {
      int i0, i1;
      gen_cand(k, c - l, &i0, &i1);
      float g = 0.f;
      if (i0 >= -l && i0 <= l) g = __builtin_fmaf(gen_at(k, l, (i0 + l) * n + c), a[i0 + l], g);
      if (i1 != i0 && i1 >= -l && i1 <= l) g = __builtin_fmaf(gen_at(k, l, (i1 + l) * n + c), a[i1 + l], g);
      s = __builtin_fmaf(g, b[c], s);
    }
  }
  return s;
}

// g = G_w^(l) a (TR: G_w^(l)T a) for G_w = sum_k w_k G_k with per-edge
// weights w: the directional derivative of the rotation rows is R G_w, so
// (R G_w) a = R (G_w a) and (R G_w)^T t = G_w^T (R^T t) need no per-edge
// table of R G_w.
// Each table entry is scaled by its w_k before it meets a: no partial sum
// depends on a alone, so nothing is hoisted out of a loop over edges that
// share a.
template <int L, bool TR>
__device__ __forceinline__ void gw_apply(const float (&w)[3], int l, const float* a, float (&g)[2 * L + 1]) {
  const int n = 2 * l + 1;
#pragma unroll
  for (int i = 0; i < 2 * L + 1; ++i) {
    if (i < n) {
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        int j0, j1;
        gen_cand(k, i - l, &j0, &j1);
        if (j0 >= -l && j0 <= l) s = __builtin_fmaf(w[k] * gen_at(k, l, TR ? (j0 + l) * n + i : i * n + j0 + l), a[j0 + l], s);
        if (j1 != j0 && j1 >= -l && j1 <= l)
          s = __builtin_fmaf(w[k] * gen_at(k, l, TR ? (j1 + l) * n + i : i * n + j1 + l), a[j1 + l], s);
      }
      g[i] = s;
    }
  }
}

// o[ridx(l,m)] = sum_n R[l][m][n] a[l*l + l + n]   (rotate degree-major -> retained rows)
template <int L, int M>
__device__ __forceinline__ void rot_fwd(RotPtr R, const float (&a)[(L + 1) * (L + 1)],
                                        float (&o)[q_count(L, M)]) {
#pragma unroll
  for (int l = 0; l <= L; ++l) {
    const int q = qhalf(l, M), n = 2 * l + 1;
#pragma unroll
    for (int m = -q; m <= q; ++m) {
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < n; ++k) s += rot_ld(R + rot_off(l, M) + (m + q) * n + k) * a[l * l + k];
      o[ridx(l, m, M)] = s;
    }
  }
}

// row (l, m) of a compact rotation table, loaded once into registers
template <int L>
__device__ __forceinline__ void load_row(RotPtr R, int off, int n, float (&r)[2 * L + 1]) {
#pragma unroll
  for (int k = 0; k < 2 * L + 1; ++k)
    if (k < n) r[k] = rot_ld(R + off + k);
}

template <int L>
__device__ __forceinline__ float row_dot(const float (&r)[2 * L + 1], const float* a, int n) {
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 2 * L + 1; ++k)
    if (k < n) s += r[k] * a[k];
  return s;
}

template <int L>
__device__ __forceinline__ void row_axpy(const float (&r)[2 * L + 1], float v, float* o, int n) {
#pragma unroll
  for (int k = 0; k < 2 * L + 1; ++k)
    if (k < n) o[k] += r[k] * v;
}

// o[l*l + l + n] += sum_m R[l][m][n] t[ridx(l,m)]   (inverse rotation of retained rows)
template <int L, int M>
__device__ __forceinline__ void rot_bwd_acc(RotPtr R, const float (&t)[q_count(L, M)],
                                            float (&o)[(L + 1) * (L + 1)]) {
#pragma unroll
  for (int l = 0; l <= L; ++l) {
    const int q = qhalf(l, M), n = 2 * l + 1;
#pragma unroll
    for (int m = -q; m <= q; ++m) {
      const float tv = t[ridx(l, m, M)];
#pragma unroll
      for (int k = 0; k < n; ++k) o[l * l + k] += rot_ld(R + rot_off(l, M) + (m + q) * n + k) * tv;
    }
  }
}

// Incoming-edge range of `node` clipped to the edge chunk [e0, e1).
__device__ inline void in_range(const GraphDev& g, int node, int* beg, int* end) {
  long b = g.dst_ptr[node], e = g.dst_ptr[node + 1];
  if (b < g.e0) b = g.e0;
  if (e > g.e1) e = g.e1;
  *beg = (int)b;
  *end = (int)(e > b ? e : b);
}

// Positions [beg, end) in src_perm of the outgoing edges of `node` that lie in
// the chunk: within a sender's segment the edge ids increase (stable sort), so
// both ends are found by binary search.
__device__ inline void out_range(const GraphDev& g, int node, int* beg, int* end) {
  int b = g.src_ptr[node], e = g.src_ptr[node + 1];
  if (g.e0 > 0 || g.e1 < g.E) {
    int lo = b, hi = e;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (g.src_perm[mid] < g.e0) lo = mid + 1;
      else hi = mid;
    }
    const int nb = lo;
    hi = e;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (g.src_perm[mid] < g.e1) lo = mid + 1;
      else hi = mid;
    }
    b = nb;
    e = lo;
  }
  *beg = b;
  *end = e;
}

// Node-centric kernels run two thread groups per node (threads [0, CW) and
// [CW, 2 CW), CW = C rounded up to 64): group p takes the tile's edges
// t = p, p + 2, ... with the same channels, doubling the waves in flight per
// node for the same LDS tile. At the end the groups' register accumulators are
// combined through LDS (`buf`, capacity `cap` floats, in row chunks) and group
// 0 writes (or adds) the node row out[r * C + c]. The caller guarantees
// cap >= CW (one row; see comb_buffer), so every round advances by a row.
constexpr int kCombFallback = 512;   // floats; CW <= 256

// `tile` (capacity tile_cap) if it holds one channel row of CW floats, else the
// dedicated fallback buffer
__device__ __forceinline__ float* comb_buffer(float* tile, int tile_cap, float* fallback, int CW, int* cap) {
  if (tile_cap >= CW) {
    *cap = tile_cap;
    return tile;
  }
  *cap = kCombFallback;
  return fallback;
}

template <int D>
__device__ inline void combine_groups(const float (&acc)[D], float* buf, int cap, int c, int grp, int CW, bool act,
                                      float* out, int C, int accumulate) {
  const int fit = cap / CW;
  const int rows = fit < 1 ? 1 : (fit < D ? fit : D);
  for (int r0 = 0; r0 < D; r0 += rows) {
    __syncthreads();
    if (grp == 1) {
#pragma unroll
      for (int r = 0; r < D; ++r)
        if (r >= r0 && r < r0 + rows) buf[(r - r0) * CW + c] = acc[r];
    }
    __syncthreads();
    if (grp == 0 && act) {
#pragma unroll
      for (int r = 0; r < D; ++r)
        if (r >= r0 && r < r0 + rows) {
          const float v = acc[r] + buf[(r - r0) * CW + c];
          float* o = out + (size_t)r * C + c;
          *o = accumulate ? *o + v : v;
        }
    }
  }
}

// Degree split of the lmax-6 node-centric backward kernels: of the two
// thread groups of a node's block, group 0 owns degrees [0, LS) and group 1
// degrees [LS, L]; both walk every edge of a tile, each thread keeping the
// node rows and accumulators of its own degrees only and writing those rows
// itself (no combine through LDS). LS balances the rotation work of the two
// groups: degree l has (2 min(l, M) + 1)(2l + 1) retained row entries.
__host__ __device__ constexpr inline int deg_cost(int l, int M) { return (2 * qhalf(l, M) + 1) * (2 * l + 1); }
__host__ __device__ constexpr inline int deg_split(int L, int M) {
  int best = 1, bv = 1 << 30;
  for (int s = 1; s <= L; ++s) {
    int a = 0, b = 0;
    for (int l = 0; l <= L; ++l) {
      if (l < s) a += deg_cost(l, M);
      else b += deg_cost(l, M);
    }
    const int v = a > b ? a : b;
    if (v < bv) {
      bv = v;
      best = s;
    }
  }
  return best;   // L = 0: 1, group 1 owns no degree
}
// node rows of the larger half
__host__ __device__ constexpr inline int half_rows(int L, int M) {
  const int s = deg_split(L, M), a = s * s, b = (L + 1) * (L + 1) - a;
  return a > b ? a : b;
}
// retained rows (l, m) of degrees [LA, LB)
__host__ __device__ constexpr inline int q_range(int LA, int LB, int M) {
  int s = 0;
  for (int l = LA; l < LB; ++l) s += 2 * qhalf(l, M) + 1;
  return s;
}

// sum over a wavefront (64 lanes)
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// sum over aligned groups of `width` lanes (a power of two <= 64), same
// butterfly order in every group; every lane receives its group's sum
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int off = width >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// head of channel c (channels past C map to head 0; their values are unused)
__device__ __forceinline__ int c_head(const Dims& d, int c) { return c < d.C ? c / d.hs() : 0; }

// Per-head sums of the per-channel values of edge slot t (one thread per
// channel c, lane/wave of a block of at most 4 waves): heads of hs = C / H
// channels. Heads that are whole waves (or H = 1) take the wave sums through
// red[(t * 4 + wave) * stride + k]; heads of 16 or 32 channels are summed
// inside the wave into hsum[t * kMaxHeads + head].
__device__ __forceinline__ void head_partial(float v, const Dims& d, int c, int t, float* red, int stride, int k,
                                             float* hsum) {
  const int hs = d.hs(), lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  if (d.H > 1 && hs < 64) {
    const float s = group_sum(v, hs);
    if (c < d.C && lane % hs == 0) hsum[t * kMaxHeads + c / hs] = s;
  } else {
    const float s = wave_sum(v);
    if (lane == 0) red[(t * 4 + wave) * stride + k] = s;
  }
}
// the head total written by head_partial (after a barrier)
__device__ __forceinline__ float head_total(const Dims& d, int t, int h, const float* red, int stride, int k,
                                            const float* hsum) {
  const int hs = d.hs();
  if (d.H > 1 && hs < 64) return hsum[t * kMaxHeads + h];
  float s = 0.f;
  for (int w = (h * hs) / 64; w < ((h + 1) * hs + 63) / 64; ++w) s += red[(t * 4 + w) * stride + k];
  return s;
}

}  // namespace so2
