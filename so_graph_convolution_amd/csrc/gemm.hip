// Grouped fp32 MFMA GEMM: 128x128 block tiles, 4 waves of 64x64, K tile 16,
// LDS double buffering, XCD-aware linear tile order.
#include "gemm.hpp"

namespace so2 {

namespace {

constexpr int BM = 128, BN = 128, BK = 16;
constexpr int PAD = 32;          // row pitch 160 floats: the two k rows of one MFMA read hit disjoint banks
constexpr int LDA_S = BM + PAD;
constexpr int LDB_S = BN + PAD;
constexpr int NT = 256;

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

struct TileRegs {
  floatx4 a[2];
  floatx4 b[2];
};

// linear block id -> tile id such that the blocks one XCD receives (round robin
// dispatch, 8 XCDs) cover a contiguous range of tiles, so tiles sharing an
// A row panel share that XCD's L2
__device__ inline int xcd_remap(int bid, int total) {
  const int q = total / 8, r = total % 8;
  const int x = bid % 8, i = bid / 8;
  return x < r ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

template <bool TA>
__device__ inline void load_a(const GemmProb& p, int m0, int k0, int kend, TileRegs& R) {
  const int t = threadIdx.x;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
    if (!TA) {
      const int i = t % 128, kq = t / 128 + 2 * r;
      const int gi = m0 + i, gk = k0 + 4 * kq;
      if (gi < p.M) {
        const float* src = p.A + (size_t)gi * p.lda + gk;
        if (gk + 3 < kend) {
          v = *reinterpret_cast<const floatx4*>(src);
        } else {
#pragma unroll
          for (int x = 0; x < 4; ++x) v[x] = (gk + x < kend) ? src[x] : 0.f;
        }
      }
    } else {
      const int k = t / 32 + 8 * r, iq = t % 32;
      const int gk = k0 + k, gi = m0 + 4 * iq;
      if (gk < kend) {
        const float* src = p.A + (size_t)gk * p.lda + gi;
        if (gi + 3 < p.M) {
          v = *reinterpret_cast<const floatx4*>(src);
        } else {
#pragma unroll
          for (int x = 0; x < 4; ++x) v[x] = (gi + x < p.M) ? src[x] : 0.f;
        }
      }
    }
    R.a[r] = v;
  }
}

template <bool TB>
__device__ inline void load_b(const GemmProb& p, int n0, int k0, int kend, TileRegs& R) {
  const int t = threadIdx.x;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    floatx4 v = {0.f, 0.f, 0.f, 0.f};
    if (!TB) {
      const int k = t / 32 + 8 * r, jq = t % 32;
      const int gk = k0 + k, gj = n0 + 4 * jq;
      if (gk < kend) {
        const float* src = p.B + (size_t)gk * p.ldb + gj;
        if (gj + 3 < p.N) {
          v = *reinterpret_cast<const floatx4*>(src);
        } else {
#pragma unroll
          for (int x = 0; x < 4; ++x) v[x] = (gj + x < p.N) ? src[x] : 0.f;
        }
      }
    } else {
      const int j = t % 128, kq = t / 128 + 2 * r;
      const int gj = n0 + j, gk = k0 + 4 * kq;
      if (gj < p.N) {
        const float* src = p.B + (size_t)gj * p.ldb + gk;
        if (gk + 3 < kend) {
          v = *reinterpret_cast<const floatx4*>(src);
        } else {
#pragma unroll
          for (int x = 0; x < 4; ++x) v[x] = (gk + x < kend) ? src[x] : 0.f;
        }
      }
    }
    R.b[r] = v;
  }
}

template <bool TA, bool TB>
__device__ inline void store_tiles(const TileRegs& R, float* As, float* Bs) {
  const int t = threadIdx.x;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    if (!TA) {
      const int i = t % 128, kq = t / 128 + 2 * r;
#pragma unroll
      for (int x = 0; x < 4; ++x) As[(4 * kq + x) * LDA_S + i] = R.a[r][x];
    } else {
      const int k = t / 32 + 8 * r, iq = t % 32;
      *reinterpret_cast<floatx4*>(As + k * LDA_S + 4 * iq) = R.a[r];
    }
    if (!TB) {
      const int k = t / 32 + 8 * r, jq = t % 32;
      *reinterpret_cast<floatx4*>(Bs + k * LDB_S + 4 * jq) = R.b[r];
    } else {
      const int j = t % 128, kq = t / 128 + 2 * r;
#pragma unroll
      for (int x = 0; x < 4; ++x) Bs[(4 * kq + x) * LDB_S + j] = R.b[r][x];
    }
  }
}

template <bool TA, bool TB>
__global__ __launch_bounds__(NT) void gemm_f32_kernel(GemmBatch batch) {
  __shared__ float As[2][BK * LDA_S];
  __shared__ float Bs[2][BK * LDB_S];

  const int tile = xcd_remap(blockIdx.x, batch.total_tiles);
  int pi = 0;
#pragma unroll 1
  for (int q = 1; q < batch.nprob; ++q)
    if (tile >= batch.p[q].tile_begin) pi = q;
  const GemmProb& p = batch.p[pi];
  int local = tile - p.tile_begin;
  const int per_split = p.tiles_m * p.tiles_n;
  const int split = local / per_split;
  local -= split * per_split;
  const int tm = local / p.tiles_n, tn = local - tm * p.tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = split * p.k_chunk;
  const int kend = min(p.K, kbeg + p.k_chunk);

  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int wm = wave / 2, wn = wave % 2;
  const int li = lane % 32, lk = lane / 32;

  floatx16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int nk = (kend - kbeg + BK - 1) / BK;
  TileRegs R;
  if (nk > 0) {
    load_a<TA>(p, m0, kbeg, kend, R);
    load_b<TB>(p, n0, kbeg, kend, R);
    store_tiles<TA, TB>(R, As[0], Bs[0]);
  }
  __syncthreads();
#pragma unroll 1
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      load_a<TA>(p, m0, kbeg + (kt + 1) * BK, kend, R);
      load_b<TB>(p, n0, kbeg + (kt + 1) * BK, kend, R);
    }
    const float* as = As[cur] + wm * 64 + li;
    const float* bs = Bs[cur] + wn * 64 + li;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 2) {
      const float a0 = as[(kk + lk) * LDA_S];
      const float a1 = as[(kk + lk) * LDA_S + 32];
      const float b0 = bs[(kk + lk) * LDB_S];
      const float b1 = bs[(kk + lk) * LDB_S + 32];
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
    }
    if (kt + 1 < nk) store_tiles<TA, TB>(R, As[cur ^ 1], Bs[cur ^ 1]);
    __syncthreads();
  }

  // epilogue: lane holds rows 8*(r/4) + 4*(lane/32) + r%4, column lane%32 of each 32x32 tile
  float* out;
  int ldo;
  bool acc_in;
  if (p.partial) {
    out = p.C + (size_t)split * p.M * p.N;
    ldo = p.N;
    acc_in = false;
  } else {
    out = p.C;
    ldo = p.ldc;
    acc_in = p.accumulate != 0;
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int j = n0 + wn * 64 + b * 32 + li;
      if (j >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = m0 + wm * 64 + a * 32 + 8 * (r / 4) + 4 * lk + (r % 4);
        if (i < p.M) {
          float* dst = out + (size_t)i * ldo + j;
          *dst = acc_in ? *dst + acc[a][b][r] : acc[a][b][r];
        }
      }
    }
}

__global__ void gemm_reduce_kernel(const float* __restrict__ P, int splits, int M, int N, float* __restrict__ C,
                                   int ldc, int accumulate) {
  const size_t n = (size_t)M * N;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (size_t)gridDim.x * blockDim.x) {
    float s = 0.f;
    for (int q = 0; q < splits; ++q) s += P[(size_t)q * n + idx];
    const size_t i = idx / N, j = idx - i * N;
    float* dst = C + i * ldc + j;
    *dst = accumulate ? *dst + s : s;
  }
}

}  // namespace

int gemm_run(GemmBatch& b, bool TA, bool TB, hipStream_t s) {
  int total = 0;
  for (int q = 0; q < b.nprob; ++q) {
    GemmProb& p = b.p[q];
    p.tiles_m = (p.M + BM - 1) / BM;
    p.tiles_n = (p.N + BN - 1) / BN;
    if (p.k_splits < 1) p.k_splits = 1;
    if (p.k_splits == 1 && p.k_chunk <= 0) p.k_chunk = p.K;
    p.tile_begin = total;
    if (p.M > 0 && p.N > 0) total += p.tiles_m * p.tiles_n * p.k_splits;
  }
  b.total_tiles = total;
  if (total == 0) return hipSuccess;
  dim3 grid(total), block(NT);
  if (!TA && !TB) hipLaunchKernelGGL((gemm_f32_kernel<false, false>), grid, block, 0, s, b);
  else if (!TA && TB) hipLaunchKernelGGL((gemm_f32_kernel<false, true>), grid, block, 0, s, b);
  else if (TA && !TB) hipLaunchKernelGGL((gemm_f32_kernel<true, false>), grid, block, 0, s, b);
  else hipLaunchKernelGGL((gemm_f32_kernel<true, true>), grid, block, 0, s, b);
  return hipGetLastError();
}

int gemm_reduce(const float* P, int splits, int M, int N, float* C, int ldc, int accumulate, hipStream_t s) {
  const size_t n = (size_t)M * N;
  if (n == 0) return hipSuccess;
  int blocks = (int)((n + 255) / 256);
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(gemm_reduce_kernel, dim3(blocks), dim3(256), 0, s, P, splits, M, N, C, ldc, accumulate);
  return hipGetLastError();
}

}  // namespace so2
