// Grouped MFMA GEMMs with LDS double buffering and an XCD-aware linear tile order.
//   float32 operands : 256x128 blocks, 8 waves of 64x64 (2x2 v_mfma_f32_32x32x2_f32), K tile 16
//   complex float32  : 128 x 64-complex blocks, three real products per complex one (below)
//   bfloat16 operands: 256x256 blocks, 16 waves of 64x64 (v_mfma_f32_32x32x16_bf16), K tile 64
//
// Operand staging: every global load runs along the operand's contiguous
// dimension (float4 per lane, consecutive lanes on consecutive addresses), and
// the LDS layout follows the global one:
//   A row-major [i][k]  -> As[i][k]  pitch BK+4      A transposed [k][i] -> As[k][i] pitch BM+4
//   B row-major [k][j]  -> Bs[k][j]  pitch BN+4      B transposed [j][k] -> Bs[j][k] pitch BK+4
// The sum over k does not depend on which k an MFMA step takes, so step s of a
// K tile (BK/2 steps of v_mfma_f32_32x32x2_f32) gives lane half lk (lanes
// 0-31, 32-63) k = (BK/2) lk + s in both operands. A lane's values of a
// k-contiguous tile are then adjacent (128-bit LDS reads; pitch BK+4 starts
// any 16 rows on distinct 4-bank groups); a k-major tile is read one value
// per step, 32 consecutive rows per lane half, and its pitch R+4 puts the two
// halves (BK/2 rows apart) on disjoint banks.
#include "gemm.hpp"
#include "gemm_tile.hpp"
#include "gemm_dma.hpp"

namespace so2 {

namespace {

// Measured on MI355X for the per-order shapes (725k rows, K and N 640..2048):
// a 2x2 MFMA wave tile with K tile 16 at four waves per SIMD (accumulators in
// VGPRs) ran at 117-128 TFLOP/s in 128x128 blocks; 4x2 or 2x4 wave tiles
// (one wave per SIMD) and K tiles of 8 or 32 were slower. 256x128 blocks of
// 8 waves halve the re-streaming of the (L2-exceeding) weight operand per
// flop: 123-131 TFLOP/s for A.B and A.B^T.
constexpr int WM = 2, WN = 2;              // 32x32 MFMA tiles per wave
constexpr int WAVES_M = 4;                 // waves along M (2 along N)
constexpr int BM = 64 * WAVES_M, BN = 128;
constexpr int BK_TILE = 16;
constexpr int WAVES_PER_SIMD = 4;
constexpr int NT = 64 * WAVES_M * 2;

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

// R = rows of the tile (BM or BN)
template <int BK, int R>
struct Cfg {
  static constexpr int PK = BK + 4;                 // pitch of k-contiguous tiles
  static constexpr int PW = R + 4;                  // pitch of k-major tiles: (BK/2) PW = 32 mod 64 banks
  static constexpr int KMAJ = BK * PW;              // floats of a k-major tile
  static constexpr int KCON = R * PK;               // floats of a k-contiguous tile
  static constexpr int NRC = (R * BK / 4) / NT;     // float4 loads per thread of a k-contiguous tile
  static constexpr int NRM = (BK * R / 4) / NT;     // float4 loads per thread of a k-major tile
};

template <bool T, int BK, int R>
constexpr int tile_floats() { return T ? Cfg<BK, R>::KMAJ : Cfg<BK, R>::KCON; }

// Load one operand tile into registers.
//   KCONTIG: the global rows run along k (row-major [row][k]); else along the
//   128-wide dimension (row-major [k][row]).
template <bool KCONTIG, int BK, int R>
__device__ inline void load_tile(const float* __restrict__ P, int ld, int r0, int rlim, int k0, int kend,
                                 floatx4 (&v)[KCONTIG ? Cfg<BK, R>::NRC : Cfg<BK, R>::NRM]) {
  const int t = threadIdx.x;
  if (KCONTIG) {
    constexpr int LPR = BK / 4;            // lanes per row
    constexpr int RPP = NT / LPR;          // rows per pass
#pragma unroll
    for (int p = 0; p < Cfg<BK, R>::NRC; ++p) {
      const int row = p * RPP + t / LPR, q = t % LPR;
      const int gr = r0 + row, gk = k0 + 4 * q;
      floatx4 x = {0.f, 0.f, 0.f, 0.f};
      if (gr < rlim) {
        const float* src = P + (size_t)gr * ld + gk;
        if (gk + 3 < kend) {
          x = *reinterpret_cast<const floatx4*>(src);
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) x[c] = (gk + c < kend) ? src[c] : 0.f;
        }
      }
      v[p] = x;
    }
  } else {
#pragma unroll
    for (int p = 0; p < Cfg<BK, R>::NRM; ++p) {
      constexpr int LPR = R / 4, KPP = NT / LPR;
      const int k = p * KPP + t / LPR, q = t % LPR;
      const int gk = k0 + k, gr = r0 + 4 * q;
      floatx4 x = {0.f, 0.f, 0.f, 0.f};
      if (gk < kend) {
        const float* src = P + (size_t)gk * ld + gr;
        if (gr + 3 < rlim) {
          x = *reinterpret_cast<const floatx4*>(src);
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c) x[c] = (gr + c < rlim) ? src[c] : 0.f;
        }
      }
      v[p] = x;
    }
  }
}

template <bool KCONTIG, int BK, int R>
__device__ inline void store_tile(float* __restrict__ S, const floatx4 (&v)[KCONTIG ? Cfg<BK, R>::NRC : Cfg<BK, R>::NRM]) {
  const int t = threadIdx.x;
  if (KCONTIG) {
    constexpr int LPR = BK / 4, RPP = NT / LPR;
#pragma unroll
    for (int p = 0; p < Cfg<BK, R>::NRC; ++p) {
      const int row = p * RPP + t / LPR, q = t % LPR;
      *reinterpret_cast<floatx4*>(S + row * Cfg<BK, R>::PK + 4 * q) = v[p];
    }
  } else {
    constexpr int LPR = R / 4, KPP = NT / LPR;
#pragma unroll
    for (int p = 0; p < Cfg<BK, R>::NRM; ++p) {
      const int k = p * KPP + t / LPR, q = t % LPR;
      *reinterpret_cast<floatx4*>(S + k * Cfg<BK, R>::PW + 4 * q) = v[p];
    }
  }
}

// MFMA operands of one K tile for lane half lk: row `row`, k = (BK/2) lk + s
template <bool KCONTIG, int BK, int R>
__device__ __forceinline__ void frag(const float* S, int row, int lk, float (&f)[BK / 2]) {
  static_assert(BK % 8 == 0, "two 128-bit reads per lane half");
  if (KCONTIG) {
    const floatx4* q = reinterpret_cast<const floatx4*>(S + row * Cfg<BK, R>::PK + (BK / 2) * lk);
#pragma unroll
    for (int v = 0; v < BK / 8; ++v) {
      const floatx4 u = q[v];
#pragma unroll
      for (int c = 0; c < 4; ++c) f[4 * v + c] = u[c];
    }
  } else {
#pragma unroll
    for (int s = 0; s < BK / 2; ++s) f[s] = S[((BK / 2) * lk + s) * Cfg<BK, R>::PW + row];
  }
}

// epilogue: lane holds rows 8*(r/4) + 4*(lane/32) + r%4, column lane%32 of each 32x32 tile
__device__ inline void store_acc(const GemmProb& p, int split, int m0, int n0, int wm, int wn, int li, int lk,
                                 const floatx16 (&acc)[WM][WN]) {
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
  for (int a = 0; a < WM; ++a)
#pragma unroll
    for (int b = 0; b < WN; ++b) {
      const int j = n0 + wn * 32 * WN + b * 32 + li;
      if (j >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = m0 + wm * 32 * WM + a * 32 + 8 * (r / 4) + 4 * lk + (r % 4);
        if (i < p.M) {
          float* dst = out + (size_t)i * ldo + j;
          *dst = acc_in ? *dst + acc[a][b][r] : acc[a][b][r];
        }
      }
    }
}

template <bool TA, bool TB, int BK>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(WAVES_PER_SIMD, 8))) void gemm_f32_kernel(
    GemmBatch batch) {
  // A is k-contiguous when not transposed; B is k-contiguous when transposed
  constexpr bool AK = !TA, BKC = TB;
  constexpr int SA = tile_floats<!AK, BK, BM>(), SB = tile_floats<!BKC, BK, BN>();
  __shared__ __attribute__((aligned(16))) float As[2][SA];
  __shared__ __attribute__((aligned(16))) float Bs[2][SB];

  int pi, local;
  decode_tile(batch, xcd_remap(blockIdx.x, batch.total_tiles), &pi, &local);
  const GemmProb& p = batch.p[pi];
  const int per_split = p.tiles_m * p.tiles_n;
  const int split = local / per_split;
  local -= split * per_split;
  const int tm = local / p.tiles_n, tn = local - tm * p.tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = split * p.k_chunk;
  const int kend = min(p.K, kbeg + p.k_chunk);

  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int wm = wave / 2, wn = wave % 2;   // waves: WAVES_M along M, 2 along N
  const int li = lane % 32, lk = lane / 32;

  floatx16 acc[WM][WN];
#pragma unroll
  for (int a = 0; a < WM; ++a)
#pragma unroll
    for (int b = 0; b < WN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int nk = (kend - kbeg + BK - 1) / BK;
  floatx4 ra[AK ? Cfg<BK, BM>::NRC : Cfg<BK, BM>::NRM];
  floatx4 rb[BKC ? Cfg<BK, BN>::NRC : Cfg<BK, BN>::NRM];
  if (nk > 0) {
    load_tile<AK, BK, BM>(static_cast<const float*>(p.A), p.lda, m0, p.M, kbeg, kend, ra);
    load_tile<BKC, BK, BN>(static_cast<const float*>(p.B), p.ldb, n0, p.N, kbeg, kend, rb);
    store_tile<AK, BK, BM>(As[0], ra);
    store_tile<BKC, BK, BN>(Bs[0], rb);
  }
  __syncthreads();
#pragma unroll 1
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      load_tile<AK, BK, BM>(static_cast<const float*>(p.A), p.lda, m0, p.M, kbeg + (kt + 1) * BK, kend, ra);
      load_tile<BKC, BK, BN>(static_cast<const float*>(p.B), p.ldb, n0, p.N, kbeg + (kt + 1) * BK, kend, rb);
    }
    const float* as = As[cur];
    const float* bs = Bs[cur];
    const int ra0 = wm * 32 * WM + li, rb0 = wn * 32 * WN + li;
    float av[WM][BK / 2], bv[WN][BK / 2];
#pragma unroll
    for (int a = 0; a < WM; ++a) frag<AK, BK, BM>(as, ra0 + 32 * a, lk, av[a]);
#pragma unroll
    for (int b = 0; b < WN; ++b) frag<BKC, BK, BN>(bs, rb0 + 32 * b, lk, bv[b]);
#pragma unroll
    for (int s = 0; s < BK / 2; ++s)
#pragma unroll
      for (int a = 0; a < WM; ++a)
#pragma unroll
        for (int b = 0; b < WN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[a][s], bv[b][s], acc[a][b], 0, 0, 0);
    if (kt + 1 < nk) {
      store_tile<AK, BK, BM>(As[cur ^ 1], ra);
      store_tile<BKC, BK, BN>(Bs[cur ^ 1], rb);
    }
    __syncthreads();
  }

  store_acc(p, split, m0, n0, wm, wn, li, lk, acc);
}


// ---------------------------------------------------------------- complex products (float32)
// Block tile 128 rows x 64 complex columns of 8 waves (4 along M x 2 along N),
// each wave 32x32 complex outputs with three accumulators (P1, P2, P3 of the
// three-product form); K tile 16; a, b, c, d staged as four LDS tiles, the
// sums a + sA b and c + sB d formed from the fragments in registers. 64 KB of
// LDS for two stages: two blocks per CU. Measured on MI355X at the per-order
// shapes (725k rows): 1.17-1.26x faster than the realified product with four
// real products.
//
// The sum over k does not depend on which k each MFMA step takes, so step s
// (0..7) of lane half lk takes k = 8 lk + s in both operands: a lane's eight
// values of a k-contiguous tile are adjacent and arrive in two 128-bit LDS
// reads (pitch 20 dwords: any 16 rows start on distinct 4-bank groups). A
// k-major tile is read one value per step at pitch R + 4, which puts the two
// lane halves (8 rows apart) on disjoint banks.
constexpr int CBM = 128, CBN = 64, CBK = 16, CNT = 512;
template <bool KCONTIG, int R>
struct CT {
  static constexpr int PK = CBK + 4;
  static constexpr int PW = R + 4;
  static constexpr int FL = KCONTIG ? R * PK : CBK * PW;
  static constexpr int V4 = R * CBK / 4;
  static constexpr int NL = (V4 + CNT - 1) / CNT;
};
template <bool KCONTIG, int R>
__device__ inline void cload(const float* __restrict__ P, int ld, int r0, int rlim, int k0, int kend,
                             floatx4 (&v)[CT<KCONTIG, R>::NL]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int p = 0; p < CT<KCONTIG, R>::NL; ++p) {
    const int idx = p * CNT + t;
    floatx4 x = {0.f, 0.f, 0.f, 0.f};
    if (idx < CT<KCONTIG, R>::V4) {
      if (KCONTIG) {
        const int row = idx / (CBK / 4), q = idx % (CBK / 4);
        const int gr = r0 + row, gk = k0 + 4 * q;
        if (gr < rlim) {
          const float* src = P + (size_t)gr * ld + gk;
          if (gk + 3 < kend) x = *reinterpret_cast<const floatx4*>(src);
          else
#pragma unroll
            for (int c = 0; c < 4; ++c) x[c] = (gk + c < kend) ? src[c] : 0.f;
        }
      } else {
        const int k = idx / (R / 4), q = idx % (R / 4);
        const int gk = k0 + k, gr = r0 + 4 * q;
        if (gk < kend) {
          const float* src = P + (size_t)gk * ld + gr;
          if (gr + 3 < rlim) x = *reinterpret_cast<const floatx4*>(src);
          else
#pragma unroll
            for (int c = 0; c < 4; ++c) x[c] = (gr + c < rlim) ? src[c] : 0.f;
        }
      }
    }
    v[p] = x;
  }
}
template <bool KCONTIG, int R>
__device__ inline void cstore(float* __restrict__ S, const floatx4 (&v)[CT<KCONTIG, R>::NL]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int p = 0; p < CT<KCONTIG, R>::NL; ++p) {
    const int idx = p * CNT + t;
    if (idx < CT<KCONTIG, R>::V4) {
      if (KCONTIG) {
        const int row = idx / (CBK / 4), q = idx % (CBK / 4);
        *reinterpret_cast<floatx4*>(S + row * CT<KCONTIG, R>::PK + 4 * q) = v[p];
      } else {
        const int k = idx / (R / 4), q = idx % (R / 4);
        *reinterpret_cast<floatx4*>(S + k * CT<KCONTIG, R>::PW + 4 * q) = v[p];
      }
    }
  }
}
// The eight values of one K tile that lane half lk feeds its MFMA steps with:
// row `row`, k = 8 lk + s.
template <bool KCONTIG, int R>
__device__ __forceinline__ void cfrag(const float* S, int row, int lk, float (&f)[CBK / 2]) {
  if (KCONTIG) {
    const floatx4* q = reinterpret_cast<const floatx4*>(S + row * CT<KCONTIG, R>::PK + 8 * lk);
    const floatx4 u = q[0], w = q[1];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      f[c] = u[c];
      f[4 + c] = w[c];
    }
  } else {
#pragma unroll
    for (int s = 0; s < CBK / 2; ++s) f[s] = S[(8 * lk + s) * CT<KCONTIG, R>::PW + row];
  }
}

// epilogue: Re = P1 - sig P2 to C, Im = P3 - P1 - sig P2 N columns right (sig = sA sB)
__device__ inline void cplx_store(const GemmProb& p, int split, int m0, int n0, int wm, int wn, int li, int lk,
                                  float sig, const floatx16& acc1, const floatx16& acc2, const floatx16& acc3) {
  float* out;
  int ldo;
  bool acc_in;
  if (p.partial) {
    out = p.C + (size_t)split * p.M * 2 * p.N;
    ldo = 2 * p.N;
    acc_in = false;
  } else {
    out = p.C;
    ldo = p.ldc;
    acc_in = p.accumulate != 0;
  }
  const int j = n0 + wn * 32 + li;
  if (j < p.N) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = m0 + wm * 32 + 8 * (r / 4) + 4 * lk + (r % 4);
      if (i < p.M) {
        const float t2 = sig * acc2[r];
        const float re = acc1[r] - t2, im = acc3[r] - acc1[r] - t2;
        float* d0 = out + (size_t)i * ldo + j;
        float* d1 = d0 + p.N;
        *d0 = acc_in ? *d0 + re : re;
        *d1 = acc_in ? *d1 + im : im;
      }
    }
  }
}

template <bool TA, bool TB>
__global__ __launch_bounds__(CNT) __attribute__((amdgpu_waves_per_eu(4, 8))) void gemm_cplx_kernel(GemmBatch batch) {
  constexpr bool AK = !TA, BKC = TB;
  __shared__ __attribute__((aligned(16))) float Aa[2][CT<AK, CBM>::FL], Ab[2][CT<AK, CBM>::FL];
  __shared__ __attribute__((aligned(16))) float Bc[2][CT<BKC, CBN>::FL], Bd[2][CT<BKC, CBN>::FL];
  int pi, local;
  decode_tile(batch, xcd_remap(blockIdx.x, batch.total_tiles), &pi, &local);
  const GemmProb& p = batch.p[pi];
  const int per_split = p.tiles_m * p.tiles_n;
  const int split = local / per_split;
  local -= split * per_split;
  const int tm = local / p.tiles_n, tn = local - tm * p.tiles_n;
  const int m0 = tm * CBM, n0 = tn * CBN;
  const int kbeg = split * p.k_chunk, kend = min(p.K, kbeg + p.k_chunk);
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int wm = wave / 2, wn = wave % 2, li = lane % 32, lk = lane / 32;
  floatx16 acc1, acc2, acc3;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc1[r] = acc2[r] = acc3[r] = 0.f;
  const float* A0 = static_cast<const float*>(p.A);
  const float* A1 = A0 + p.dA;
  const float* B0 = static_cast<const float*>(p.B);
  const float* B1 = B0 + p.dB;
  const float sA = p.sA, sB = p.sB;
  const int nk = (kend - kbeg + CBK - 1) / CBK;
  floatx4 ra0[CT<AK, CBM>::NL], ra1[CT<AK, CBM>::NL], rb0[CT<BKC, CBN>::NL], rb1[CT<BKC, CBN>::NL];
  auto load = [&](int k0) {
    cload<AK, CBM>(A0, p.lda, m0, p.M, k0, kend, ra0);
    cload<AK, CBM>(A1, p.lda, m0, p.M, k0, kend, ra1);
    cload<BKC, CBN>(B0, p.ldb, n0, p.N, k0, kend, rb0);
    cload<BKC, CBN>(B1, p.ldb, n0, p.N, k0, kend, rb1);
  };
  auto store = [&](int b) {
    cstore<AK, CBM>(Aa[b], ra0);
    cstore<AK, CBM>(Ab[b], ra1);
    cstore<BKC, CBN>(Bc[b], rb0);
    cstore<BKC, CBN>(Bd[b], rb1);
  };
  if (nk > 0) {
    load(kbeg);
    store(0);
  }
  __syncthreads();
  const int ar = wm * 32 + li, br = wn * 32 + li;
#pragma unroll 1
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load(kbeg + (kt + 1) * CBK);
    float fa[CBK / 2], fb[CBK / 2], fc[CBK / 2], fd[CBK / 2];
    cfrag<AK, CBM>(Aa[cur], ar, lk, fa);
    cfrag<AK, CBM>(Ab[cur], ar, lk, fb);
    cfrag<BKC, CBN>(Bc[cur], br, lk, fc);
    cfrag<BKC, CBN>(Bd[cur], br, lk, fd);
#pragma unroll
    for (int s = 0; s < CBK / 2; ++s) {
      const float fs = fa[s] + sA * fb[s], fw = fc[s] + sB * fd[s];
      acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[s], fc[s], acc1, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_32x32x2f32(fb[s], fd[s], acc2, 0, 0, 0);
      acc3 = __builtin_amdgcn_mfma_f32_32x32x2f32(fs, fw, acc3, 0, 0, 0);
    }
    if (kt + 1 < nk) store(cur ^ 1);
    __syncthreads();
  }
  cplx_store(p, split, m0, n0, wm, wn, li, lk, sA * sB, acc1, acc2, acc3);
}

constexpr int kF32WNW = 2;   // float32 blocks: 256 x 64 kF32WNW
constexpr int kCxWNW = 2;    // complex blocks: 128 x 32 kCxWNW complex

// WNW waves along N (64 columns each), WAVES_M along M
template <bool TA, bool TB, int WNW>
__global__ __launch_bounds__(64 * WAVES_M * WNW) __attribute__((amdgpu_waves_per_eu(WAVES_PER_SIMD, 8))) void
gemm_f32_dma_kernel(GemmBatch batch) {
  constexpr bool AK = !TA, BKC = TB;
  constexpr int BNW = 64 * WNW, NWV = WAVES_M * WNW;
  using DA = DT<AK, BM>;
  using DB = DT<BKC, BNW>;
  constexpr int SL = (DA::NB + DB::NB) / NWV;
  static_assert(SL * NWV == DA::NB + DB::NB, "equal loads per wave and stage");
  constexpr int STG = DA::FL + DB::FL;
  __shared__ __attribute__((aligned(16))) float S[DNS * STG];
  int pi, local;
  decode_tile(batch, xcd_remap(blockIdx.x, batch.total_tiles), &pi, &local);
  const GemmProb& p = batch.p[pi];
  const int per_split = p.tiles_m * p.tiles_n;
  const int split = local / per_split;
  local -= split * per_split;
  const int tm = local / p.tiles_n, tn = local - tm * p.tiles_n;
  const int m0 = tm * BM, n0 = tn * BNW;
  const int kbeg = split * p.k_chunk, kend = min(p.K, kbeg + p.k_chunk);
  const int nkk = kend - kbeg, nk = (nkk + 15) / 16;
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int wm = wave / WNW, wn = wave % WNW, li = lane % 32, lk = lane / 32;
  DSlot sl[SL];
#pragma unroll
  for (int j = 0; j < SL; ++j) {
    const int g = SL * wave + j;
    sl[j] = g < DA::NB ? dslot<AK, BM>(g, static_cast<const float*>(p.A), p.lda, m0, p.M, kbeg, lane, 0)
                       : dslot<BKC, BNW>(g - DA::NB, static_cast<const float*>(p.B), p.ldb, n0, p.N, kbeg, lane, DA::FL);
  }
  floatx16 acc[WM][WN];
#pragma unroll
  for (int a = 0; a < WM; ++a)
#pragma unroll
    for (int b = 0; b < WN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
  if (nk > 0) dstage(sl, S, 0, nkk, lane);
  if (nk > 1) dstage(sl, S + STG, 1, nkk, lane);
  const int ra0 = wm * 32 * WM + li, rb0 = wn * 32 * WN + li;
  int cur = 0;
#pragma unroll 1
  for (int kt = 0; kt < nk; ++kt) {
    dsync<SL>(kt + 1 < nk);
    if (kt + 2 < nk) dstage(sl, S + (cur == 0 ? 2 : cur - 1) * STG, kt + 2, nkk, lane);
    const float* st = S + cur * STG;
    // the compiler's MFMA-loop schedule (interleaves the fragment reads with
    // the products): +4-7% on A.B^T, 0-2% elsewhere, same results
    __builtin_amdgcn_iglp_opt(1);
    float av[WM][8], bv[WN][8];
#pragma unroll
    for (int a = 0; a < WM; ++a) dfrag<AK, BM>(st, ra0 + 32 * a, lk, av[a]);
#pragma unroll
    for (int b = 0; b < WN; ++b) dfrag<BKC, BNW>(st + DA::FL, rb0 + 32 * b, lk, bv[b]);
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int a = 0; a < WM; ++a)
#pragma unroll
        for (int b = 0; b < WN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[a][s], bv[b][s], acc[a][b], 0, 0, 0);
    cur = cur == 2 ? 0 : cur + 1;
  }
  store_acc(p, split, m0, n0, wm, wn, li, lk, acc);
}

// WNW waves along N (32 complex columns each), 4 along M
template <bool TA, bool TB, int WNW>
__global__ __launch_bounds__(256 * WNW) __attribute__((amdgpu_waves_per_eu(4, 8))) void gemm_cplx_dma_kernel(
    GemmBatch batch) {
  constexpr bool AK = !TA, BKC = TB;
  constexpr int BNW = 32 * WNW, NWV = 4 * WNW;
  using DA = DT<AK, CBM>;
  using DB = DT<BKC, BNW>;
  constexpr int SL = (2 * DA::NB + 2 * DB::NB) / NWV;
  static_assert(SL * NWV == 2 * DA::NB + 2 * DB::NB, "equal loads per wave and stage");
  constexpr int STG = 2 * DA::FL + 2 * DB::FL;
  __shared__ __attribute__((aligned(16))) float S[DNS * STG];
  int pi, local;
  decode_tile(batch, xcd_remap(blockIdx.x, batch.total_tiles), &pi, &local);
  const GemmProb& p = batch.p[pi];
  const int per_split = p.tiles_m * p.tiles_n;
  const int split = local / per_split;
  local -= split * per_split;
  const int tm = local / p.tiles_n, tn = local - tm * p.tiles_n;
  const int m0 = tm * CBM, n0 = tn * BNW;
  const int kbeg = split * p.k_chunk, kend = min(p.K, kbeg + p.k_chunk);
  const int nkk = kend - kbeg, nk = (nkk + 15) / 16;
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int wm = wave / WNW, wn = wave % WNW, li = lane % 32, lk = lane / 32;
  const float* A0 = static_cast<const float*>(p.A);
  const float* B0 = static_cast<const float*>(p.B);
  DSlot sl[SL];
#pragma unroll
  for (int j = 0; j < SL; ++j) {
    const int g = SL * wave + j;
    if (g < 2 * DA::NB) {
      const int part = g / DA::NB;
      sl[j] = dslot<AK, CBM>(g - part * DA::NB, A0 + (part ? p.dA : 0), p.lda, m0, p.M, kbeg, lane, part * DA::FL);
    } else {
      const int h = g - 2 * DA::NB, part = h / DB::NB;
      sl[j] = dslot<BKC, BNW>(h - part * DB::NB, B0 + (part ? p.dB : 0), p.ldb, n0, p.N, kbeg, lane,
                              2 * DA::FL + part * DB::FL);
    }
  }
  floatx16 acc1, acc2, acc3;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc1[r] = acc2[r] = acc3[r] = 0.f;
  const float sA = p.sA, sB = p.sB;
  if (nk > 0) dstage(sl, S, 0, nkk, lane);
  if (nk > 1) dstage(sl, S + STG, 1, nkk, lane);
  const int ar = wm * 32 + li, br = wn * 32 + li;
  int cur = 0;
#pragma unroll 1
  for (int kt = 0; kt < nk; ++kt) {
    dsync<SL>(kt + 1 < nk);
    if (kt + 2 < nk) dstage(sl, S + (cur == 0 ? 2 : cur - 1) * STG, kt + 2, nkk, lane);
    const float* st = S + cur * STG;
    __builtin_amdgcn_iglp_opt(1);   // as in the float32 kernel: 0.3-2% here
    float fa[8], fb[8], fc[8], fd[8];
    dfrag<AK, CBM>(st, ar, lk, fa);
    dfrag<AK, CBM>(st + DA::FL, ar, lk, fb);
    dfrag<BKC, BNW>(st + 2 * DA::FL, br, lk, fc);
    dfrag<BKC, BNW>(st + 2 * DA::FL + DB::FL, br, lk, fd);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const float fs = fa[s] + sA * fb[s], fw = fc[s] + sB * fd[s];
      acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[s], fc[s], acc1, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_32x32x2f32(fb[s], fd[s], acc2, 0, 0, 0);
      acc3 = __builtin_amdgcn_mfma_f32_32x32x2f32(fs, fw, acc3, 0, 0, 0);
    }
    cur = cur == 2 ? 0 : cur + 1;
  }
  cplx_store(p, split, m0, n0, wm, wn, li, lk, sA * sB, acc1, acc2, acc3);
}

// ---------------------------------------------------------------- bfloat16 operands
// Block tile 256x256 of 16 waves (64x64 each, 2x2 v_mfma_f32_32x32x16_bf16),
// K tile 64, one block per CU (147 KB of LDS for two stages). Measured on
// MI355X for the per-order shapes (725k rows): 256x128 blocks with K tile 32
// reached 425-700 TFLOP/s for A.B^T and 375-515 for A^T.B; this tiling
// 495-805 and 453-652 (the longer K tile gives the next tile's loads more MFMA
// time to land behind).
//
// LDS tiles hold every operand k-contiguous: row r of a tile is BKH bf16 (16-byte
// chunks of 8 k values) at a pitch of BKH/2 + 4 dwords, and the chunks of rows
// 8..15 of every 16 rows are swapped pairwise. An MFMA operand read is one
// 16-byte chunk per lane (row lane%32, chunk 2*ks + lane/32); with the pitch,
// any 8 consecutive rows of one chunk fall on disjoint banks, and the swap
// keeps the transposing stores of k-major operands (below) off each other's
// banks.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int BMH = 256, BNH = 256;          // block tile
constexpr int NWH = (BMH / 64) * (BNH / 64);  // waves (64x64 wave tiles)
constexpr int NTH = 64 * NWH;                 // threads
constexpr int BKH = 64;                       // K tile
constexpr int PD = BKH / 2 + 4;               // LDS row pitch (dwords)
constexpr int CPR = BKH / 8;                  // 16-byte chunks per row
static_assert(kGemmKTile % BKH == 0 && kGemmKTile % BK_TILE == 0 && kGemmKTile % CBK == 0,
              "split chunks must be whole K tiles");

__device__ __forceinline__ int lds_chunk(int row, int q) { return row * PD + 4 * (q ^ ((row >> 3) & 1)); }

template <int R>
struct CfgH {
  static constexpr int NKC = (R * CPR + NTH - 1) / NTH;        // 16-byte chunks per thread, k-contiguous operand
  static constexpr int UNITS = R * BKH / 16;                   // 8k x 2row units of a k-major operand
  static constexpr int NKM = (UNITS + NTH - 1) / NTH;
};

// k-contiguous operand (global [row][k]): one 16-byte chunk per load
template <int R>
__device__ inline void ldh_kc(const unsigned short* __restrict__ P, int ld, int r0, int rlim, int k0, int kend,
                              u32x4 (&v)[CfgH<R>::NKC]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int p = 0; p < CfgH<R>::NKC; ++p) {
    const int idx = p * NTH + t, row = idx / CPR, q = idx % CPR;
    const int gr = r0 + row, gk = k0 + 8 * q;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (idx < R * CPR && gr < rlim && gk < kend) {
      const unsigned short* src = P + (size_t)gr * ld + gk;
      if (gk + 8 <= kend) {
        x = *reinterpret_cast<const u32x4*>(src);
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c)
          if (gk + c < kend) x[c / 2] |= (unsigned)src[c] << (16 * (c % 2));
      }
    }
    v[p] = x;
  }
}

template <int R>
__device__ inline void sth_kc(unsigned* S, const u32x4 (&v)[CfgH<R>::NKC]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int p = 0; p < CfgH<R>::NKC; ++p) {
    const int idx = p * NTH + t;
    if (idx < R * CPR) *reinterpret_cast<u32x4*>(S + lds_chunk(idx / CPR, idx % CPR)) = v[p];
  }
}

// k-major operand (global [k][row]): unit u = (rows 2c, 2c+1) x (k 8g .. 8g+7),
// c = u % (R/2), g = u / (R/2): eight 4-byte loads (consecutive lanes on
// consecutive row pairs), transposed in registers into one 16-byte chunk per row.
template <int R>
__device__ inline void ldh_km(const unsigned short* __restrict__ P, int ld, int r0, int rlim, int k0, int kend,
                              unsigned (&w)[CfgH<R>::NKM][8]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int p = 0; p < CfgH<R>::NKM; ++p) {
    const int u = p * NTH + t;
    const int c = u % (R / 2), g = u / (R / 2);
    const int gr = r0 + 2 * c;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      unsigned x = 0u;
      const int gk = k0 + 8 * g + j;
      if (u < CfgH<R>::UNITS && gk < kend) {
        const unsigned short* src = P + (size_t)gk * ld + gr;
        if (gr + 1 < rlim) x = *reinterpret_cast<const unsigned*>(src);
        else if (gr < rlim) x = src[0];
      }
      w[p][j] = x;
    }
  }
}

template <int R>
__device__ inline void sth_km(unsigned* S, const unsigned (&w)[CfgH<R>::NKM][8]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int p = 0; p < CfgH<R>::NKM; ++p) {
    const int u = p * NTH + t;
    if (u >= CfgH<R>::UNITS) continue;
    const int c = u % (R / 2), g = u / (R / 2);
    u32x4 lo, hi;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo[i] = (w[p][2 * i] & 0xffffu) | (w[p][2 * i + 1] << 16);
      hi[i] = (w[p][2 * i] >> 16) | (w[p][2 * i + 1] & 0xffff0000u);
    }
    *reinterpret_cast<u32x4*>(S + lds_chunk(2 * c, g)) = lo;
    *reinterpret_cast<u32x4*>(S + lds_chunk(2 * c + 1, g)) = hi;
  }
}

// TA = false: C = A.B^T (both operands k-contiguous); TA = true: C = A^T.B
// (both k-major)
template <bool TA>
__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(4, 8))) void gemm_bf16_kernel(GemmBatch batch) {
  constexpr int NWN = BNH / 64;
  __shared__ unsigned As[2][BMH * PD];
  __shared__ unsigned Bs[2][BNH * PD];

  int pi, local;
  decode_tile(batch, xcd_remap(blockIdx.x, batch.total_tiles), &pi, &local);
  const GemmProb& p = batch.p[pi];
  const int per_split = p.tiles_m * p.tiles_n;
  const int split = local / per_split;
  local -= split * per_split;
  const int tm = local / p.tiles_n, tn = local - tm * p.tiles_n;
  const int m0 = tm * BMH, n0 = tn * BNH;
  const int kbeg = split * p.k_chunk;
  const int kend = min(p.K, kbeg + p.k_chunk);
  const unsigned short* A = static_cast<const unsigned short*>(p.A);
  const unsigned short* B = static_cast<const unsigned short*>(p.B);

  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int wm = wave / NWN, wn = wave % NWN;
  const int li = lane % 32, lk = lane / 32;

  floatx16 acc[WM][WN];
#pragma unroll
  for (int a = 0; a < WM; ++a)
#pragma unroll
    for (int b = 0; b < WN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int nk = (kend - kbeg + BKH - 1) / BKH;
  u32x4 ra[TA ? 1 : CfgH<BMH>::NKC], rb[TA ? 1 : CfgH<BNH>::NKC];
  unsigned wa[TA ? CfgH<BMH>::NKM : 1][8], wb[TA ? CfgH<BNH>::NKM : 1][8];
  auto load = [&](int k0) {
    if constexpr (TA) {
      ldh_km<BMH>(A, p.lda, m0, p.M, k0, kend, wa);
      ldh_km<BNH>(B, p.ldb, n0, p.N, k0, kend, wb);
    } else {
      ldh_kc<BMH>(A, p.lda, m0, p.M, k0, kend, ra);
      ldh_kc<BNH>(B, p.ldb, n0, p.N, k0, kend, rb);
    }
  };
  auto store = [&](int buf) {
    if constexpr (TA) {
      sth_km<BMH>(As[buf], wa);
      sth_km<BNH>(Bs[buf], wb);
    } else {
      sth_kc<BMH>(As[buf], ra);
      sth_kc<BNH>(Bs[buf], rb);
    }
  };
  if (nk > 0) {
    load(kbeg);
    store(0);
  }
  __syncthreads();
#pragma unroll 1
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load(kbeg + (kt + 1) * BKH);
    const unsigned* as = As[cur];
    const unsigned* bs = Bs[cur];
    __builtin_amdgcn_iglp_opt(1);   // compiler MFMA-loop schedule: 0-3% here, same results
    const int ra0 = wm * 32 * WM + li, rb0 = wn * 32 * WN + li;
#pragma unroll
    for (int ks = 0; ks < BKH / 16; ++ks) {
      const int q = 2 * ks + lk;
      bf16x8 av[WM], bv[WN];
#pragma unroll
      for (int a = 0; a < WM; ++a)
        av[a] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(as + lds_chunk(ra0 + 32 * a, q)));
#pragma unroll
      for (int b = 0; b < WN; ++b)
        bv[b] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(bs + lds_chunk(rb0 + 32 * b, q)));
#pragma unroll
      for (int a = 0; a < WM; ++a)
#pragma unroll
        for (int b = 0; b < WN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
    if (kt + 1 < nk) store(cur ^ 1);
    __syncthreads();
  }
  store_acc(p, split, m0, n0, wm, wn, li, lk, acc);
}

__global__ void gemm_reduce_kernel(const float* __restrict__ P, int splits, int M, int N, float* __restrict__ C,
                                   int ldc, int accumulate, int trans) {
  const size_t n = (size_t)M * N;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (size_t)gridDim.x * blockDim.x) {
    float s = 0.f;
    for (int q = 0; q < splits; ++q) s += P[(size_t)q * n + idx];
    const size_t i = idx / N, j = idx - i * N;
    float* dst = trans ? C + j * ldc + i : C + i * ldc + j;
    *dst = accumulate ? *dst + s : s;
  }
}

// direct-to-LDS kernels: every operand 16-byte aligned, leading dimensions
// (and complex part offsets) multiples of four elements, and the dimension a
// k-major operand's chunks run along a multiple of four
bool dma_ok(const GemmBatch& b, bool TA, bool TB) {
  for (int q = 0; q < b.nprob; ++q) {
    const GemmProb& p = b.p[q];
    if (p.M <= 0 || p.N <= 0) continue;
    if ((reinterpret_cast<uintptr_t>(p.A) | reinterpret_cast<uintptr_t>(p.B)) % 16) return false;
    if (p.lda % 4 || p.ldb % 4) return false;
    if (p.cplx && (p.dA % 4 || p.dB % 4)) return false;
    if ((TA && p.M % 4) || (!TB && p.N % 4)) return false;
  }
  return true;
}

}  // namespace

int gemm_run(GemmBatch& b, bool TA, bool TB, bool bf16, hipStream_t s) {
  constexpr int BK = BK_TILE;
  for (int q = 0; q < b.nprob; ++q)
    if (b.p[q].gate) return hipErrorNotSupported;   // the gated epilogue lives in the split and bf16 A.B^T kernels
  const bool cx = b.nprob > 0 && b.p[0].cplx;
  if (bf16 && TA == TB) return hipErrorInvalidValue;
  if (cx && (bf16 || (TA && TB))) return hipErrorInvalidValue;
  for (int q = 0; q < b.nprob; ++q)
    if ((b.p[q].cplx != 0) != cx) return hipErrorInvalidValue;
  const bool dma = !bf16 && dma_ok(b, TA, TB);
  // real products at most 64 columns wide (the radial map's gradients, with
  // the n_rbf side as columns): blocks of 256 x 64, four waves
  bool narrow = dma && !cx && !(TA && TB);
  for (int q = 0; q < b.nprob && narrow; ++q) narrow = b.p[q].N <= 64;
  const int bm = cx ? CBM : (bf16 ? BMH : BM);
  const int bn = cx ? (dma ? 32 * kCxWNW : CBN) : (bf16 ? BNH : (narrow ? 64 : (dma ? 64 * kF32WNW : BN)));
  int total = 0;
  for (int q = 0; q < b.nprob; ++q) {
    GemmProb& p = b.p[q];
    p.tiles_m = (p.M + bm - 1) / bm;
    p.tiles_n = (p.N + bn - 1) / bn;
    if (p.k_splits < 1) p.k_splits = 1;
    if (p.k_splits == 1 && p.k_chunk <= 0) p.k_chunk = p.K;
    p.tile_begin = total;
    if (p.M > 0 && p.N > 0) total += p.tiles_m * p.tiles_n * p.k_splits;
  }
  b.total_tiles = total;
  if (total == 0) return hipSuccess;
  dim3 grid(total), block(NT);
  if (dma) {
    constexpr int W = kF32WNW, CW = kCxWNW;
    const dim3 fb(64 * WAVES_M * W), cb(256 * CW);
    if (cx) {
      if (!TA && !TB) hipLaunchKernelGGL((gemm_cplx_dma_kernel<false, false, CW>), grid, cb, 0, s, b);
      else if (!TA && TB) hipLaunchKernelGGL((gemm_cplx_dma_kernel<false, true, CW>), grid, cb, 0, s, b);
      else hipLaunchKernelGGL((gemm_cplx_dma_kernel<true, false, CW>), grid, cb, 0, s, b);
    } else if (!TA && !TB && narrow) {
      hipLaunchKernelGGL((gemm_f32_dma_kernel<false, false, 1>), grid, dim3(64 * WAVES_M), 0, s, b);
    } else if (!TA && !TB) {
      hipLaunchKernelGGL((gemm_f32_dma_kernel<false, false, W>), grid, fb, 0, s, b);
    } else if (!TA && TB && narrow) {
      hipLaunchKernelGGL((gemm_f32_dma_kernel<false, true, 1>), grid, dim3(64 * WAVES_M), 0, s, b);
    } else if (!TA && TB) {
      hipLaunchKernelGGL((gemm_f32_dma_kernel<false, true, W>), grid, fb, 0, s, b);
    } else if (TA && !TB && narrow) {
      hipLaunchKernelGGL((gemm_f32_dma_kernel<true, false, 1>), grid, dim3(64 * WAVES_M), 0, s, b);
    } else if (TA && !TB) {
      hipLaunchKernelGGL((gemm_f32_dma_kernel<true, false, W>), grid, fb, 0, s, b);
    } else {
      hipLaunchKernelGGL((gemm_f32_dma_kernel<true, true, W>), grid, fb, 0, s, b);
    }
    return hipGetLastError();
  }
  if (cx) {
    if (!TA && !TB) hipLaunchKernelGGL((gemm_cplx_kernel<false, false>), grid, dim3(CNT), 0, s, b);
    else if (!TA && TB) hipLaunchKernelGGL((gemm_cplx_kernel<false, true>), grid, dim3(CNT), 0, s, b);
    else hipLaunchKernelGGL((gemm_cplx_kernel<true, false>), grid, dim3(CNT), 0, s, b);
    return hipGetLastError();
  }
  if (bf16) {
    if (TA) hipLaunchKernelGGL((gemm_bf16_kernel<true>), grid, dim3(NTH), 0, s, b);
    else hipLaunchKernelGGL((gemm_bf16_kernel<false>), grid, dim3(NTH), 0, s, b);
    return hipGetLastError();
  }
  if (!TA && !TB) hipLaunchKernelGGL((gemm_f32_kernel<false, false, BK>), grid, block, 0, s, b);
  else if (!TA && TB) hipLaunchKernelGGL((gemm_f32_kernel<false, true, BK>), grid, block, 0, s, b);
  else if (TA && !TB) hipLaunchKernelGGL((gemm_f32_kernel<true, false, BK>), grid, block, 0, s, b);
  else hipLaunchKernelGGL((gemm_f32_kernel<true, true, BK>), grid, block, 0, s, b);
  return hipGetLastError();
}

// four adjacent columns per thread with 16-byte loads and stores (same order of
// the split sums per element as gemm_reduce_kernel)
__global__ void gemm_reduce4_kernel(const float* __restrict__ P, int splits, int M, int N, float* __restrict__ C,
                                    int ldc, int accumulate) {
  const size_t n4 = (size_t)M * N / 4;
  const size_t n = (size_t)M * N;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n4; idx += (size_t)gridDim.x * blockDim.x) {
    floatx4 s = {0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < splits; ++q) {
      const floatx4 v = *reinterpret_cast<const floatx4*>(P + (size_t)q * n + 4 * idx);
#pragma unroll
      for (int c = 0; c < 4; ++c) s[c] += v[c];
    }
    const size_t i = 4 * idx / N, j = 4 * idx - i * N;
    floatx4* dst = reinterpret_cast<floatx4*>(C + i * ldc + j);
    if (accumulate) {
      const floatx4 o = *dst;
#pragma unroll
      for (int c = 0; c < 4; ++c) s[c] += o[c];
    }
    *dst = s;
  }
}

int gemm_reduce(const float* P, int splits, int M, int N, float* C, int ldc, int accumulate, hipStream_t s,
                int trans) {
  const size_t n = (size_t)M * N;
  if (n == 0) return hipSuccess;
  if (!trans && N % 4 == 0 && ldc % 4 == 0 &&
      (reinterpret_cast<uintptr_t>(P) | reinterpret_cast<uintptr_t>(C)) % 16 == 0) {
    int blocks = (int)((n / 4 + 255) / 256);
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(gemm_reduce4_kernel, dim3(blocks), dim3(256), 0, s, P, splits, M, N, C, ldc, accumulate);
    return hipGetLastError();
  }
  int blocks = (int)((n + 255) / 256);
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(gemm_reduce_kernel, dim3(blocks), dim3(256), 0, s, P, splits, M, N, C, ldc, accumulate, trans);
  return hipGetLastError();
}

}  // namespace so2
