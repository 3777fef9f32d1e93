// float32 GEMMs on the bfloat16 matrix cores: every float32 operand is the
// exact sum of three bfloat16 pieces, and the products of the pieces run on
// v_mfma_f32_32x32x16_bf16 with float32 accumulation.
//
// Split (truncation, no rounding): for a float32 x with a 24-bit significand,
//   h = x with the low 16 bits cleared,  r = x - h  (exact),
//   m = r with the low 16 bits cleared,  l = r - m  (exact, at most 8 bits),
// so x = h + m + l exactly and each piece is a bfloat16 value (its upper 16
// bits). A product x y is the sum of the nine piece products, each exact in
// float32 (8-bit by 8-bit significands). NP = 9 takes all nine; NP = 6 drops
// m l, l m and l l, whose sum is below 2^-23 |x y| (2^-8 per piece step).
//
// The float32 matrix cores run at 1/16 of the bfloat16 rate on gfx950 (157.3
// vs 2500 TFLOP/s dense), so six or nine bfloat16 products per float32
// product still leave 1.8-2.6x the float32 peak, and one k tile of operands
// feeds 16 NP MFMAs per wave: the kernel is bound by the matrix cores, not by
// operand traffic.
//
// Block tile 256 x 256 of eight waves (128 x 64 each: 4 x 2 tiles of 32 x 32,
// 128 accumulator registers, two waves per SIMD), K tile 16. The operand
// tiles arrive as float32 straight into LDS (global_load_lds_dwordx4, the
// float32 kernels' tile layouts) in a ring of four stages; each wave splits
// the fragments it multiplies (its four A and two B fragments of the tile).
// The two waves of a SIMD overlap one's split arithmetic with the other's
// matrix products.
#include "gemm.hpp"
#include "gemm_dma.hpp"
#include "gemm_tile.hpp"
#include "numeric.hpp"

namespace so2 {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int ZM = 256, ZN = 256;   // block tile
constexpr int ZST = 4;              // stages
constexpr int ZNT = 512;            // threads (eight waves: 2 along M, 4 along N)

// the three pieces of the eight float32 values of one operand fragment
struct Pieces {
  bf16x8 h, m, l;
};
__device__ __forceinline__ unsigned hi16(float x) { return __float_as_uint(x) & 0xffff0000u; }
__device__ __forceinline__ Pieces split8(const float (&f)[8]) {
  unsigned ph[4], pm[4], pl[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float x0 = f[2 * q], x1 = f[2 * q + 1];
    const float r0 = x0 - __uint_as_float(hi16(x0)), r1 = x1 - __uint_as_float(hi16(x1));
    const float s0 = r0 - __uint_as_float(hi16(r0)), s1 = r1 - __uint_as_float(hi16(r1));
    // upper halves of (x0, x1) -> one dword, element 2q in the low half
    ph[q] = __builtin_amdgcn_perm(__float_as_uint(x1), __float_as_uint(x0), 0x07060302u);
    pm[q] = __builtin_amdgcn_perm(__float_as_uint(r1), __float_as_uint(r0), 0x07060302u);
    pl[q] = __builtin_amdgcn_perm(__float_as_uint(s1), __float_as_uint(s0), 0x07060302u);
  }
  Pieces p;
  p.h = __builtin_bit_cast(bf16x8, u32x4{ph[0], ph[1], ph[2], ph[3]});
  p.m = __builtin_bit_cast(bf16x8, u32x4{pm[0], pm[1], pm[2], pm[3]});
  p.l = __builtin_bit_cast(bf16x8, u32x4{pl[0], pl[1], pl[2], pl[3]});
  return p;
}

__device__ __forceinline__ floatx16 mfma(const bf16x8& a, const bf16x8& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// the NP piece products of one row of 32 x 32 tiles (a with each b), smallest
// pieces first; consecutive MFMAs go to different accumulators
template <int NP>
__device__ __forceinline__ void row_products(const Pieces& a, const Pieces (&b)[2], floatx16 (&acc)[2]) {
  if constexpr (NP == 9) {
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[j] = mfma(a.l, b[j].l, acc[j]);
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[j] = mfma(a.m, b[j].l, acc[j]);
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[j] = mfma(a.l, b[j].m, acc[j]);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) acc[j] = mfma(a.h, b[j].l, acc[j]);
#pragma unroll
  for (int j = 0; j < 2; ++j) acc[j] = mfma(a.m, b[j].m, acc[j]);
#pragma unroll
  for (int j = 0; j < 2; ++j) acc[j] = mfma(a.l, b[j].h, acc[j]);
#pragma unroll
  for (int j = 0; j < 2; ++j) acc[j] = mfma(a.h, b[j].m, acc[j]);
#pragma unroll
  for (int j = 0; j < 2; ++j) acc[j] = mfma(a.m, b[j].h, acc[j]);
#pragma unroll
  for (int j = 0; j < 2; ++j) acc[j] = mfma(a.h, b[j].h, acc[j]);
}

__device__ __forceinline__ float zsig(float v) { return 1.f / (1.f + __expf(-v)); }

// Gated epilogue of the first linear (GemmProb::gate): C = u as usual and
// Z = SiLU(u) (degree 0) or sigmoid(gamma) u, gamma the row's gate column of
// the element's degree and channel. Lane (li, lk) of MFMA tile (a, b) holds
// column 32 b + li and rows 32 a + 8 g + 4 lk + i of the wave's 128 x 64 tile.
template <typename ZT>
__device__ __forceinline__ void gated_store(const GemmBatch& batch, const GemmProb& p, const floatx16 (&acc)[4][2],
                                            int i0, int j0) {
  const int C = batch.gC, ga = p.gate - 1, hwid = (batch.gL - ga + 1) * C;
  ZT* Zo = static_cast<ZT*>(p.Z);
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int j = j0 + 32 * b;
    if (j >= p.N) continue;
    const int l = ga + (j % hwid) / C, c = j % C;
    const float* g = p.gam + (l > 0 ? (l - 1) * C + c : 0);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = i0 + 32 * a + 8 * (r / 4) + (r % 4);
        if (i < p.M) {
          const float u = acc[a][b][r];
          p.C[(size_t)i * p.ldc + j] = u;
          const float z = l == 0 ? u * zsig(u) : zsig(g[(size_t)i * batch.ldgam]) * u;
          st(Zo + (size_t)i * batch.ldz + j, z);
        }
      }
  }
}

// wait until this wave's loads of the tile to be read have landed (`ahead`
// later tiles may still be in flight, four loads each) and publish it to the
// block; the wait on lgkmcnt also retires this wave's fragment reads
__device__ __forceinline__ void zsync(int ahead) {
  if (ahead >= 2) asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)" ::: "memory");
  else if (ahead == 1) asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// C = op(A) op(B) with float32 operands (op as in GemmProb), NP piece products
template <bool TA, bool TB, int NP>
__global__ __launch_bounds__(ZNT) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_x3_kernel(
    GemmBatch batch) {
  constexpr bool AK = !TA, BKC = TB;
  using DA = DT<AK, ZM>;
  using DB = DT<BKC, ZN>;
  constexpr int SL = (DA::NB + DB::NB) / (ZNT / 64);
  static_assert(SL == 4, "four loads per wave and stage");
  constexpr int STG = DA::FL + DB::FL;
  __shared__ __attribute__((aligned(16))) float S[ZST * STG];
  int pi, local;
  decode_tile(batch, xcd_remap(blockIdx.x, batch.total_tiles), &pi, &local);
  const GemmProb& p = batch.p[pi];
  const int per_split = p.tiles_m * p.tiles_n;
  const int split = local / per_split;
  local -= split * per_split;
  const int tm = local / p.tiles_n, tn = local - tm * p.tiles_n;
  const int m0 = tm * ZM, n0 = tn * ZN;
  const int kbeg = split * p.k_chunk, kend = min(p.K, kbeg + p.k_chunk);
  const int nkk = kend - kbeg, nk = (nkk + 15) / 16;
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int wm = wave >> 2, wn = wave & 3, li = lane % 32, lk = lane / 32;
  DSlot sl[SL];
#pragma unroll
  for (int j = 0; j < SL; ++j) {
    const int g = SL * wave + j;
    sl[j] = g < DA::NB ? dslot<AK, ZM>(g, static_cast<const float*>(p.A), p.lda, m0, p.M, kbeg, lane, 0)
                       : dslot<BKC, ZN>(g - DA::NB, static_cast<const float*>(p.B), p.ldb, n0, p.N, kbeg, lane,
                                        DA::FL);
  }
  floatx16 acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

#pragma unroll
  for (int t = 0; t < ZST - 1; ++t)
    if (t < nk) dstage(sl, S + t * STG, t, nkk, lane);
  const int ra = wm * 128 + li, rb = wn * 64 + li;
#pragma unroll 1
  for (int kt = 0; kt < nk; ++kt) {
    zsync(min(ZST - 2, nk - 1 - kt));
    if (kt + ZST - 1 < nk) dstage(sl, S + ((kt + ZST - 1) % ZST) * STG, kt + ZST - 1, nkk, lane);
    const float* st = S + (kt % ZST) * STG;
    Pieces pb[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float f[8];
      dfrag<BKC, ZN>(st + DA::FL, rb + 32 * b, lk, f);
      pb[b] = split8(f);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      float f[8];
      dfrag<AK, ZM>(st, ra + 32 * a, lk, f);
      const Pieces pa = split8(f);
      row_products<NP>(pa, pb, acc[a]);
    }
  }

  // epilogue: lane (li, lk) of MFMA tile (a, b) holds column 32 b + li, rows
  // 32 a + 8 g + 4 lk + i (g, i < 4) of the wave's 128 x 64 tile
  const int i0 = m0 + wm * 128 + 4 * lk, j0 = n0 + wn * 64 + li;
  if (p.gate) {
    gated_store<float>(batch, p, acc, i0, j0);
    return;
  }
  if (p.partial || !p.accumulate) {
    float* out = p.partial ? p.C + (size_t)split * p.M * p.N : p.C;
    const int ldo = p.partial ? p.N : p.ldc;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int j = j0 + 32 * b;
        if (j >= p.N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = i0 + 32 * a + 8 * (r / 4) + (r % 4);
          if (i < p.M) out[(size_t)i * ldo + j] = acc[a][b][r];
        }
      }
  } else {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int j = j0 + 32 * b;
        if (j >= p.N) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = i0 + 32 * a + 8 * (r / 4) + (r % 4);
          if (i < p.M) p.C[(size_t)i * p.ldc + j] += acc[a][b][r];
        }
      }
  }
}

// A.B^T with bfloat16 operands, both k-contiguous (the forward products with
// the transposed weight copy, the data-gradient products), on the same block
// structure: 256 x 256 blocks of eight 128 x 64 waves at two per SIMD, a
// four-stage ring of direct-to-LDS tiles. A tile holds 32 k per row as 16
// dwords (two bfloat16 each), in the float32 kernels' k-contiguous layout; a
// lane half's eight dwords of a fragment read are its k values of two MFMA
// steps (4 dwords = 8 k each). A and B fragments take the same dwords, so
// every k of the tile meets its partner exactly once, whichever lanes carry
// it.
__global__ __launch_bounds__(ZNT) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_b16_kernel(GemmBatch batch) {
  using DA = DT<true, ZM>;
  using DB = DT<true, ZN>;
  constexpr int SL = (DA::NB + DB::NB) / (ZNT / 64);
  static_assert(SL == 4, "four loads per wave and stage");
  constexpr int STG = DA::FL + DB::FL;
  __shared__ __attribute__((aligned(16))) float S[ZST * STG];
  int pi, local;
  decode_tile(batch, xcd_remap(blockIdx.x, batch.total_tiles), &pi, &local);
  const GemmProb& p = batch.p[pi];
  const int per_split = p.tiles_m * p.tiles_n;
  const int split = local / per_split;
  local -= split * per_split;
  const int tm = local / p.tiles_n, tn = local - tm * p.tiles_n;
  const int m0 = tm * ZM, n0 = tn * ZN;
  // k in dwords (pairs of bfloat16); K and the split chunks are even
  const int kbeg = split * p.k_chunk / 2, kend = min(p.K, split * p.k_chunk + p.k_chunk) / 2;
  const int nkk = kend - kbeg, nk = (nkk + 15) / 16;
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int wm = wave >> 2, wn = wave & 3, li = lane % 32, lk = lane / 32;
  DSlot sl[SL];
#pragma unroll
  for (int j = 0; j < SL; ++j) {
    const int g = SL * wave + j;
    sl[j] = g < DA::NB ? dslot<true, ZM>(g, static_cast<const float*>(p.A), p.lda / 2, m0, p.M, kbeg, lane, 0)
                       : dslot<true, ZN>(g - DA::NB, static_cast<const float*>(p.B), p.ldb / 2, n0, p.N, kbeg, lane,
                                         DA::FL);
  }
  floatx16 acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

#pragma unroll
  for (int t = 0; t < ZST - 1; ++t)
    if (t < nk) dstage(sl, S + t * STG, t, nkk, lane);
  const int ra = wm * 128 + li, rb = wn * 64 + li;
#pragma unroll 1
  for (int kt = 0; kt < nk; ++kt) {
    zsync(min(ZST - 2, nk - 1 - kt));
    if (kt + ZST - 1 < nk) dstage(sl, S + ((kt + ZST - 1) % ZST) * STG, kt + ZST - 1, nkk, lane);
    const float* st = S + (kt % ZST) * STG;
    bf16x8 fb[2][2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float f[8];
      dfrag<true, ZN>(st + DA::FL, rb + 32 * b, lk, f);
      fb[b][0] = __builtin_bit_cast(bf16x8, u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]),
                                                  __float_as_uint(f[2]), __float_as_uint(f[3])});
      fb[b][1] = __builtin_bit_cast(bf16x8, u32x4{__float_as_uint(f[4]), __float_as_uint(f[5]),
                                                  __float_as_uint(f[6]), __float_as_uint(f[7])});
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      float f[8];
      dfrag<true, ZM>(st, ra + 32 * a, lk, f);
      const bf16x8 a0 = __builtin_bit_cast(bf16x8, u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]),
                                                         __float_as_uint(f[2]), __float_as_uint(f[3])});
      const bf16x8 a1 = __builtin_bit_cast(bf16x8, u32x4{__float_as_uint(f[4]), __float_as_uint(f[5]),
                                                         __float_as_uint(f[6]), __float_as_uint(f[7])});
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[a][b] = mfma(a0, fb[b][0], acc[a][b]);
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[a][b] = mfma(a1, fb[b][1], acc[a][b]);
    }
  }
  const int i0 = m0 + wm * 128 + 4 * lk, j0 = n0 + wn * 64 + li;
  if (p.gate) {
    gated_store<bf16s>(batch, p, acc, i0, j0);
    return;
  }
  float* out = p.partial ? p.C + (size_t)split * p.M * p.N : p.C;
  const int ldo = p.partial ? p.N : p.ldc;
  const bool add = p.accumulate && !p.partial;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int j = j0 + 32 * b;
      if (j >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = i0 + 32 * a + 8 * (r / 4) + (r % 4);
        if (i < p.M) {
          float* o = out + (size_t)i * ldo + j;
          *o = add ? *o + acc[a][b][r] : acc[a][b][r];
        }
      }
    }
}

// A^T.B with bfloat16 operands, both k-major (the weight gradients: A [K][M],
// B [K][N], K = edges), on 256 x 256 blocks of eight 128 x 64 waves. A k tile
// of 64 arrives through registers: each thread loads an 8 (k) x 8 (columns)
// block of one operand as eight 16-byte rows, transposes it with byte
// permutes (one per output dword) and writes eight 16-byte k-runs, one per
// column, into a k-contiguous LDS tile (128 bytes per column, 16-byte units
// swizzled by (row ^ row / 8) mod 8 so that a fragment read and the 16
// lanes of a quarter-wave fall on distinct bank groups). Two stages: the
// next tile's loads are in flight while the current one is multiplied.
constexpr int TK = 64;   // k per tile
__device__ __forceinline__ int t_unit(int row, int u) { return row * 8 + (u ^ ((row ^ (row >> 3)) & 7)); }

__global__ __launch_bounds__(ZNT) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_b16t_kernel(GemmBatch batch) {
  __shared__ __attribute__((aligned(16))) u32x4 T[2][512 * 8];   // [stage][row (A 0..255, B 256..511)][unit]
  int pi, local;
  decode_tile(batch, xcd_remap(blockIdx.x, batch.total_tiles), &pi, &local);
  const GemmProb& p = batch.p[pi];
  const int per_split = p.tiles_m * p.tiles_n;
  const int split = local / per_split;
  local -= split * per_split;
  const int tm = local / p.tiles_n, tn = local - tm * p.tiles_n;
  const int m0 = tm * ZM, n0 = tn * ZN;
  const int kbeg = split * p.k_chunk, kend = min(p.K, kbeg + p.k_chunk);
  const int nk = (kend - kbeg + TK - 1) / TK;
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int wm = wave >> 2, wn = wave & 3, li = lane % 32, lk = lane / 32;
  // staging role: operand, k block (8 k) and column block (8 columns)
  const int op = threadIdx.x >> 8, idx = threadIdx.x & 255, kb = idx >> 5, cb = idx & 31;
  const unsigned short* src = static_cast<const unsigned short*>(op ? p.B : p.A);
  const int ld = op ? p.ldb : p.lda, lim = op ? p.N : p.M;
  const int col = (op ? n0 : m0) + 8 * cb;
  const bool colok = col < lim;   // widths are multiples of eight: a column block is all in or all out
  floatx16 acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
  u32x4 rg[8];
  auto load = [&](int t) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int k = kbeg + t * TK + kb * 8 + kk;
      rg[kk] = (colok && k < kend) ? *reinterpret_cast<const u32x4*>(src + (size_t)k * ld + col) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store = [&](int stg) {
#pragma unroll
    for (int mm = 0; mm < 8; ++mm) {
      const unsigned sel = (mm & 1) ? 0x07060302u : 0x05040100u;
      u32x4 o;
#pragma unroll
      for (int kp = 0; kp < 4; ++kp) o[kp] = __builtin_amdgcn_perm(rg[2 * kp + 1][mm >> 1], rg[2 * kp][mm >> 1], sel);
      T[stg][t_unit(256 * op + 8 * cb + mm, kb)] = o;
    }
  };
  if (nk > 0) {
    load(0);
    store(0);
  }
  __syncthreads();
  const int ra = wm * 128 + li, rb = 256 + wn * 64 + li;
#pragma unroll 1
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load(kt + 1);
    const u32x4* st = T[kt & 1];
#pragma unroll
    for (int sq = 0; sq < TK / 16; ++sq) {
      const int u = 2 * sq + lk;
      bf16x8 fb[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) fb[b] = __builtin_bit_cast(bf16x8, st[t_unit(rb + 32 * b, u)]);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const bf16x8 fa = __builtin_bit_cast(bf16x8, st[t_unit(ra + 32 * a, u)]);
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = mfma(fa, fb[b], acc[a][b]);
      }
    }
    if (kt + 1 < nk) store((kt + 1) & 1);
    __syncthreads();
  }
  const int i0 = m0 + wm * 128 + 4 * lk, j0 = n0 + wn * 64 + li;
  float* out = p.partial ? p.C + (size_t)split * p.M * p.N : p.C;
  const int ldo = p.partial ? p.N : p.ldc;
  const bool add = p.accumulate && !p.partial;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int j = j0 + 32 * b;
      if (j >= p.N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = i0 + 32 * a + 8 * (r / 4) + (r % 4);
        if (i < p.M) {
          float* o = out + (size_t)i * ldo + j;
          *o = add ? *o + acc[a][b][r] : acc[a][b][r];
        }
      }
    }
}

// bfloat16 k-major operands of the A^T.B kernel: 16-byte aligned rows and
// column blocks (leading dimensions, M and N multiples of eight), split
// chunks multiples of the k tile
bool b16t_ok(const GemmBatch& b) {
  for (int q = 0; q < b.nprob; ++q) {
    const GemmProb& p = b.p[q];
    if (p.M <= 0 || p.N <= 0) continue;
    if (p.cplx || p.gate) return false;
    if ((reinterpret_cast<uintptr_t>(p.A) | reinterpret_cast<uintptr_t>(p.B)) % 16) return false;
    if (p.lda % 8 || p.ldb % 8 || p.M % 8 || p.N % 8) return false;
    if (p.k_splits > 1 && p.k_chunk % TK) return false;
  }
  return true;
}

// bfloat16 operands of the direct-to-LDS A.B^T kernel: 16-byte aligned rows
// (leading dimensions multiples of eight elements), even K and split chunks
bool b16_ok(const GemmBatch& b) {
  for (int q = 0; q < b.nprob; ++q) {
    const GemmProb& p = b.p[q];
    if (p.M <= 0 || p.N <= 0) continue;
    if (p.cplx) return false;
    if ((reinterpret_cast<uintptr_t>(p.A) | reinterpret_cast<uintptr_t>(p.B)) % 16) return false;
    if (p.lda % 8 || p.ldb % 8 || p.K % 2) return false;
    if (p.k_splits > 1 && p.k_chunk % 32) return false;
    if (p.gate && (p.k_splits > 1 || p.partial || p.accumulate)) return false;
  }
  return true;
}

// operands of the direct-to-LDS layouts: real problems, 16-byte aligned,
// leading dimensions multiples of four, and a k-major operand a multiple of
// four wide along its rows (its loads are four-column chunks)
bool zdma_ok(const GemmBatch& b, bool TA, bool TB) {
  for (int q = 0; q < b.nprob; ++q) {
    const GemmProb& p = b.p[q];
    if (p.M <= 0 || p.N <= 0) continue;
    if (p.cplx) return false;
    if ((reinterpret_cast<uintptr_t>(p.A) | reinterpret_cast<uintptr_t>(p.B)) % 16) return false;
    if (p.lda % 4 || p.ldb % 4) return false;
    if ((TA && p.M % 4) || (!TB && p.N % 4)) return false;
    if (p.k_splits > 1 && p.k_chunk % 16) return false;
    if (p.gate && (p.k_splits > 1 || p.partial || p.accumulate)) return false;
  }
  return true;
}

// tile counts of every problem of a batch; the batch's block count
int z_tiles(GemmBatch& b) {
  int total = 0;
  for (int q = 0; q < b.nprob; ++q) {
    GemmProb& p = b.p[q];
    p.tiles_m = (p.M + ZM - 1) / ZM;
    p.tiles_n = (p.N + ZN - 1) / ZN;
    if (p.k_splits < 1) p.k_splits = 1;
    if (p.k_splits == 1 && p.k_chunk <= 0) p.k_chunk = p.K;
    p.tile_begin = total;
    if (p.M > 0 && p.N > 0) total += p.tiles_m * p.tiles_n * p.k_splits;
  }
  b.total_tiles = total;
  return total;
}

}  // namespace

// bfloat16 A^T.B with register-staged transposed tiles; hipErrorNotSupported
// (nothing launched) for operands its layout does not take
int gemm_b16t_run(GemmBatch& b, hipStream_t s) {
  if (!b16t_ok(b)) return hipErrorNotSupported;
  const int total = z_tiles(b);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(gemm_b16t_kernel, dim3(total), dim3(ZNT), 0, s, b);
  return hipGetLastError();
}

// bfloat16 A.B^T on the direct-to-LDS block structure; hipErrorNotSupported
// (nothing launched) for operands its layout does not take
int gemm_b16_run(GemmBatch& b, hipStream_t s) {
  if (!b16_ok(b)) return hipErrorNotSupported;
  {
    const int e = gemm_b3_run(b, s);
    if (e != hipErrorNotSupported) return e;
  }
  const int total = z_tiles(b);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(gemm_b16_kernel, dim3(total), dim3(ZNT), 0, s, b);
  return hipGetLastError();
}

// float32 products through bfloat16 pieces; hipErrorNotSupported (nothing
// launched) for operands the direct-to-LDS layouts do not take, complex
// problems, or A^T.B^T
int gemm_x3_run(GemmBatch& b, bool TA, bool TB, int nprod, hipStream_t s) {
  if (nprod == 6) {
    const int e = gemm_s3_run(b, TA, TB, s);
    if (e != hipErrorNotSupported) return e;
  }
  if ((TA && TB) || (nprod != 6 && nprod != 9) || !zdma_ok(b, TA, TB)) return hipErrorNotSupported;
  const int total = z_tiles(b);
  if (total == 0) return hipSuccess;
  const dim3 grid(total), block(ZNT);
  if (nprod == 6) {
    if (!TA && !TB) hipLaunchKernelGGL((gemm_x3_kernel<false, false, 6>), grid, block, 0, s, b);
    else if (!TA) hipLaunchKernelGGL((gemm_x3_kernel<false, true, 6>), grid, block, 0, s, b);
    else hipLaunchKernelGGL((gemm_x3_kernel<true, false, 6>), grid, block, 0, s, b);
  } else {
    if (!TA && !TB) hipLaunchKernelGGL((gemm_x3_kernel<false, false, 9>), grid, block, 0, s, b);
    else if (!TA) hipLaunchKernelGGL((gemm_x3_kernel<false, true, 9>), grid, block, 0, s, b);
    else hipLaunchKernelGGL((gemm_x3_kernel<true, false, 9>), grid, block, 0, s, b);
  }
  return hipGetLastError();
}

}  // namespace so2
