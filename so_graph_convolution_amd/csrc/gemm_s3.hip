// float32 GEMMs on the bfloat16 matrix cores with every operand element split
// once per block. As in the fragment-split kernel, a float32 x is the exact
// sum of three bfloat16 pieces (truncation: h = x with the low 16 bits
// cleared, m likewise of x - h, l = x - h - m) and a float32 product is taken
// as the six piece products h.l, m.m, l.h, h.m, m.h, h.h (smallest first;
// the dropped m.l, l.m, l.l sum below 2^-23 |x y|). Here the block splits
// each staged element once, on its way into LDS, instead of each wave
// splitting the fragments it multiplies (two to four waves share a fragment).
//
// Block tile 256 x 256 of four waves (2 x 2, 128 x 128 each: 4 x 4 tiles of
// v_mfma_f32_32x32x16_bf16, 256 accumulator registers, one wave per SIMD),
// k tile 16 float32. Per k tile a thread loads 16 elements of A and 16 of B
// (four 16-byte loads each) into registers one tile ahead, splits them and
// writes the pieces to the other of two LDS stages while the wave's 96 MFMAs
// of the current tile run. A k-contiguous operand is loaded as 64-byte row
// segments (four lanes per row), a k-major one as 4 k x 4 column blocks that
// the thread transposes in registers. LDS holds, per operand and piece, 256
// rows of 16 k (two 16-byte units, unit u of row r at u ^ ((r / 8) mod 2):
// a fragment read of 16 rows covers the 64 banks once).
#include "gemm.hpp"
#include "gemm_tile.hpp"

namespace so2 {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int TM = 256, TN = 256, TKK = 16;   // block tile, k per tile
constexpr int NT = 256;                       // threads
constexpr int STAGE_UNITS = 2 * 3 * 256 * 2;  // 16-byte units per stage: [operand][piece][row][unit]

__device__ __forceinline__ int s_unit(int op, int piece, int row, int u) {
  return ((op * 3 + piece) * 256 + row) * 2 + (u ^ ((row >> 3) & 1));
}

// three bfloat16 pieces of four float32 values, two per dword (element 2i in the low half)
__device__ __forceinline__ void split4(const float (&x)[4], u32x2& ph, u32x2& pm, u32x2& pl) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const float x0 = x[2 * q], x1 = x[2 * q + 1];
    const float r0 = x0 - __uint_as_float(__float_as_uint(x0) & 0xffff0000u);
    const float r1 = x1 - __uint_as_float(__float_as_uint(x1) & 0xffff0000u);
    const float s0 = r0 - __uint_as_float(__float_as_uint(r0) & 0xffff0000u);
    const float s1 = r1 - __uint_as_float(__float_as_uint(r1) & 0xffff0000u);
    ph[q] = __builtin_amdgcn_perm(__float_as_uint(x1), __float_as_uint(x0), 0x07060302u);
    pm[q] = __builtin_amdgcn_perm(__float_as_uint(r1), __float_as_uint(r0), 0x07060302u);
    pl[q] = __builtin_amdgcn_perm(__float_as_uint(s1), __float_as_uint(s0), 0x07060302u);
  }
}

// One operand's share of a k tile for thread `tid`.
//   k-contiguous (element (k, r) at P[r ld + k]): chunk q = tid mod 4 (k 4q..4q+3)
//     of rows tid / 4 + 64 j, j < 4; rows past the edge load the last row.
//   k-major (element (k, r) at P[k ld + r]): k rows 4 kb .. 4 kb + 3, kb = tid / 64,
//     columns 4 cb .. 4 cb + 3, cb = tid mod 64 (the last whole block past the edge).
// Values past the end of the split's k range are zero.
template <bool KM>
struct Stager {
  const float* base;   // this thread's first element in k tile 0 of the split
  long jstep;          // elements between the thread's four loads
  int kofs;            // k of the thread's first value within a tile
  __device__ void init(const float* P, int ld, int r0, int rlim, int kbeg, int tid) {
    if (KM) {
      const int kb = tid / 64, cb = tid % 64;
      const int col = min(r0 + 4 * cb, rlim - 4);
      kofs = 4 * kb;
      base = P + (size_t)(kbeg + kofs) * ld + col;
      jstep = ld;
    } else {
      const int q = tid % 4;
      kofs = 4 * q;
      base = P + kbeg + kofs;
      jstep = 0;
      row0 = r0 + tid / 4;
      rl = rlim;
      pld = ld;
    }
  }
  int row0 = 0, rl = 0, pld = 0;
  // load tile t (k0 = 16 t within the split, nkk > 0 k values in the split).
  // Every load is issued (no branch): a k past the range reads the split's
  // last k instead, and ok[j] = false makes store() write zeros for it (the
  // select waits for the data, so it is left to the store, a tile later).
  __device__ void load(int t, int nkk, float (&x)[4][4], bool (&ok)[4]) const {
    const int k0 = TKK * t;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float* p;
      if (KM) {
        const int k = k0 + kofs + j;
        ok[j] = k < nkk;
        p = base + (long)(min(k, nkk - 1) - kofs) * jstep;
      } else {
        const int row = min(row0 + 64 * j, rl - 1);
        const int k = k0 + kofs;
        ok[j] = k < nkk;
        p = base + (size_t)row * pld + (min(k, nkk - 4) - kofs);
      }
      const f32x4 v = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
      for (int c = 0; c < 4; ++c) x[j][c] = v[c];
    }
  }
  // split unit u (< 4) of the thread's share and write it to LDS stage S
  // (operand op): k-major, column 4 cb + u at k 4 kb .. 4 kb + 3; k-contiguous,
  // row tid / 4 + 64 u at k 4q .. 4q + 3 (16-byte unit k / 8, half (k / 4) mod 2)
  __device__ __forceinline__ void store(u32x4* S, int op, int tid, const float (&x)[4][4], const bool (&ok)[4],
                                        int u) const {
    u32x2* S2 = reinterpret_cast<u32x2*>(S);
    int row, kq;
    u32x2 h, m, l;
    if (KM) {
      const float v[4] = {ok[0] ? x[0][u] : 0.f, ok[1] ? x[1][u] : 0.f, ok[2] ? x[2][u] : 0.f,
                          ok[3] ? x[3][u] : 0.f};
      split4(v, h, m, l);
      row = 4 * (tid % 64) + u;
      kq = tid / 64;
    } else {
      const float v[4] = {ok[u] ? x[u][0] : 0.f, ok[u] ? x[u][1] : 0.f, ok[u] ? x[u][2] : 0.f, ok[u] ? x[u][3] : 0.f};
      split4(v, h, m, l);
      row = tid / 4 + 64 * u;
      kq = tid % 4;
    }
    S2[2 * s_unit(op, 0, row, kq / 2) + kq % 2] = h;
    S2[2 * s_unit(op, 1, row, kq / 2) + kq % 2] = m;
    S2[2 * s_unit(op, 2, row, kq / 2) + kq % 2] = l;
  }
};

struct Frag {
  bf16x8 h, m, l;
};
__device__ __forceinline__ Frag frag(const u32x4* S, int op, int row, int lk) {
  Frag f;
  f.h = __builtin_bit_cast(bf16x8, S[s_unit(op, 0, row, lk)]);
  f.m = __builtin_bit_cast(bf16x8, S[s_unit(op, 1, row, lk)]);
  f.l = __builtin_bit_cast(bf16x8, S[s_unit(op, 2, row, lk)]);
  return f;
}
__device__ __forceinline__ floatx16 mfma(const bf16x8& a, const bf16x8& b, const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// C = op(A) op(B) with float32 operands; AKM: A stored k-major (A^T.B), BKM:
// B stored k-major (A.B and A^T.B)
template <bool AKM, bool BKM>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_s3_kernel(GemmBatch batch) {
  __shared__ u32x4 T[2][STAGE_UNITS];
  int pi, local;
  decode_tile(batch, xcd_remap(blockIdx.x, batch.total_tiles), &pi, &local);
  const GemmProb& p = batch.p[pi];
  const int per_split = p.tiles_m * p.tiles_n;
  const int split = local / per_split;
  local -= split * per_split;
  const int tm = local / p.tiles_n, tn = local - tm * p.tiles_n;
  const int m0 = tm * TM, n0 = tn * TN;
  const int kbeg = split * p.k_chunk, kend = min(p.K, kbeg + p.k_chunk);
  const int nkk = kend - kbeg, nk = (nkk + TKK - 1) / TKK;
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int wm = wave >> 1, wn = wave & 1, li = lane % 32, lk = lane / 32;
  Stager<AKM> sa;
  Stager<BKM> sb;
  sa.init(static_cast<const float*>(p.A), p.lda, m0, p.M, kbeg, tid);
  sb.init(static_cast<const float*>(p.B), p.ldb, n0, p.N, kbeg, tid);
  floatx16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  float xa[4][4], xb[4][4];
  bool oka[4], okb[4];
  if (nk > 0) {
    sa.load(0, nkk, xa, oka);
    sb.load(0, nkk, xb, okb);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      sa.store(T[0], 0, tid, xa, oka, u);
      sb.store(T[0], 1, tid, xb, okb, u);
    }
    sa.load(min(1, nk - 1), nkk, xa, oka);
    sb.load(min(1, nk - 1), nkk, xb, okb);
  }
  __syncthreads();
  const int ra = wm * 128 + li, rb = wn * 128 + li;
#pragma unroll 1
  for (int kt = 0; kt < nk; ++kt) {
    const u32x4* st = T[kt & 1];
    Frag fa[4], fb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fa[i] = frag(st, 0, ra + 32 * i, lk);
      fb[i] = frag(st, 1, rb + 32 * i, lk);
    }
    // The next tile's split goes to the other stage (read by every wave
    // before the last barrier; after the last tile a stale copy, never read)
    // in eight units, each ahead of 8 of the first 64 products (two A tiles
    // of one piece product against the four B tiles), so the VALU work
    // issues while the matrix core runs; scheduling barriers keep that order.
    // The loads of the tile after it and the last 32 products follow.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if (c < 4) sa.store(T[(kt + 1) & 1], 0, tid, xa, oka, c);
      else sb.store(T[(kt + 1) & 1], 1, tid, xb, okb, c - 4);
      const int pr = c / 2;
#pragma unroll
      for (int a = 2 * (c % 2); a < 2 * (c % 2) + 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const bf16x8& x = pr == 0 ? fa[a].h : pr == 1 ? fa[a].m : pr == 2 ? fa[a].l : fa[a].h;
          const bf16x8& y = pr == 0 ? fb[b].l : pr == 1 ? fb[b].m : pr == 2 ? fb[b].h : fb[b].m;
          acc[a][b] = mfma(x, y, acc[a][b]);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
    // the loads of the tile after it (the last tile again at the end: never stored)
    sa.load(min(kt + 2, nk - 1), nkk, xa, oka);
    sb.load(min(kt + 2, nk - 1), nkk, xb, okb);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = mfma(fa[a].m, fb[b].h, acc[a][b]);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = mfma(fa[a].h, fb[b].h, acc[a][b]);
    __syncthreads();
  }

  // lane (li, lk) of MFMA tile (a, b) holds column 32 b + li, rows
  // 32 a + 8 g + 4 lk + i (g, i < 4) of the wave's 128 x 128 tile
  const int i0 = m0 + wm * 128 + 4 * lk, j0 = n0 + wn * 128 + li;
  float* out = p.partial ? p.C + (size_t)split * p.M * p.N : p.C;
  const int ldo = p.partial ? p.N : p.ldc;
  const bool add = p.accumulate && !p.partial;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
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

// bfloat16 A.B^T (both operands k-contiguous) on the same block structure:
// 256 x 256 blocks of four 128 x 128 waves, 64 k per tile in two LDS stages
// of 64 KB (per operand 256 rows of eight 16-byte units, unit u of row r at
// u ^ ((r / 2) mod 8), so a fragment read of 16 rows covers the 64 banks
// once). Each thread loads 16 units (eight lanes per 128-byte row segment) a
// tile ahead and writes them to the other stage while the wave's 64 MFMAs of
// the current tile run; within a tile the fragments of k step s + 1 are read
// while the 16 MFMAs of step s run.
constexpr int BK = 64;   // bfloat16 k per tile
__device__ __forceinline__ int b_unit(int op, int row, int u) { return (op * 256 + row) * 8 + (u ^ ((row >> 1) & 7)); }

struct BFrag {
  bf16x8 a[4], b[4];
};
__device__ __forceinline__ void bread(const u32x4* S, int ra, int rb, int u, BFrag& F) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    F.a[i] = __builtin_bit_cast(bf16x8, S[b_unit(0, ra + 32 * i, u)]);
    F.b[i] = __builtin_bit_cast(bf16x8, S[b_unit(1, rb + 32 * i, u)]);
  }
}
__device__ __forceinline__ void bmma(const BFrag& F, floatx16 (&acc)[4][4]) {
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = mfma(F.a[a], F.b[b], acc[a][b]);
}

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_b3_kernel(GemmBatch batch) {
  __shared__ u32x4 T[2][2 * 256 * 8];
  int pi, local;
  decode_tile(batch, xcd_remap(blockIdx.x, batch.total_tiles), &pi, &local);
  const GemmProb& p = batch.p[pi];
  const int per_split = p.tiles_m * p.tiles_n;
  const int split = local / per_split;
  local -= split * per_split;
  const int tm = local / p.tiles_n, tn = local - tm * p.tiles_n;
  const int m0 = tm * TM, n0 = tn * TN;
  const int kbeg = split * p.k_chunk, kend = min(p.K, kbeg + p.k_chunk);
  const int nkk = kend - kbeg, nk = (nkk + BK - 1) / BK;
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int wm = wave >> 1, wn = wave & 1, li = lane % 32, lk = lane / 32;
  // staging: unit su (k 8 su .. 8 su + 7 of the tile) of rows sr + 32 j, j < 8,
  // of each operand; rows past the edge load the last row, a unit past the
  // split's k range loads its last unit and is stored as zeros
  const int su = tid % 8, sr = tid / 8;
  const unsigned short* Ap = static_cast<const unsigned short*>(p.A) + kbeg;
  const unsigned short* Bp = static_cast<const unsigned short*>(p.B) + kbeg;
  u32x4 xa[8], xb[8];
  bool oka = false, okb = false;
  auto load = [&](const unsigned short* P, int ld, int r0, int rlim, int t, u32x4 (&x)[8], bool& ok) {
    const int k = BK * t + 8 * su;
    ok = k < nkk;
    const int kk = min(k, nkk - 8);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = min(r0 + sr + 32 * j, rlim - 1);
      x[j] = *reinterpret_cast<const u32x4*>(P + (size_t)row * ld + kk);
    }
  };
  auto store = [&](u32x4* S, int op, const u32x4 (&x)[8], bool ok, int j0) {
#pragma unroll
    for (int j = j0; j < j0 + 4; ++j) S[b_unit(op, sr + 32 * j, su)] = ok ? x[j] : u32x4{0u, 0u, 0u, 0u};
  };
  floatx16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
  if (nk > 0) {
    load(Ap, p.lda, m0, p.M, 0, xa, oka);
    load(Bp, p.ldb, n0, p.N, 0, xb, okb);
    store(T[0], 0, xa, oka, 0);
    store(T[0], 0, xa, oka, 4);
    store(T[0], 1, xb, okb, 0);
    store(T[0], 1, xb, okb, 4);
    load(Ap, p.lda, m0, p.M, min(1, nk - 1), xa, oka);
    load(Bp, p.ldb, n0, p.N, min(1, nk - 1), xb, okb);
  }
  __syncthreads();
  const int ra = wm * 128 + li, rb = wn * 128 + li;
#pragma unroll 1
  for (int kt = 0; kt < nk; ++kt) {
    const u32x4* st = T[kt & 1];
    u32x4* nx = T[(kt + 1) & 1];   // the next tile (after the last tile a stale copy, never read)
    // k step s takes unit 4 (s / 2) + 2 lk + s mod 2 (k 16 lk + 8 (s mod 2) ..
    // of the tile's 32-k half s / 2): the k values each MFMA meets are those
    // of gemm_b16_kernel's 32-k tiles, so the two agree bit for bit
    BFrag F0, F1;
    bread(st, ra, rb, 2 * lk, F0);
    __builtin_amdgcn_sched_barrier(0);
    // k step 0: step 1's fragments, A's first half of the next tile
    bread(st, ra, rb, 2 * lk + 1, F1);
    store(nx, 0, xa, oka, 0);
    bmma(F0, acc);
    __builtin_amdgcn_sched_barrier(0);
    // k step 1: step 2's fragments, A's second half, then A's loads of the tile after
    bread(st, ra, rb, 4 + 2 * lk, F0);
    store(nx, 0, xa, oka, 4);
    load(Ap, p.lda, m0, p.M, min(kt + 2, nk - 1), xa, oka);
    bmma(F1, acc);
    __builtin_amdgcn_sched_barrier(0);
    // k step 2: step 3's fragments, B's first half
    bread(st, ra, rb, 5 + 2 * lk, F1);
    store(nx, 1, xb, okb, 0);
    bmma(F0, acc);
    __builtin_amdgcn_sched_barrier(0);
    // k step 3: B's second half, then B's loads
    store(nx, 1, xb, okb, 4);
    load(Bp, p.ldb, n0, p.N, min(kt + 2, nk - 1), xb, okb);
    bmma(F1, acc);
    __syncthreads();
  }
  const int i0 = m0 + wm * 128 + 4 * lk, j0 = n0 + wn * 128 + li;
  float* out = p.partial ? p.C + (size_t)split * p.M * p.N : p.C;
  const int ldo = p.partial ? p.N : p.ldc;
  const bool add = p.accumulate && !p.partial;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
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

// operands of the bfloat16 kernel: real, ungated problems, 16-byte aligned
// rows (leading dimensions multiples of eight), K a multiple of eight, split
// chunks multiples of the 64-k tile
bool b3_ok(const GemmBatch& b) {
  for (int q = 0; q < b.nprob; ++q) {
    const GemmProb& p = b.p[q];
    if (p.M <= 0 || p.N <= 0) continue;
    if (p.cplx || p.gate) return false;
    if ((reinterpret_cast<uintptr_t>(p.A) | reinterpret_cast<uintptr_t>(p.B)) % 16) return false;
    if (p.lda % 8 || p.ldb % 8 || p.K % 8) return false;
    if (p.k_splits > 1 && p.k_chunk % BK) return false;
  }
  return true;
}

// operands the kernel takes: real, ungated problems; 16-byte aligned operands
// with leading dimensions multiples of four; K a multiple of four where an
// operand is k-contiguous, the row width (M or N) a multiple of four where it
// is k-major; split chunks multiples of the k tile
bool s3_ok(const GemmBatch& b, bool TA, bool TB) {
  for (int q = 0; q < b.nprob; ++q) {
    const GemmProb& p = b.p[q];
    if (p.M <= 0 || p.N <= 0) continue;
    if (p.cplx || p.gate) return false;
    if ((reinterpret_cast<uintptr_t>(p.A) | reinterpret_cast<uintptr_t>(p.B)) % 16) return false;
    if (p.lda % 4 || p.ldb % 4) return false;
    if ((!TA || TB) && p.K % 4) return false;
    if ((TA && p.M % 4) || (!TB && p.N % 4)) return false;
    if (p.k_splits > 1 && p.k_chunk % TKK) return false;
  }
  return true;
}

int s3_tiles(GemmBatch& b) {
  int total = 0;
  for (int q = 0; q < b.nprob; ++q) {
    GemmProb& p = b.p[q];
    p.tiles_m = (p.M + TM - 1) / TM;
    p.tiles_n = (p.N + TN - 1) / TN;
    if (p.k_splits < 1) p.k_splits = 1;
    if (p.k_splits == 1 && p.k_chunk <= 0) p.k_chunk = p.K;
    p.tile_begin = total;
    if (p.M > 0 && p.N > 0) total += p.tiles_m * p.tiles_n * p.k_splits;
  }
  b.total_tiles = total;
  return total;
}

}  // namespace

int gemm_b3_run(GemmBatch& b, hipStream_t s) {
  if (!b3_ok(b)) return hipErrorNotSupported;
  const int total = s3_tiles(b);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(gemm_b3_kernel, dim3(total), dim3(NT), 0, s, b);
  return hipGetLastError();
}

int gemm_s3_run(GemmBatch& b, bool TA, bool TB, hipStream_t s) {
  if ((TA && TB) || !s3_ok(b, TA, TB)) return hipErrorNotSupported;
  const int total = s3_tiles(b);
  if (total == 0) return hipSuccess;
  const dim3 grid(total), block(NT);
  if (!TA && !TB) hipLaunchKernelGGL((gemm_s3_kernel<false, true>), grid, block, 0, s, b);
  else if (!TA) hipLaunchKernelGGL((gemm_s3_kernel<false, false>), grid, block, 0, s, b);
  else hipLaunchKernelGGL((gemm_s3_kernel<true, true>), grid, block, 0, s, b);
  return hipGetLastError();
}

}  // namespace so2
