// Grouped GEMMs on CDNA4 matrix cores: float32 operands
// (v_mfma_f32_32x32x2_f32) or bfloat16 operands (v_mfma_f32_32x32x16_bf16),
// float32 accumulation and output in both cases.
//
// The per-order SO(2) linears (TrimSO(2) page, Section 3.1 and Eq.(1)) are
// the one dense contraction of the convolution: for every retained order a
// [rows x k] by [k x n] product. One launch covers several such problems.
//   C = op(A) op(B)   (or C += ... with accumulate)
//   op(A)[i][k] = TA ? A[k*lda + i] : A[i*lda + k]
//   op(B)[k][j] = TB ? B[j*ldb + k] : B[k*ldb + j]
// The bfloat16 kernels take A.B^T and A^T.B only (a forward product uses the
// transposed copy of the weight).
// TA problems (weight gradients, K = edges) are split over K; every split
// writes its own partial tile and gemm_reduce sums the splits in a fixed
// order, so results are bitwise reproducible (no atomics).
//
// Complex problems (float32 only): the per-order products of orders m >= 1
// are complex products (TrimSO(2) page, Eq.(1): u+ + i u- = (T+ + i T-)(W0 + i W1)),
// taken with three real products instead of four:
//   op(A) = a + i sA b,  op(B) = c + i sB d   (b, d at element offsets dA, dB from a, c)
//   P1 = a c, P2 = b d, P3 = (a + sA b)(c + sB d)
//   Re = P1 - sA sB P2,  Im = P3 - P1 - sA sB P2
// M, N, K are the complex sizes; the real part goes to C, the imaginary part
// N columns to its right (a split writes [M][2N] partials).
#pragma once
#include <hip/hip_runtime.h>

namespace so2 {

constexpr int kGemmMaxProbs = 32;   // problems per launch (kernel argument < 4 KB)

struct GemmProb {
  const void* A;     // float or bfloat16 elements (one type per launch)
  const void* B;
  float* C;          // output, or the partial buffer [k_splits][M][N] of a split problem
  int M, N, K;
  int lda, ldb, ldc;
  int tiles_m, tiles_n;
  int k_splits;      // >= 1
  int k_chunk;       // K rows per split (multiple of the K tile)
  int accumulate;    // add into C (non-partial problems only)
  int partial;       // write split s to C + s*M*N (row pitch N) instead of C
  int tile_begin;    // first linear tile of this problem
  int cplx;          // complex problem (all problems of a launch agree)
  int dA, dB;        // complex: element offsets of b from a and of d from c
  float sA, sB;      // complex: signs of b and d (+1 or -1)
  // gated epilogue (0: none; a + 1: the first linear's output block of order
  // a): besides C it writes Z = the gated activation of C, reading the gate
  // pre-activations of each row from gam (see GemmBatch)
  int gate;
  void* Z;           // Z block of this problem (row pitch GemmBatch::ldz)
  const float* gam;  // gate columns (l = 1..L, c) of this problem's first row (row pitch GemmBatch::ldgam)
};

struct GemmBatch {
  GemmProb p[kGemmMaxProbs];
  int nprob;
  int total_tiles;
  // gated epilogue, shared by the batch: channels C, degree L, row pitches of
  // Z and of the gate columns. Column j of block a holds degree
  // l = a + (j mod (L - a + 1) C) / C and channel j mod C; l = 0 takes
  // SiLU(u), l >= 1 takes sigmoid(gam[(l - 1) C + c]) u.
  int gC, gL, ldz, ldgam;
};
static_assert(sizeof(GemmBatch) <= 4096, "a GemmBatch is passed as one kernel argument (4 KB at most)");

// Fill tiling fields and launch. Every problem of one batch shares TA/TB and
// the operand type. Returns a hipError_t (hipErrorInvalidValue for a bfloat16
// A.B or A^T.B^T).
int gemm_run(GemmBatch& b, bool TA, bool TB, bool bf16, hipStream_t s);

// float32 products through bfloat16 pieces (each operand the exact sum of
// three bfloat16 values; nprod = 6 or 9 piece products per float32 product) on
// 256 x 256 blocks of eight 128 x 64 waves; real problems only, no A^T.B^T.
// hipErrorNotSupported (nothing launched) unless every operand is 16-byte
// aligned with leading dimensions (and a k-major operand's width) multiples of four.
int gemm_x3_run(GemmBatch& b, bool TA, bool TB, int nprod, hipStream_t s);
// The six-product float32 GEMM with every staged element split once per block
// (256 x 256 blocks of four 128 x 128 waves); gemm_x3_run takes it first for
// nprod = 6. hipErrorNotSupported (nothing launched) for complex or gated
// problems, A^T.B^T, operands not 16-byte aligned or with leading dimensions
// not multiples of four, K not a multiple of four where an operand is
// k-contiguous, a k-major operand's width not a multiple of four.
int gemm_s3_run(GemmBatch& b, bool TA, bool TB, hipStream_t s);
// bfloat16 A.B^T on the same four-wave blocks (64 k per tile, register-staged
// loads a tile ahead); gemm_b16_run takes it first. hipErrorNotSupported
// (nothing launched) for complex or gated problems, operands not 16-byte
// aligned or with leading dimensions or K not multiples of eight.
int gemm_b3_run(GemmBatch& b, hipStream_t s);
// bfloat16 A.B^T on the same block structure; hipErrorNotSupported (nothing
// launched) unless operands are 16-byte aligned, leading dimensions multiples
// of eight and K even (split chunks multiples of 32).
int gemm_b16_run(GemmBatch& b, hipStream_t s);
// bfloat16 A^T.B (both operands k-major) on 256 x 256 blocks of eight 128 x 64
// waves with register-staged, transposed tiles; hipErrorNotSupported (nothing
// launched) unless rows are 16-byte aligned, M, N and leading dimensions
// multiples of eight and split chunks multiples of 64.
int gemm_b16t_run(GemmBatch& b, hipStream_t s);
// Gated problems (GemmProb::gate) run only on gemm_x3_run (Z float32) and
// gemm_b16_run (Z bfloat16); gemm_run does not take them.

// K tile of the kernels: split chunks of TA problems are multiples of it
constexpr int kGemmKTile = 64;

// C[i*ldc + j] (+)= sum_{s < splits} P[s][i][j]  (fixed order); with trans,
// C[j*ldc + i] instead (the partials hold the transposed product)
int gemm_reduce(const float* P, int splits, int M, int N, float* C, int ldc, int accumulate, hipStream_t s,
                int trans = 0);

}  // namespace so2
