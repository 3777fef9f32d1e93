// Host-side helpers shared by the library's entry-point translation units:
// the thread's last-error message, the workspace bump allocator, and the GEMM
// launch helpers of the per-order products.
#pragma once
#include <hip/hip_runtime.h>

#include <string>
#include <vector>

#include "../../include/so2conv.h"
#include "gemm.hpp"

namespace so2 {

// set the calling thread's last-error message (read by so2conv_last_error) and return code
int fail(int code, const std::string& msg);
int set_error(int code, const std::string& msg);   // the same, for translation units without this header's macros
void clear_error();
const char* last_error();

#define SO2_HIP(expr)                                                                       \
  do {                                                                                      \
    int _e = (int)(expr);                                                                   \
    if (_e != 0) return ::so2::fail(SO2_EHIP, std::string("HIP error in ") + #expr + ": " + \
                                                  hipGetErrorString((hipError_t)_e));       \
  } while (0)

inline size_t al(size_t v) { return (v + 255) & ~size_t(255); }

// Bump allocator over the caller's workspace. With a null base it only
// measures: every stage lays out its buffers through one function, used both
// to size the workspace and to carve it.
struct Arena {
  char* base;
  size_t used;
  void* bytes(size_t n) {
    void* p = base ? base + used : nullptr;
    used += al(n);
    return p;
  }
  float* take(size_t floats) { return static_cast<float*>(bytes(sizeof(float) * floats)); }
};

// one GEMM problem C (+)= op(A) op(B) of M x N x K (see GemmProb)
GemmProb prob(const void* A, int lda, const void* B, int ldb, float* C, int ldc, int M, int N, int K, int acc = 0);

// Operand kinds of run_batch: float32 on the float32 matrix cores, bfloat16,
// or float32 through bfloat16 pieces (gemm_x3_run; problems it does not take
// run on the float32 matrix cores).
enum { kOpF32 = 0, kOpBF16 = 1, kOpSplit = 2 };

// Batch-wide fields of the gated epilogue (GemmBatch::gC, gL, ldz, ldgam)
struct GateCols {
  int C, L, ldz, ldgam;
};
// run_batch's return when gated problems reach a launch whose kernels have no
// gated epilogue (nothing of that launch ran; the caller falls back)
constexpr int kNoFusedGate = 1;

// launch the problems (all with the same TA, TB and operand kind), several per
// launch; records their timing when GEMM profiling is on. With `gate`, the
// problems carry the gated epilogue.
int run_batch(std::vector<GemmProb>& ps, bool TA, bool TB, int op, hipStream_t s, const GateCols* gate = nullptr);

// splits and K chunk of a split-K product over K rows (a multiple of the GEMM K
// tile); run_tn's partial buffer holds sum over segments of splits * M * N floats
void split_plan(long K, int* splits, int* chunk, bool small = false);

// Weight gradient G[M][N] (+)= sum over segments of A_s^T B_s, A_s [K_s][lda], B_s [K_s][ldb];
// deterministic split-K through the partial buffer P.
struct TnSeg {
  const void* A;
  int lda;
  const void* B;
  int ldb;
  long K;
};
int run_tn(const TnSeg* segs, int nseg, int M, int N, float* G, int ldg, int accumulate, float* P, int op,
           hipStream_t s);

// zero n floats
int fill(float* p, size_t n, hipStream_t s);

}  // namespace so2
