// Compile-time (lmax, mmax) instantiation of the per-channel kernels: the
// per-channel rotation products are fully unrolled so that node and edge rows
// stay in registers.
#pragma once
#include <hip/hip_runtime.h>

namespace so2 {

// Supported pairs: the pages' workloads (lmax 2..6 with mmax 2, lmax 4 with
// mmax 1..4) plus small cases.
template <template <int, int> class K, typename... Args>
inline int dispatch_lm(int L, int M, Args&&... args) {
  switch (L * 8 + M) {
    case 0 * 8 + 0: return K<0, 0>::run(args...);
    case 1 * 8 + 1: return K<1, 1>::run(args...);
    case 2 * 8 + 1: return K<2, 1>::run(args...);
    case 2 * 8 + 2: return K<2, 2>::run(args...);
    case 3 * 8 + 1: return K<3, 1>::run(args...);
    case 3 * 8 + 2: return K<3, 2>::run(args...);
    case 4 * 8 + 1: return K<4, 1>::run(args...);
    case 4 * 8 + 2: return K<4, 2>::run(args...);
    case 4 * 8 + 3: return K<4, 3>::run(args...);
    case 4 * 8 + 4: return K<4, 4>::run(args...);
    case 5 * 8 + 2: return K<5, 2>::run(args...);
    case 6 * 8 + 2: return K<6, 2>::run(args...);
    default: return (int)hipErrorInvalidValue;
  }
}

inline bool lm_pair_compiled(int L, int M) {
  switch (L * 8 + M) {
    case 0: case 9: case 17: case 18: case 25: case 26: case 33: case 34: case 35: case 36: case 42: case 50:
      return true;
    default:
      return false;
  }
}

}  // namespace so2
