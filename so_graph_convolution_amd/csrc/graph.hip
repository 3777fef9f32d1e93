// Graph preparation: the incoming-edge list grouped by receiver (TrimSO(2)
// page, Appendix B.3) as a CSR over target-sorted edges, and the same grouping
// by sender for the source-side sums of the backward (Section 3.3, Eq.(4)).
//   dst_ptr[n]  = first edge with dst >= n          (edges are sorted by dst)
//   src_perm    = edge ids sorted stably by src       (LSD radix sort)
//   src_ptr[n]  = first position in src_perm with src >= n
// Validation writes a nonzero error word if an index is out of range or dst
// is not non-decreasing.
#include <hipcub/hipcub.hpp>
#include "ops.hpp"

namespace so2 {

namespace {

__global__ void validate_kernel(int N, long E, const int* __restrict__ src, const int* __restrict__ dst, int* err) {
  for (long e = (long)blockIdx.x * blockDim.x + threadIdx.x; e < E; e += (long)gridDim.x * blockDim.x) {
    const int s = src[e], t = dst[e];
    int bad = 0;
    if (s < 0 || s >= N) bad |= 1;
    if (t < 0 || t >= N) bad |= 2;
    if (e + 1 < E && dst[e + 1] < t) bad |= 4;
    if (bad) atomicOr(err, bad);
  }
}

__global__ void iota_kernel(long E, int* __restrict__ v) {
  for (long e = (long)blockIdx.x * blockDim.x + threadIdx.x; e < E; e += (long)gridDim.x * blockDim.x) v[e] = (int)e;
}

// ptr[n] = lower_bound(keys, n), n = 0..N
__global__ void lower_bound_kernel(int N, long E, const int* __restrict__ keys, int* __restrict__ ptr) {
  for (long n = (long)blockIdx.x * blockDim.x + threadIdx.x; n <= N; n += (long)gridDim.x * blockDim.x) {
    long lo = 0, hi = E;
    while (lo < hi) {
      const long mid = (lo + hi) >> 1;
      if (keys[mid] < n) lo = mid + 1;
      else hi = mid;
    }
    ptr[n] = (int)lo;
  }
}

inline int grid_for(long n) {
  long b = (n + 255) / 256;
  if (b > 16384) b = 16384;
  if (b < 1) b = 1;
  return (int)b;
}

inline int key_bits(int N) {
  int b = 1;
  while ((1L << b) < N) ++b;
  return b;
}

size_t cub_bytes(int N, long E) {
  size_t bytes = 0;
  hipcub::DeviceRadixSort::SortPairs(nullptr, bytes, (const int*)nullptr, (int*)nullptr, (const int*)nullptr,
                                     (int*)nullptr, (int)E, 0, key_bits(N));
  return bytes;
}

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

}  // namespace

size_t graph_ws_bytes(int N, long E) {
  return 2 * align256(sizeof(int) * (size_t)(E > 0 ? E : 1)) + align256(cub_bytes(N, E)) + 256;
}

int launch_graph_prepare(int N, long E, const int* src, const int* dst, int* dst_ptr, int* src_perm, int* src_ptr,
                         void* ws, size_t ws_bytes, int* err_word, hipStream_t s) {
  if (ws_bytes < graph_ws_bytes(N, E)) return hipErrorInvalidValue;
  char* p = static_cast<char*>(ws);
  int* keys_sorted = reinterpret_cast<int*>(p);
  p += align256(sizeof(int) * (size_t)(E > 0 ? E : 1));
  int* ids = reinterpret_cast<int*>(p);
  p += align256(sizeof(int) * (size_t)(E > 0 ? E : 1));
  void* tmp = p;
  size_t tmp_bytes = cub_bytes(N, E);

  if (err_word && E > 0) {
    hipLaunchKernelGGL(validate_kernel, dim3(grid_for(E)), dim3(256), 0, s, N, E, src, dst, err_word);
  }
  hipLaunchKernelGGL(lower_bound_kernel, dim3(grid_for((long)N + 1)), dim3(256), 0, s, N, E, dst, dst_ptr);
  if (E > 0) {
    hipLaunchKernelGGL(iota_kernel, dim3(grid_for(E)), dim3(256), 0, s, E, ids);
    hipError_t e = hipcub::DeviceRadixSort::SortPairs(tmp, tmp_bytes, src, keys_sorted, ids, src_perm, (int)E, 0,
                                                      key_bits(N), s);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(lower_bound_kernel, dim3(grid_for((long)N + 1)), dim3(256), 0, s, N, E, keys_sorted, src_ptr);
  return hipGetLastError();
}

}  // namespace so2
