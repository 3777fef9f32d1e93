// Storage types of the GEMM operands. The bfloat16 path keeps node arrays,
// GEMM outputs and every reduction in float32 and stores only the per-edge
// operands of the per-order linears (and the realified weights) as bfloat16,
// rounded to nearest even.
#pragma once
#include <hip/hip_runtime.h>

namespace so2 {

struct bf16s {
  unsigned short u;
};

__host__ __device__ inline float bf16_to_f32(unsigned short h) {
  return __builtin_bit_cast(float, (unsigned)h << 16);
}

// round to nearest even; NaN stays NaN (a select, not a branch: no divergent
// control flow around every store)
__host__ __device__ inline unsigned short f32_to_bf16(float f) {
  const unsigned u = __builtin_bit_cast(unsigned, f);
  const unsigned rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const unsigned quiet = (u >> 16) | 0x40u;
  return (unsigned short)(((u & 0x7fffffffu) > 0x7f800000u) ? quiet : rounded);
}

// four consecutive elements (16-byte aligned float, 8-byte aligned bf16)
__device__ __forceinline__ void ld4(const float* p, float (&v)[4]) {
  const float4 x = *reinterpret_cast<const float4*>(p);
  v[0] = x.x;
  v[1] = x.y;
  v[2] = x.z;
  v[3] = x.w;
}
__device__ __forceinline__ void st4(float* p, const float (&v)[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st4(bf16s* p, const float (&v)[4]) {
  uint2 u;
  u.x = (unsigned)f32_to_bf16(v[0]) | ((unsigned)f32_to_bf16(v[1]) << 16);
  u.y = (unsigned)f32_to_bf16(v[2]) | ((unsigned)f32_to_bf16(v[3]) << 16);
  *reinterpret_cast<uint2*>(p) = u;
}

__device__ __forceinline__ void st(float* p, float v) { *p = v; }
__device__ __forceinline__ void st(bf16s* p, float v) { p->u = f32_to_bf16(v); }
__device__ __forceinline__ float ld(const float* p) { return *p; }
__device__ __forceinline__ float ld(const bf16s* p) { return bf16_to_f32(p->u); }

}  // namespace so2
