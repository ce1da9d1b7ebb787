// Row helpers of the bandwidth-bound token kernels: 8 consecutive elements of a
// row moved between memory (16 bytes of bf16 or 32 bytes of float32, aligned)
// and float32 registers.
#pragma once

#include "common.h"

namespace moe {

// 8 consecutive elements kept as loaded (one or two 16-byte loads) and converted
// element by element where they are used: half the registers of a float32 copy
// for 16-bit rows, so more row loads fit in flight.
template <typename T> struct Raw16;
template <> struct Raw16<bf16> {
  typedef bf16x8 type;
  __device__ __forceinline__ static type load(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
  __device__ __forceinline__ static float get(const type& v, int i) { return static_cast<float>(v[i]); }
};
template <> struct Raw16<float> {
  struct type { f32x4 a, b; };
  __device__ __forceinline__ static type load(const float* p) {
    return {*reinterpret_cast<const f32x4*>(p), *reinterpret_cast<const f32x4*>(p + 4)};
  }
  __device__ __forceinline__ static float get(const type& v, int i) { return i < 4 ? v.a[i] : v.b[i - 4]; }
};

__device__ __forceinline__ void load8(const bf16* p, float* v) {
  const bf16x8 q = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = static_cast<float>(q[i]);
}
__device__ __forceinline__ void store8(bf16* p, const float* v) {
  bf16x8 q;
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = static_cast<bf16>(v[i]);
  *reinterpret_cast<bf16x8*>(p) = q;
}
__device__ __forceinline__ void load8(const float* p, float* v) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[i + 4] = b[i]; }
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  f32x4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) { a[i] = v[i]; b[i] = v[i + 4]; }
  *reinterpret_cast<f32x4*>(p) = a;
  *reinterpret_cast<f32x4*>(p + 4) = b;
}

// Sum over the 64 lanes of a wavefront; every lane ends with the same bits.
__device__ __forceinline__ float wave_sum64(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace moe
