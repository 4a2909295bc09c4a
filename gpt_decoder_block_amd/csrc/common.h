// Shared device helpers for the gfx950 kernels: storage types, 16-byte vector
// access, wavefront (64-lane) and workgroup reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define GDB_WAVE 64

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }

// Number of elements of T in one 16-byte vector.
template <typename T> struct V16 { static constexpr int n = 16 / sizeof(T); };

// Load / store one 16-byte vector of T as floats.
__device__ __forceinline__ void ld16(const float* p, float* o) {
  f32x4 v = *(const f32x4*)p;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = v[i];
}
__device__ __forceinline__ void ld16(const bf16* p, float* o) {
  bf16x8 v = *(const bf16x8*)p;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (float)v[i];
}
__device__ __forceinline__ void st16(float* p, const float* o) {
  f32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = o[i];
  *(f32x4*)p = v;
}
__device__ __forceinline__ void st16(bf16* p, const float* o) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (bf16)o[i];
  *(bf16x8*)p = v;
}

// Non-temporal variants (streamed data read or written once: no reuse expected
// from the caches, which lets the copy engines stream closer to the HBM limit)
__device__ __forceinline__ void ld16_nt(const float* p, float* o) {
  const f32x4 v = __builtin_nontemporal_load((const f32x4*)p);
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = v[i];
}
__device__ __forceinline__ void ld16_nt(const bf16* p, float* o) {
  const bf16x8 v = __builtin_nontemporal_load((const bf16x8*)p);
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (float)v[i];
}
__device__ __forceinline__ void st16_nt(float* p, const float* o) {
  f32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = o[i];
  __builtin_nontemporal_store(v, (f32x4*)p);
}
__device__ __forceinline__ void st16_nt(bf16* p, const float* o) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (bf16)o[i];
  __builtin_nontemporal_store(v, (bf16x8*)p);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Sum over a workgroup of NT threads (NT multiple of 64); every thread gets the
// result.  `red` must hold NT/64 floats of LDS.
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) s += red[i];
  return s;
}
template <int NT>
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float s = -INFINITY;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) s = fmaxf(s, red[i]);
  return s;
}

// exp(x) through the hardware base-2 exponential.
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
