// fp8 operands of the MLP GEMMs in the largest model of "Comment Entraîner
// Votre Propre ChatGPT Pour 50€ ?" (section "1. Le modèle GPT": most layers'
// matrix products in fp8).  Per-tensor dynamic scaling: amax = max |x|, scale
// s = amax / 448, code = e4m3(x / s) rounded to nearest even and saturating
// at 448 (OCP e4m3fn: 3 mantissa bits, exponent bias 7, subnormal step 2^-9).
// The scale and the division are float32 operations.
//
// Both kernels are bandwidth-bound.  The quantiser reads a 64x64 tile once and
// writes the codes row-major and, through LDS, transposed, so that every fp8
// GEMM of the forward and the backward reads both operands K-contiguous.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace gdb {

namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// max |x| over n elements: one atomic max per workgroup on the float's bit
// pattern (non-negative floats order like their bits, so the result does not
// depend on the order).
template <typename T>
__global__ __launch_bounds__(256) void amax_k(const T* __restrict__ x, size_t n, unsigned* __restrict__ out) {
  constexpr int VN = V16<T>::n;
  __shared__ float red[4];
  float m = 0.f;
  const size_t nv = n / VN;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < nv; i += (size_t)gridDim.x * 256) {
    float v[VN];
    ld16(x + i * VN, v);
#pragma unroll
    for (int e = 0; e < VN; ++e) m = fmaxf(m, fabsf(v[e]));
  }
  m = block_max<256>(m, red);
  if (threadIdx.x == 0) atomicMax(out, __float_as_uint(m));
}

__global__ void zero_u32_k(unsigned* p) { *p = 0u; }

// e4m3fn code of q (|q| up to a little above 448), round to nearest even.
__device__ __forceinline__ unsigned e4m3_code(float q) {
  const unsigned sign = (__float_as_uint(q) >> 24) & 0x80u;
  const float a = fabsf(q);
  unsigned code;
  if (a >= 0.015625f) {  // normal: keep 3 mantissa bits, ties to even
    unsigned b = __float_as_uint(a);
    b += 0x7FFFFu + ((b >> 20) & 1u);
    b &= 0xFFF00000u;
    b = __float_as_uint(fminf(__uint_as_float(b), 448.0f));
    code = (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);
  } else {  // subnormal step 2^-9; 8 * 2^-9 = 2^-6 has the code 8 as well
    code = (unsigned)rintf(a * 512.0f);
  }
  return sign | code;
}

// Tile of 128 rows x 64 columns, 256 threads.  Thread t quantises 16
// consecutive codes of rows t/4 and 64 + t/4; the transpose goes through LDS
// (one 32-bit word per 4 codes): output row c of the tile gathers its 128
// codes as eight 16-byte pieces, so each transposed row segment is one whole
// 128-byte line written by eight consecutive lanes.
template <typename T>
__global__ __launch_bounds__(256) void quant_k(const T* __restrict__ x, int R, int Cc, const float* __restrict__ amax,
                                                uint8_t* __restrict__ xq, uint8_t* __restrict__ xqt, int Rp) {
  __shared__ unsigned tile[128][17];
  const int r0 = blockIdx.y * 128, c0 = blockIdx.x * 64;
  const int t = threadIdx.x;
  const int cs = (t & 3) * 16, c = c0 + cs;
  const float am = amax[0];
  const float s = am / 448.0f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int rr = (t >> 2) + 64 * h, r = r0 + rr;
    unsigned w[4] = {0u, 0u, 0u, 0u};
    if (r < R && c < Cc && am > 0.f) {
      float v[16];
      if (sizeof(T) == 2) {
        ld16(x + (size_t)r * Cc + c, v);
        ld16(x + (size_t)r * Cc + c + 8, v + 8);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) ld16(x + (size_t)r * Cc + c + 4 * i, v + 4 * i);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int b = 0; b < 4; ++b) w[i] |= e4m3_code(v[4 * i + b] / s) << (8 * b);
    }
    if (xq && r < R && c < Cc) {
      u32x4_t o = {w[0], w[1], w[2], w[3]};
      *(u32x4_t*)(xq + (size_t)r * Cc + c) = o;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) tile[rr][(t & 3) * 4 + i] = w[i];
  }
  if (!xqt) return;  // uniform over the workgroup
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    // piece (t & 7) of output row 32h + t/8: codes of tile rows 16(t&7) .. +15
    const int oc = 32 * h + (t >> 3), rs = 16 * (t & 7);
    const int word = oc >> 2, sh = 8 * (oc & 3);
    unsigned o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      unsigned v = 0u;
#pragma unroll
      for (int b = 0; b < 4; ++b) v |= ((tile[rs + 4 * q + b][word] >> sh) & 0xFFu) << (8 * b);
      o[q] = v;
    }
    const int cc = c0 + oc, rw = r0 + rs;
    if (cc < Cc && rw < Rp) *(u32x4_t*)(xqt + (size_t)cc * Rp + rw) = u32x4_t{o[0], o[1], o[2], o[3]};
  }
}

}  // namespace

hipError_t fp8_amax_zero(float* amax, hipStream_t s) {
  hipLaunchKernelGGL(zero_u32_k, dim3(1), dim3(1), 0, s, (unsigned*)amax);
  return hipGetLastError();
}

hipError_t fp8_amax(int dt, const void* x, size_t n, float* amax, hipStream_t s) {
  hipLaunchKernelGGL(zero_u32_k, dim3(1), dim3(1), 0, s, (unsigned*)amax);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n == 0) return e;
  const size_t nv = n / (dt == BF16 ? 8 : 4);
  const unsigned grid = (unsigned)std::min<size_t>((nv + 255) / 256, 2048);
  if (dt == BF16) hipLaunchKernelGGL(amax_k<bf16>, dim3(grid), dim3(256), 0, s, (const bf16*)x, n, (unsigned*)amax);
  else hipLaunchKernelGGL(amax_k<float>, dim3(grid), dim3(256), 0, s, (const float*)x, n, (unsigned*)amax);
  return hipGetLastError();
}

hipError_t fp8_quant(int dt, const void* x, int R, int Cc, const float* amax, uint8_t* xq, uint8_t* xqt, int Rp,
                     hipStream_t s) {
  const int rows = xqt ? Rp : R;
  if (rows == 0 || Cc == 0) return hipSuccess;
  const dim3 grid((Cc + 63) / 64, (rows + 127) / 128);
  if (dt == BF16) hipLaunchKernelGGL(quant_k<bf16>, grid, dim3(256), 0, s, (const bf16*)x, R, Cc, amax, xq, xqt, Rp);
  else hipLaunchKernelGGL(quant_k<float>, grid, dim3(256), 0, s, (const float*)x, R, Cc, amax, xq, xqt, Rp);
  return hipGetLastError();
}

}  // namespace gdb
