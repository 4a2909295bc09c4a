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
// One workgroup per CU at most (256), each thread with four 16-byte loads in
// flight per iteration: every workgroup ends in an atomic on the one result
// word.  Against 2048 workgroups the amax + quantise of a d26 weight went
// 36.7 -> 17.7 us, of a [32768, 1664] gradient 64.6 -> 46.0 us.
template <typename T>
__global__ __launch_bounds__(256) void amax_k(const T* __restrict__ x, size_t n, unsigned* __restrict__ out) {
  constexpr int VN = V16<T>::n;
  __shared__ float red[4];
  float m = 0.f;
  const size_t nv = n / VN, stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < nv; i += 4 * stride) {
    float v[4][VN];
#pragma unroll
    for (int u = 0; u < 4; ++u) ld16(x + (i + u * stride) * VN, v[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < VN; ++e) m = fmaxf(m, fabsf(v[u][e]));
  }
  for (; i < nv; i += stride) {
    float v[VN];
    ld16(x + i * VN, v);
#pragma unroll
    for (int e = 0; e < VN; ++e) m = fmaxf(m, fabsf(v[e]));
  }
  m = block_max<256>(m, red);
  if (threadIdx.x == 0) atomicMax(out, __float_as_uint(m));
}

__global__ void zero_u32_k(unsigned* p, int n) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0u;
}

// Tile of 128 rows x TC columns (TC = 64 or 128), 256 threads.  Thread t
// quantises 16 consecutive codes of rows t/TPR + (256/TPR)h, TPR = TC/16
// threads per row; the transpose goes through LDS (one 32-bit word per 4
// codes): output row c of the tile gathers its 128 codes as eight 16-byte
// pieces, so each transposed row segment is one whole 128-byte line written
// by eight consecutive lanes.  With TC = 128 the row-major codes of a row are
// one whole line too, and the row's 256 bytes (bf16) are read by 8 threads:
// a [32768, 6656] activation 0.305 -> 0.261 ms (amax pass included); tensors
// with fewer than 2048 such tiles keep TC = 64 for more workgroups.
template <typename T, int TC>
__global__ __launch_bounds__(256) void quant_k(const T* __restrict__ x, int R, int Cc, const float* __restrict__ amax,
                                                uint8_t* __restrict__ xq, uint8_t* __restrict__ xqt, int Rp) {
  constexpr int TPR = TC / 16, RPP = 256 / TPR;  // threads per row, rows per pass
  __shared__ unsigned tile[128][TC / 4 + 1];
  const int r0 = blockIdx.y * 128, c0 = blockIdx.x * TC;
  const int t = threadIdx.x;
  const int cs = (t % TPR) * 16, c = c0 + cs;
  const float am = amax[0];
  const float s = am / 448.0f;
  // The quotient x / s, correctly rounded, from the reciprocal: with
  // y = RN(1/s), q0 = RN(x y) and the exact remainder e = x - q0 s (one FMA),
  // RN(q0 + e y) is RN(x / s) (Markstein's theorem; s normal, so 1/s is
  // finite).  Three operations instead of a full division per element.
  const float y = 1.0f / s;
  const bool recip = s >= 1.17549435e-38f;  // s normal
#pragma unroll
  for (int h = 0; h < 128 / RPP; ++h) {
    const int rr = t / TPR + RPP * h, r = r0 + rr;
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
      float q[16];
      if (recip) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float q0 = v[e] * y;
          q[e] = fmaf(fmaf(-q0, s, v[e]), y, q0);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) q[e] = v[e] / s;
      }
      // codes: the hardware conversion to OCP e4m3fn (3 mantissa bits,
      // exponent bias 7, subnormal step 2^-9, round to nearest even) of the
      // quotient clamped to the largest finite code, 448, which is the
      // saturation.  Checked by probe against a bit-level encoder on every
      // e4m3 value, every midpoint between neighbouring codes and the fp32
      // values on either side of each midpoint.
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float c4[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) c4[b] = fminf(fmaxf(q[4 * i + b], -448.0f), 448.0f);
        int pk = __builtin_amdgcn_cvt_pk_fp8_f32(c4[0], c4[1], 0, false);
        pk = __builtin_amdgcn_cvt_pk_fp8_f32(c4[2], c4[3], pk, true);
        w[i] = (unsigned)pk;
      }
    }
    if (xq && r < R && c < Cc) {
      u32x4_t o = {w[0], w[1], w[2], w[3]};
      *(u32x4_t*)(xq + (size_t)r * Cc + c) = o;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) tile[rr][(t % TPR) * 4 + i] = w[i];
  }
  if (!xqt) return;  // uniform over the workgroup
  __syncthreads();
#pragma unroll
  for (int h = 0; h < TC / 32; ++h) {
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

hipError_t fp8_amax_zero(float* amax, hipStream_t s, int count) {
  hipLaunchKernelGGL(zero_u32_k, dim3(1), dim3(64), 0, s, (unsigned*)amax, count);
  return hipGetLastError();
}

hipError_t fp8_amax(int dt, const void* x, size_t n, float* amax, hipStream_t s, bool zero) {
  if (zero) {
    const hipError_t e = fp8_amax_zero(amax, s);
    if (e != hipSuccess) return e;
  }
  if (n == 0) return hipSuccess;
  const size_t nv = n / (dt == BF16 ? 8 : 4);
  const unsigned grid = (unsigned)std::min<size_t>((nv + 255) / 256, 256);
  if (dt == BF16) hipLaunchKernelGGL(amax_k<bf16>, dim3(grid), dim3(256), 0, s, (const bf16*)x, n, (unsigned*)amax);
  else hipLaunchKernelGGL(amax_k<float>, dim3(grid), dim3(256), 0, s, (const float*)x, n, (unsigned*)amax);
  return hipGetLastError();
}

hipError_t fp8_quant(int dt, const void* x, int R, int Cc, const float* amax, uint8_t* xq, uint8_t* xqt, int Rp,
                     hipStream_t s) {
  const int rows = xqt ? Rp : R;
  if (rows == 0 || Cc == 0) return hipSuccess;
  const size_t wide = (size_t)((Cc + 127) / 128) * ((rows + 127) / 128);
  if (wide >= 2048) {
    const dim3 grid((Cc + 127) / 128, (rows + 127) / 128);
    if (dt == BF16) hipLaunchKernelGGL((quant_k<bf16, 128>), grid, dim3(256), 0, s, (const bf16*)x, R, Cc, amax, xq, xqt, Rp);
    else hipLaunchKernelGGL((quant_k<float, 128>), grid, dim3(256), 0, s, (const float*)x, R, Cc, amax, xq, xqt, Rp);
  } else {
    const dim3 grid((Cc + 63) / 64, (rows + 127) / 128);
    if (dt == BF16) hipLaunchKernelGGL((quant_k<bf16, 64>), grid, dim3(256), 0, s, (const bf16*)x, R, Cc, amax, xq, xqt, Rp);
    else hipLaunchKernelGGL((quant_k<float, 64>), grid, dim3(256), 0, s, (const float*)x, R, Cc, amax, xq, xqt, Rp);
  }
  return hipGetLastError();
}

}  // namespace gdb
