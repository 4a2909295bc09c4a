// Bandwidth-bound kernels: RMSNorm forward/backward, embedding gather/scatter,
// QK RMS-norm + rotary embedding forward/backward, fused softmax cross-entropy,
// deterministic loss and split-K reductions.
//
// Each kernel reads and writes every element once with 16-byte vector
// accesses (rows are multiples of 8 elements); per-row statistics are
// wavefront or workgroup reductions in fp32.
#include "common.h"
#include "kernels.h"

namespace gdb {

// ------------------------------------------------------------------- fill
__global__ __launch_bounds__(256) void fill_f32_k(float* p, size_t n, float v) {
  size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  size_t stride = (size_t)gridDim.x * 256 * 4;
  for (; i + 3 < n; i += stride) {
    f32x4 q = {v, v, v, v};
    *(f32x4*)(p + i) = q;
  }
  if (i < n)
    for (size_t j = i; j < n; ++j) p[j] = v;
}

hipError_t fill_f32(float* p, size_t n, float v, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 1023) / 1024;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_f32_k, dim3((unsigned)blocks), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

// -------------------------------------------------------------- transpose
// out [Cc, R] = in [R, Cc]^T in bf16 (R, Cc multiples of 8), one 64x64 tile
// per workgroup staged in LDS: rows are read and written as 16-byte chunks,
// eight consecutive lanes cover one 128-byte line on both sides.  The
// backward turns each weight into a K-major copy with it, so the data
// gradients run on the GEMM's both-operands-K-major layout.
__global__ __launch_bounds__(256) void transpose_bf16_k(const bf16* __restrict__ in, int R, int Cc,
                                                       bf16* __restrict__ out) {
  __shared__ bf16 t[64][66];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = threadIdx.x + 256 * k, r = i >> 3, cc = (i & 7) * 8;
    if (r0 + r < R && c0 + cc < Cc) {
      const bf16x8 v = *(const bf16x8*)(in + (size_t)(r0 + r) * Cc + c0 + cc);
#pragma unroll
      for (int e = 0; e < 8; ++e) t[r][cc + e] = v[e];
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = threadIdx.x + 256 * k, c = i >> 3, rr = (i & 7) * 8;
    if (c0 + c < Cc && r0 + rr < R) {
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = t[rr + e][c];
      *(bf16x8*)(out + (size_t)(c0 + c) * R + r0 + rr) = v;
    }
  }
}

hipError_t transpose_bf16(const void* in, int R, int Cc, void* out, hipStream_t s) {
  if (R <= 0 || Cc <= 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_bf16_k, dim3((Cc + 63) / 64, (R + 63) / 64), dim3(256), 0, s, (const bf16*)in, R, Cc,
                     (bf16*)out);
  return hipGetLastError();
}

// ---------------------------------------------------------------- RMSNorm
// One wavefront per row; up to MAXV 16-byte vectors per lane stay in registers
// (C <= 64*MAXV*VN), longer rows are streamed twice.
constexpr int RMS_MAXV = 4;
// The norms stream their [N, C] operands once per call, so their register-
// resident rows are read and written with non-temporal accesses: measured on
// the d24 shapes, from a cold cache the forward runs 59 -> 38 us and the
// backward 115 -> 67 us (a 16-byte-vector copy reaches 6.2 TB/s this way
// against 4.7 TB/s without).
template <typename T>
__device__ __forceinline__ void rld16(const T* p, float* o) { ld16_nt(p, o); }
template <typename T>
__device__ __forceinline__ void rst16(T* p, const float* o) { st16_nt(p, o); }

template <typename T>
__device__ __forceinline__ void rmsnorm_row(const T* __restrict__ x, T* __restrict__ xn, float* __restrict__ r,
                                            int row, int l, int C, float eps, float& am) {
  constexpr int VN = V16<T>::n;
  const T* xr = x + (size_t)row * C;
  T* yr = xn + (size_t)row * C;
  const int nv = C / VN;
  float ss = 0.f;
  if (nv <= 64 * RMS_MAXV) {
    float v[RMS_MAXV][VN];
#pragma unroll
    for (int i = 0; i < RMS_MAXV; ++i) {
      const int vi = l + 64 * i;
      if (vi < nv) {
        rld16(xr + vi * VN, v[i]);
#pragma unroll
        for (int e = 0; e < VN; ++e) ss += v[i][e] * v[i][e];
      }
    }
    const float ri = rsqrtf(wave_sum(ss) / (float)C + eps);
#pragma unroll
    for (int i = 0; i < RMS_MAXV; ++i) {
      const int vi = l + 64 * i;
      if (vi < nv) {
#pragma unroll
        for (int e = 0; e < VN; ++e) {
          v[i][e] *= ri;
          am = fmaxf(am, fabsf(v[i][e]));
        }
        rst16(yr + vi * VN, v[i]);
      }
    }
    if (l == 0) r[row] = ri;
  } else {
    for (int vi = l; vi < nv; vi += 64) {
      float v[VN];
      ld16(xr + vi * VN, v);
#pragma unroll
      for (int e = 0; e < VN; ++e) ss += v[e] * v[e];
    }
    const float ri = rsqrtf(wave_sum(ss) / (float)C + eps);
    for (int vi = l; vi < nv; vi += 64) {
      float v[VN];
      ld16(xr + vi * VN, v);
#pragma unroll
      for (int e = 0; e < VN; ++e) {
        v[e] *= ri;
        am = fmaxf(am, fabsf(v[e]));
      }
      st16(yr + vi * VN, v);
    }
    if (l == 0) r[row] = ri;
  }
}

// amax (optional): the largest |xn| stored, one atomic per workgroup
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_fwd_k(const T* __restrict__ x, T* __restrict__ xn,
                                                      float* __restrict__ r, int N, int C, float eps,
                                                      unsigned* __restrict__ amax) {
  __shared__ float red[4];
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
  float am = 0.f;
  if (row < N) rmsnorm_row<T>(x, xn, r, row, l, C, eps, am);
  if (amax) {
    am = block_max<256>(am, red);
    // rounding is monotone: the largest stored value is the rounded largest value
    if (threadIdx.x == 0) atomicMax(amax, __float_as_uint((float)(T)am));
  }
}

template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_bwd_k(const T* __restrict__ dy, const T* __restrict__ y,
                                                      const float* __restrict__ r, const T* dres, T* dx,
                                                      int N, int C) {
  constexpr int VN = V16<T>::n;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
  if (row >= N) return;
  const size_t off = (size_t)row * C;
  const int nv = C / VN;
  const float ri = r[row];
  float dot = 0.f;
  if (nv <= 64 * RMS_MAXV) {
    // the residual gradient is loaded with dy and y, before the reduction,
    // so its latency is not exposed after it
    float g[RMS_MAXV][VN], h[RMS_MAXV][VN], rs[RMS_MAXV][VN];
#pragma unroll
    for (int i = 0; i < RMS_MAXV; ++i) {
      const int vi = l + 64 * i;
      if (vi < nv) {
        rld16(dy + off + vi * VN, g[i]);
        rld16(y + off + vi * VN, h[i]);
        if (dres) rld16(dres + off + vi * VN, rs[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < RMS_MAXV; ++i) {
      const int vi = l + 64 * i;
      if (vi < nv) {
#pragma unroll
        for (int e = 0; e < VN; ++e) dot += g[i][e] * h[i][e];
      }
    }
    const float m = wave_sum(dot) / (float)C;
#pragma unroll
    for (int i = 0; i < RMS_MAXV; ++i) {
      const int vi = l + 64 * i;
      if (vi < nv) {
        float o[VN];
#pragma unroll
        for (int e = 0; e < VN; ++e) o[e] = ri * (g[i][e] - h[i][e] * m) + (dres ? rs[i][e] : 0.f);
        rst16(dx + off + vi * VN, o);
      }
    }
  } else {
    for (int vi = l; vi < nv; vi += 64) {
      float g[VN], h[VN];
      ld16(dy + off + vi * VN, g);
      ld16(y + off + vi * VN, h);
#pragma unroll
      for (int e = 0; e < VN; ++e) dot += g[e] * h[e];
    }
    const float m = wave_sum(dot) / (float)C;
    for (int vi = l; vi < nv; vi += 64) {
      float g[VN], h[VN], o[VN], rs[VN];
      ld16(dy + off + vi * VN, g);
      ld16(y + off + vi * VN, h);
      if (dres) ld16(dres + off + vi * VN, rs);
#pragma unroll
      for (int e = 0; e < VN; ++e) o[e] = ri * (g[e] - h[e] * m) + (dres ? rs[e] : 0.f);
      st16(dx + off + vi * VN, o);
    }
  }
}

hipError_t rmsnorm_fwd(int dt, const void* x, void* xn, float* r, int N, int C, float eps, hipStream_t s,
                       float* amax) {
  if (N == 0) return hipSuccess;
  dim3 g((N + 3) / 4), b(256);
  if (dt == BF16)
    hipLaunchKernelGGL(rmsnorm_fwd_k<bf16>, g, b, 0, s, (const bf16*)x, (bf16*)xn, r, N, C, eps, (unsigned*)amax);
  else
    hipLaunchKernelGGL(rmsnorm_fwd_k<float>, g, b, 0, s, (const float*)x, (float*)xn, r, N, C, eps, (unsigned*)amax);
  return hipGetLastError();
}

hipError_t rmsnorm_bwd(int dt, const void* dxn, const void* xn, const float* r, const void* dres, void* dx,
                       int N, int C, hipStream_t s) {
  if (N == 0) return hipSuccess;
  dim3 g((N + 3) / 4), b(256);
  if (dt == BF16)
    hipLaunchKernelGGL(rmsnorm_bwd_k<bf16>, g, b, 0, s, (const bf16*)dxn, (const bf16*)xn, r,
                       (const bf16*)dres, (bf16*)dx, N, C);
  else
    hipLaunchKernelGGL(rmsnorm_bwd_k<float>, g, b, 0, s, (const float*)dxn, (const float*)xn, r,
                       (const float*)dres, (float*)dx, N, C);
  return hipGetLastError();
}

// ------------------------------------------------------ streaming copy
// The bandwidth reference of the memory-bound kernels: a plain copy of
// 16-byte vectors with non-temporal loads and stores, four vectors in
// flight per thread, grid-stride over the buffer.
__global__ __launch_bounds__(256) void stream_copy_k(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n) {
  constexpr int U = 4;
  const size_t stride = (size_t)gridDim.x * 256 * U;
  for (size_t i = (size_t)blockIdx.x * 256 * U + threadIdx.x; i < n; i += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (i + (size_t)u * 256 < n) v[u] = __builtin_nontemporal_load(src + i + (size_t)u * 256);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (i + (size_t)u * 256 < n) __builtin_nontemporal_store(v[u], dst + i + (size_t)u * 256);
  }
}

// -------------------------------------------------------------- embedding
template <typename T>
__global__ __launch_bounds__(256) void embed_fwd_k(const int32_t* __restrict__ ids, const T* __restrict__ wte,
                                                    T* __restrict__ x, int N, int C, int V) {
  constexpr int VN = V16<T>::n;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
  if (row >= N) return;
  int id = ids[row];
  id = id < 0 ? 0 : (id >= V ? V - 1 : id);
  const T* src = wte + (size_t)id * C;
  T* dst = x + (size_t)row * C;
  for (int vi = l; vi < C / VN; vi += 64) *(uint4*)(dst + vi * VN) = *(const uint4*)(src + vi * VN);
}

// One wave per token; lane l adds columns l, l+64, ... so each atomic
// instruction covers 256 contiguous bytes of the dWte row.
template <typename T>
__global__ __launch_bounds__(256) void embed_bwd_k(const int32_t* __restrict__ ids, const T* __restrict__ dx,
                                                    float* __restrict__ dwte, int N, int C, int V) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
  if (row >= N) return;
  int id = ids[row];
  id = id < 0 ? 0 : (id >= V ? V - 1 : id);
  float* dst = dwte + (size_t)id * C;
  const T* src = dx + (size_t)row * C;
#pragma unroll 4
  for (int c = l; c < C; c += 64) unsafeAtomicAdd(dst + c, to_f(src[c]));
}

hipError_t stream_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 256 * 4 - 1) / (256 * 4);
  hipLaunchKernelGGL(stream_copy_k, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, s,
                     (const u32x4*)src, (u32x4*)dst, n);
  return hipGetLastError();
}

// ------------------------------------------------------------ debug scan
// Flag word of the non-finite scan (one per device, as every __device__
// variable).  The host takes its address with hipGetSymbolAddress.
__device__ unsigned g_nonfinite_flag;

__global__ void nonfinite_clear_k(unsigned* flag) { *flag = 0u; }

// exponent field all ones (NaN or infinity), on the raw bits
template <typename T>
__global__ __launch_bounds__(256) void nonfinite_k(const T* __restrict__ x, size_t n, unsigned* flag) {
  bool bad = false;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    if constexpr (sizeof(T) == 4) {
      bad |= (__float_as_uint(x[i]) & 0x7F800000u) == 0x7F800000u;
    } else {
      bad |= (__builtin_bit_cast(unsigned short, x[i]) & 0x7F80u) == 0x7F80u;
    }
  }
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(flag, 1u);
}

hipError_t any_nonfinite(int dt, const void* x, size_t n, hipStream_t s, bool* bad) {
  *bad = false;
  static unsigned* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!addr[dev]) {
    e = hipGetSymbolAddress((void**)&addr[dev], HIP_SYMBOL(g_nonfinite_flag));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(nonfinite_clear_k, dim3(1), dim3(1), 0, s, addr[dev]);
  if (n) {
    const unsigned grid = (unsigned)std::min<size_t>((n + 255) / 256, 4096);
    if (dt == F32) hipLaunchKernelGGL(nonfinite_k<float>, dim3(grid), dim3(256), 0, s, (const float*)x, n, addr[dev]);
    else hipLaunchKernelGGL(nonfinite_k<bf16>, dim3(grid), dim3(256), 0, s, (const bf16*)x, n, addr[dev]);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  unsigned h = 0;
  if ((e = hipMemcpyAsync(&h, addr[dev], sizeof(h), hipMemcpyDeviceToHost, s)) != hipSuccess) return e;
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;
  *bad = h != 0u;
  return hipSuccess;
}

hipError_t embed_fwd(int dt, const int32_t* ids, const void* wte, void* x, int N, int C, int V, hipStream_t s) {
  if (N == 0) return hipSuccess;
  dim3 g((N + 3) / 4), b(256);
  if (dt == BF16)
    hipLaunchKernelGGL(embed_fwd_k<bf16>, g, b, 0, s, ids, (const bf16*)wte, (bf16*)x, N, C, V);
  else
    hipLaunchKernelGGL(embed_fwd_k<float>, g, b, 0, s, ids, (const float*)wte, (float*)x, N, C, V);
  return hipGetLastError();
}

hipError_t embed_bwd(int dt, const int32_t* ids, const void* dx, float* dwte, int N, int C, int V,
                     int accumulate, hipStream_t s) {
  if (!accumulate) {
    hipError_t e = fill_f32(dwte, (size_t)V * C, 0.f, s);
    if (e != hipSuccess) return e;
  }
  if (N == 0) return hipSuccess;
  dim3 g((N + 3) / 4), b(256);
  if (dt == BF16)
    hipLaunchKernelGGL(embed_bwd_k<bf16>, g, b, 0, s, ids, (const bf16*)dx, dwte, N, C, V);
  else
    hipLaunchKernelGGL(embed_bwd_k<float>, g, b, 0, s, ids, (const float*)dx, dwte, N, C, V);
  return hipGetLastError();
}

// ------------------------------------------------------ QK norm + RoPE
// One workgroup per token row.  A head of D elements is handled by D/2
// threads, thread j holding the rotary pair (j, j + D/2); the head's mean
// square is a reduction over those D/2 lanes.  Then v is copied with 16-byte
// vectors.
template <typename T>
__global__ __launch_bounds__(256) void qk_norm_rope_fwd_k(const T* __restrict__ qkv, T* __restrict__ out,
                                                           float* __restrict__ rinv, const float* __restrict__ rope,
                                                           int T_, int H, int Hkv, int D, float eps) {
  const int row = blockIdx.x;
  const int t = row % T_;
  const int HD = D / 2;
  const int nqk = H + Hkv;
  const int ld = (H + 2 * Hkv) * D;
  const T* src = qkv + (size_t)row * ld;
  T* dst = out + (size_t)row * ld;
  const int heads_per_pass = 256 / HD;
  const int hh = threadIdx.x / HD, j = threadIdx.x % HD;
  const float c = rope[((size_t)t * HD + j) * 2], sn = rope[((size_t)t * HD + j) * 2 + 1];
  for (int h0 = 0; h0 < nqk; h0 += heads_per_pass) {
    const int h = h0 + hh;
    const bool act = h < nqk;
    float a = 0.f, b = 0.f;
    if (act) {
      a = to_f(src[h * D + j]);
      b = to_f(src[h * D + j + HD]);
    }
    float ss = a * a + b * b;
    for (int o = HD / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
    const float r = rsqrtf(ss / (float)D + eps);
    if (act) {
      a *= r;
      b *= r;
      dst[h * D + j] = from_f<T>(a * c - b * sn);
      dst[h * D + j + HD] = from_f<T>(a * sn + b * c);
      if (j == 0) rinv[(size_t)row * nqk + h] = r;
    }
  }
  constexpr int VN = V16<T>::n;
  const int voff = nqk * D, nv = Hkv * D / VN;
  for (int vi = threadIdx.x; vi < nv; vi += 256)
    *(uint4*)(dst + voff + vi * VN) = *(const uint4*)(src + voff + vi * VN);
}

// Backward, one workgroup per token: thread (head, jq) owns the 4 rotary
// pairs (j, j + D/2), j = 4jq .. 4jq+3, read as 4-element vectors.
template <typename T>
__global__ __launch_bounds__(256) void qk_norm_rope_bwd_k(T* d, const T* __restrict__ qkvh,
                                                           const float* __restrict__ rinv,
                                                           const float* __restrict__ rope, int T_, int H,
                                                           int Hkv, int D) {
  typedef T T4 __attribute__((ext_vector_type(4)));
  const int row = blockIdx.x;
  const int t = row % T_;
  const int HD = D / 2, TPH = HD / 4;  // threads per head
  const int nqk = H + Hkv;
  const int ld = (H + 2 * Hkv) * D;
  T* g = d + (size_t)row * ld;
  const T* y = qkvh + (size_t)row * ld;
  const int heads_per_pass = 256 / TPH;
  const int hh = threadIdx.x / TPH, jq = threadIdx.x % TPH, j0 = 4 * jq;
  const f32x4 cs0 = *(const f32x4*)(rope + ((size_t)t * HD + j0) * 2);      // (cos, sin) of j0, j0+1
  const f32x4 cs1 = *(const f32x4*)(rope + ((size_t)t * HD + j0 + 2) * 2);  // (cos, sin) of j0+2, j0+3
  const float c[4] = {cs0[0], cs0[2], cs1[0], cs1[2]}, sn[4] = {cs0[1], cs0[3], cs1[1], cs1[3]};
  for (int h0 = 0; h0 < nqk; h0 += heads_per_pass) {
    const int h = h0 + hh;
    const bool act = h < nqk;
    T4 ga4{}, gb4{}, ya4{}, yb4{};
    if (act) {
      ga4 = *(const T4*)(g + h * D + j0);
      gb4 = *(const T4*)(g + h * D + HD + j0);
      ya4 = *(const T4*)(y + h * D + j0);
      yb4 = *(const T4*)(y + h * D + HD + j0);
    }
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) dot += to_f(ga4[e]) * to_f(ya4[e]) + to_f(gb4[e]) * to_f(yb4[e]);
    for (int o = TPH / 2; o > 0; o >>= 1) dot += __shfl_xor(dot, o, 64);
    const float m = dot / (float)D;
    if (act) {
      const float r = rinv[(size_t)row * nqk + h];
      T4 oa, ob;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ua = to_f(ga4[e]) - to_f(ya4[e]) * m, ub = to_f(gb4[e]) - to_f(yb4[e]) * m;
        // inverse rotation
        oa[e] = from_f<T>(r * (ua * c[e] + ub * sn[e]));
        ob[e] = from_f<T>(r * (-ua * sn[e] + ub * c[e]));
      }
      *(T4*)(g + h * D + j0) = oa;
      *(T4*)(g + h * D + HD + j0) = ob;
    }
  }
}

hipError_t qk_norm_rope_fwd(int dt, const void* qkv, void* qkvh, float* rinv, const float* rope, int B, int T,
                            int H, int Hkv, int D, float eps, hipStream_t s) {
  const int N = B * T;
  if (N == 0) return hipSuccess;
  if (dt == BF16)
    hipLaunchKernelGGL(qk_norm_rope_fwd_k<bf16>, dim3(N), dim3(256), 0, s, (const bf16*)qkv, (bf16*)qkvh, rinv,
                       rope, T, H, Hkv, D, eps);
  else
    hipLaunchKernelGGL(qk_norm_rope_fwd_k<float>, dim3(N), dim3(256), 0, s, (const float*)qkv, (float*)qkvh,
                       rinv, rope, T, H, Hkv, D, eps);
  return hipGetLastError();
}

hipError_t qk_norm_rope_bwd(int dt, void* d, const void* qkvh, const float* rinv, const float* rope, int B,
                            int T, int H, int Hkv, int D, hipStream_t s) {
  const int N = B * T;
  if (N == 0) return hipSuccess;
  if (dt == BF16)
    hipLaunchKernelGGL(qk_norm_rope_bwd_k<bf16>, dim3(N), dim3(256), 0, s, (bf16*)d, (const bf16*)qkvh, rinv,
                       rope, T, H, Hkv, D);
  else
    hipLaunchKernelGGL(qk_norm_rope_bwd_k<float>, dim3(N), dim3(256), 0, s, (float*)d, (const float*)qkvh, rinv,
                       rope, T, H, Hkv, D);
  return hipGetLastError();
}

// ------------------------------------------------------- cross-entropy
// One workgroup per row of logits (256 threads; the bf16 kernel CE_NT).  The row (up to
// 256*CE_MAXV vectors) is read once into registers: max, sum of exp,
// log-sum-exp, then (softmax - onehot)/N is written over the logits.
constexpr int CE_MAXV = 16;
// threads per row of the bf16 kernel (each holds 256 * CE_MAXV / CE_NT vectors)
#ifndef CE_NT
#define CE_NT 512
#endif

template <typename T>
__global__ __launch_bounds__(256) void ce_k(T* z, const int32_t* __restrict__ tgt, float* __restrict__ row_loss,
                                             int N, int V) {
  constexpr int VN = V16<T>::n;
  __shared__ float red[4];
  const int n = blockIdx.x;
  T* zr = z + (size_t)n * V;
  const int nv = V / VN;
  int y = tgt[n];
  y = y < 0 ? 0 : (y >= V ? V - 1 : y);
  const float zy = to_f(zr[y]);
  float v[CE_MAXV][VN];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < CE_MAXV; ++i) {
    const int vi = threadIdx.x + 256 * i;
    if (vi < nv) {
      ld16(zr + vi * VN, v[i]);
#pragma unroll
      for (int e = 0; e < VN; ++e) mx = fmaxf(mx, v[i][e]);
    }
  }
  mx = block_max<256>(mx, red);
  float se = 0.f;
#pragma unroll
  for (int i = 0; i < CE_MAXV; ++i) {
    const int vi = threadIdx.x + 256 * i;
    if (vi < nv) {
#pragma unroll
      for (int e = 0; e < VN; ++e) se += fast_exp(v[i][e] - mx);
    }
  }
  se = block_sum<256>(se, red);
  const float lse = mx + logf(se);
  const float invN = 1.0f / (float)N;
#pragma unroll
  for (int i = 0; i < CE_MAXV; ++i) {
    const int vi = threadIdx.x + 256 * i;
    if (vi < nv) {
      float o[VN];
#pragma unroll
      for (int e = 0; e < VN; ++e) {
        float p = fast_exp(v[i][e] - lse);
        if (vi * VN + e == y) p -= 1.0f;
        o[e] = p * invN;
      }
      st16(zr + vi * VN, o);
    }
  }
  if (threadIdx.x == 0) row_loss[n] = lse - zy;
}


// bf16 logits: the row is kept in registers as its raw bf16 pairs (half the
// registers of fp32 values, so twice the rows per CU hide the memory
// latency) and widened on each of the three uses; the exponentials are taken
// in base 2 on log2(e)-scaled logits.  The logits are read and dz written
// with non-temporal accesses (one pass over 4.3 GB at d24: 0.90 -> 0.82 ms).
template <int NT>
__global__ __launch_bounds__(NT) void ce_bf16_k(bf16* z, const int32_t* __restrict__ tgt,
                                                  float* __restrict__ row_loss, int N, int V) {
  constexpr int MV = CE_MAXV * 256 / NT;  // 16-byte vectors per thread
  __shared__ float red[NT / 64];
  constexpr float L2E = 1.4426950408889634f;
  const int n = blockIdx.x;
  bf16* zr = z + (size_t)n * V;
  const int nv = V / 8;
  int y = tgt[n];
  y = y < 0 ? 0 : (y >= V ? V - 1 : y);
  const float zy = (float)zr[y];
  u32x4 raw[MV];
#pragma unroll
  for (int i = 0; i < MV; ++i) {
    const int vi = threadIdx.x + NT * i;
    raw[i] = vi < nv ? __builtin_nontemporal_load((const u32x4*)(zr + vi * 8))
                     : u32x4{0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
  }
  // bf16 pair -> two floats: the low half shifted up, the high half masked
  auto lo = [](unsigned w) { return __uint_as_float(w << 16); };
  auto hi = [](unsigned w) { return __uint_as_float(w & 0xffff0000u); };
  // the max of each word's two values with the running max in one v_max3:
  // fmaxf on values made by bit operations would first quiet possible NaNs
  // with an extra v_max per value (a finite row has none; a row holding a
  // NaN gives a NaN loss either way)
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < MV; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      asm("v_max3_f32 %0, %1, %2, %3" : "=v"(mx) : "v"(mx), "v"(lo(raw[i][q])), "v"(hi(raw[i][q])));
  mx = block_max<NT>(mx, red);
  // an empty asm marks the raw words as changed, so the widened floats are
  // recomputed in each pass rather than kept live (which would double the
  // registers per row)
#pragma unroll
  for (int i = 0; i < MV; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) asm volatile("" : "+v"(raw[i][q]));
  const float m2 = mx * L2E;
  float se = 0.f;
#pragma unroll
  for (int i = 0; i < MV; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      se += __builtin_amdgcn_exp2f(fmaf(lo(raw[i][q]), L2E, -m2)) + __builtin_amdgcn_exp2f(fmaf(hi(raw[i][q]), L2E, -m2));
  se = block_sum<NT>(se, red);
#pragma unroll
  for (int i = 0; i < MV; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) asm volatile("" : "+v"(raw[i][q]));
  const float lse = mx + logf(se);
  const float l2 = lse * L2E;
  const float invN = 1.0f / (float)N;
  // p/N = 2^(z log2(e) - lse log2(e) - log2(N)): the division by N rides in
  // the exponent (no multiply per element)
  const float l2n = l2 + log2f((float)N);
#pragma unroll
  for (int i = 0; i < MV; ++i) {
    const int vi = threadIdx.x + NT * i;
    if (vi < nv) {
      bf16x8 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        o[2 * q] = (bf16)__builtin_amdgcn_exp2f(fmaf(lo(raw[i][q]), L2E, -l2n));
        o[2 * q + 1] = (bf16)__builtin_amdgcn_exp2f(fmaf(hi(raw[i][q]), L2E, -l2n));
      }
      __builtin_nontemporal_store(o, (bf16x8*)(zr + vi * 8));
    }
  }
  // the target's entry, rewritten by the thread that stored its vector
  if ((y >> 3) % NT == (int)threadIdx.x) zr[y] = (bf16)((__builtin_amdgcn_exp2f(fmaf(zy, L2E, -l2)) - 1.0f) * invN);
  if (threadIdx.x == 0) row_loss[n] = lse - zy;
}

// Rows longer than the register-resident capacity: three streamed passes.
template <typename T>
__global__ __launch_bounds__(256) void ce_long_k(T* z, const int32_t* __restrict__ tgt, float* __restrict__ row_loss,
                                                  int N, int V) {
  constexpr int VN = V16<T>::n;
  __shared__ float red[4];
  const int n = blockIdx.x;
  T* zr = z + (size_t)n * V;
  const int nv = V / VN;
  int y = tgt[n];
  y = y < 0 ? 0 : (y >= V ? V - 1 : y);
  const float zy = to_f(zr[y]);
  float mx = -INFINITY;
  for (int vi = threadIdx.x; vi < nv; vi += 256) {
    float v[VN];
    ld16(zr + vi * VN, v);
    for (int e = 0; e < VN; ++e) mx = fmaxf(mx, v[e]);
  }
  mx = block_max<256>(mx, red);
  float se = 0.f;
  for (int vi = threadIdx.x; vi < nv; vi += 256) {
    float v[VN];
    ld16(zr + vi * VN, v);
    for (int e = 0; e < VN; ++e) se += fast_exp(v[e] - mx);
  }
  se = block_sum<256>(se, red);
  const float lse = mx + logf(se);
  const float invN = 1.0f / (float)N;
  for (int vi = threadIdx.x; vi < nv; vi += 256) {
    float v[VN];
    ld16(zr + vi * VN, v);
    for (int e = 0; e < VN; ++e) {
      float p = fast_exp(v[e] - lse);
      if (vi * VN + e == y) p -= 1.0f;
      v[e] = p * invN;
    }
    st16(zr + vi * VN, v);
  }
  if (threadIdx.x == 0) row_loss[n] = lse - zy;
}

hipError_t ce_fwd_bwd(int dt, void* z, const int32_t* tgt, float* row_loss, int N, int V, hipStream_t s) {
  if (N == 0) return hipSuccess;
  const int vn = dt == BF16 ? 8 : 4;
  const bool fits = V / vn <= 256 * CE_MAXV;
  if (dt == BF16) {
    if (fits) hipLaunchKernelGGL(ce_bf16_k<CE_NT>, dim3(N), dim3(CE_NT), 0, s, (bf16*)z, tgt, row_loss, N, V);
    else hipLaunchKernelGGL(ce_long_k<bf16>, dim3(N), dim3(256), 0, s, (bf16*)z, tgt, row_loss, N, V);
  } else {
    if (fits) hipLaunchKernelGGL(ce_k<float>, dim3(N), dim3(256), 0, s, (float*)z, tgt, row_loss, N, V);
    else hipLaunchKernelGGL(ce_long_k<float>, dim3(N), dim3(256), 0, s, (float*)z, tgt, row_loss, N, V);
  }
  return hipGetLastError();
}

// Deterministic: fixed per-thread strides, fixed reduction tree.
__global__ __launch_bounds__(1024) void loss_reduce_k(const float* __restrict__ row_loss, float* loss, int N) {
  __shared__ float red[16];
  float s = 0.f;
  for (int i = threadIdx.x; i < N; i += 1024) s += row_loss[i];
  s = block_sum<1024>(s, red);
  if (threadIdx.x == 0) loss[0] = N > 0 ? s / (float)N : 0.f;
}

hipError_t loss_reduce(const float* row_loss, float* loss, int N, hipStream_t s) {
  hipLaunchKernelGGL(loss_reduce_k, dim3(1), dim3(1024), 0, s, row_loss, loss, N);
  return hipGetLastError();
}

// ------------------------------------------------------ split-K reduce
__global__ __launch_bounds__(256) void splitk_reduce_k(const float* __restrict__ part, float* __restrict__ C,
                                                        int splits, size_t MN, int accumulate) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= MN) return;  // MN is a multiple of 4 (feature sizes are multiples of 8)
  f32x4 acc = accumulate ? *(const f32x4*)(C + i) : f32x4{0.f, 0.f, 0.f, 0.f};
  for (int z = 0; z < splits; ++z) acc += *(const f32x4*)(part + (size_t)z * MN + i);
  *(f32x4*)(C + i) = acc;
}

// two-phase plan: the slice count depends on the element's tile row or column
__global__ __launch_bounds__(256) void splitk_reduce2_k(const float* __restrict__ part, float* __restrict__ C, int N,
                                                         size_t MN, int splits, int split_cols, int first1,
                                                         int splits2, int accumulate) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= MN) return;  // N is a multiple of 4, so the 4 elements share a row and a 256-column tile
  const size_t m = i / N, n = i - m * N;
  const int t = split_cols ? (int)(n >> 8) : (int)(m >> 8);
  const int ns = t < first1 ? splits : splits2;
  f32x4 acc = accumulate ? *(const f32x4*)(C + i) : f32x4{0.f, 0.f, 0.f, 0.f};
  for (int z = 0; z < ns; ++z) acc += *(const f32x4*)(part + (size_t)z * MN + i);
  *(f32x4*)(C + i) = acc;
}

hipError_t splitk_reduce2(const float* partial, float* C, int M, int N, int splits, int split_cols, int first1,
                          int splits2, int accumulate, hipStream_t s) {
  const size_t MN = (size_t)M * N;
  if (MN == 0) return hipSuccess;
  const size_t blocks = (MN / 4 + 255) / 256;
  hipLaunchKernelGGL(splitk_reduce2_k, dim3((unsigned)blocks), dim3(256), 0, s, partial, C, N, MN, splits, split_cols,
                     first1, splits2, accumulate);
  return hipGetLastError();
}

hipError_t splitk_reduce(const float* partial, float* C, int splits, size_t MN, int accumulate, hipStream_t s) {
  if (MN == 0) return hipSuccess;
  size_t blocks = (MN / 4 + 255) / 256;
  hipLaunchKernelGGL(splitk_reduce_k, dim3((unsigned)blocks), dim3(256), 0, s, partial, C, splits, MN, accumulate);
  return hipGetLastError();
}

}  // namespace gdb
