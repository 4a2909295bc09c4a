// Optimizer step after the backward, as the Japanese and French articles
// describe it (section "2. Muonオプティマイザー" / "2. L'optimiseur Muon"):
// AdamW for embeddings, lm_head and scalars; for matrices Muon, momentum
// orthogonalised by the Polar Express Newton-Schulz loop
//   A = X^T X;  B = b A + c A^2;  X = a X + X B.
// The loop's three products run on the MFMA GEMM: the Gram (a long
// contraction onto a small output) split over K into fp32 partials that one
// pass adds and casts, the other two with the axpy in the GEMM's epilogue.
// This file holds that pass and the bandwidth kernels around the products:
// the Frobenius norm that scales the loop's input, the momentum update, the
// parameter update and AdamW.  Reductions are deterministic: fixed grids
// write one partial per workgroup, one workgroup adds them in order.
#include "common.h"
#include "kernels.h"

namespace gdb {

namespace {

constexpr int OPT_NT = 256;

// per-workgroup sums of squares of x [n] (n a multiple of 4)
__device__ __forceinline__ float sumsq4(f32x4 v) { return v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3]; }

// item blockIdx.y of a stack of matrices of n4*4 elements each; partials at
// part[item * OPT_PART + block]
__global__ __launch_bounds__(OPT_NT) void sumsq_part_k(const float* __restrict__ x, size_t n4, float* part) {
  __shared__ float red[OPT_NT / 64];
  x += (size_t)blockIdx.y * n4 * 4;
  part += (size_t)blockIdx.y * OPT_PART;
  float acc = 0.f;
  for (size_t i = (size_t)blockIdx.x * OPT_NT + threadIdx.x; i < n4; i += (size_t)gridDim.x * OPT_NT)
    acc += sumsq4(((const f32x4*)x)[i]);
  acc = block_sum<OPT_NT>(acc, red);
  if (threadIdx.x == 0) part[blockIdx.x] = acc;
}

// momentum: buf = mu*buf + g; u = nesterov ? g + mu*buf : buf; partial sums of u^2
__global__ __launch_bounds__(OPT_NT) void muon_momentum_k(const float* __restrict__ g, float* __restrict__ buf,
                                                         float* __restrict__ u, size_t n4, float mu, int nesterov,
                                                         float* part) {
  __shared__ float red[OPT_NT / 64];
  const size_t off = (size_t)blockIdx.y * n4 * 4;
  g += off; buf += off; u += off;
  part += (size_t)blockIdx.y * OPT_PART;
  float acc = 0.f;
  for (size_t i = (size_t)blockIdx.x * OPT_NT + threadIdx.x; i < n4; i += (size_t)gridDim.x * OPT_NT) {
    const f32x4 gv = ((const f32x4*)g)[i];
    const f32x4 b = mu * ((const f32x4*)buf)[i] + gv;
    ((f32x4*)buf)[i] = b;
    const f32x4 uv = nesterov ? gv + mu * b : b;
    ((f32x4*)u)[i] = uv;
    acc += sumsq4(uv);
  }
  acc = block_sum<OPT_NT>(acc, red);
  if (threadIdx.x == 0) part[blockIdx.x] = acc;
}

// inv[item] = 1 / (sqrt(sum of the item's partials) * norm_scale + eps), item =
// blockIdx.x; thread t adds partials t, t + 256, ... then a fixed tree
__global__ __launch_bounds__(OPT_NT) void norm_final_k(const float* part, int np, float norm_scale, float eps,
                                                       float* inv) {
  __shared__ float red[OPT_NT / 64];
  part += (size_t)blockIdx.x * OPT_PART;
  float acc = 0.f;
  for (int i = threadIdx.x; i < np; i += OPT_NT) acc += part[i];
  acc = block_sum<OPT_NT>(acc, red);
  if (threadIdx.x == 0) inv[blockIdx.x] = 1.0f / (sqrtf(acc) * norm_scale + eps);
}

// x0 = g * inv[item] in the iteration's dtype, item = blockIdx.y
template <typename T>
__global__ __launch_bounds__(OPT_NT) void scale_cast_k(const float* __restrict__ g, const float* inv,
                                                      T* __restrict__ x, size_t n4) {
  const float sc = inv[blockIdx.y];
  g += (size_t)blockIdx.y * n4 * 4;
  x += (size_t)blockIdx.y * n4 * 4;
  for (size_t i = (size_t)blockIdx.x * OPT_NT + threadIdx.x; i < n4; i += (size_t)gridDim.x * OPT_NT) {
    const f32x4 v = ((const f32x4*)g)[i] * sc;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[4 * i + e] = from_f<T>(v[e]);
  }
}

// out = alpha * (sum of split-K partials) + beta * R, in the iteration's dtype
// (R of that dtype, or null): the three lines of the Newton-Schulz loop
template <typename T>
__global__ __launch_bounds__(OPT_NT) void splitk_axpby_k(const float* __restrict__ part, int splits, size_t n4,
                                                        float alpha, float beta, const T* __restrict__ R,
                                                        T* __restrict__ out) {
  for (size_t i = (size_t)blockIdx.x * OPT_NT + threadIdx.x; i < n4; i += (size_t)gridDim.x * OPT_NT) {
    f32x4 acc = ((const f32x4*)part)[i];
    for (int z = 1; z < splits; ++z) acc += ((const f32x4*)(part + (size_t)z * n4 * 4))[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v = alpha * acc[e];
      if (R) v = fmaf(beta, to_f(R[4 * i + e]), v);
      out[4 * i + e] = from_f<T>(v);
    }
  }
}

// p = p*(1 - lr*wd) - lr*scale*x; optional low-precision copy of p
template <typename T>
__global__ __launch_bounds__(OPT_NT) void muon_apply_k(float* __restrict__ p, const T* __restrict__ x,
                                                      bf16* __restrict__ plow, size_t n4, float decay, float step) {
  for (size_t i = (size_t)blockIdx.x * OPT_NT + threadIdx.x; i < n4; i += (size_t)gridDim.x * OPT_NT) {
    f32x4 pv = ((f32x4*)p)[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) pv[e] = pv[e] * decay - step * to_f(x[4 * i + e]);
    ((f32x4*)p)[i] = pv;
    if (plow) {
#pragma unroll
      for (int e = 0; e < 4; ++e) plow[4 * i + e] = (bf16)pv[e];
    }
  }
}

// NorMuon row statistics: one wavefront per row r of the stacked NS output x
// ([rows][n]): vmean = mean of x^2 over the row, then the per-neuron second
// moment v = beta2*v + (1 - beta2)*vmean and step = 1/sqrt(max(v, 1e-10)).
template <typename T>
__global__ __launch_bounds__(256) void normuon_rows_k(const T* __restrict__ x, size_t rows, int n,
                                                      float* __restrict__ v, float beta2, float* __restrict__ vmean,
                                                      float* __restrict__ step) {
  constexpr int VN = V16<T>::n;
  const size_t r = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (r >= rows) return;  // wave-uniform
  const T* xr = x + r * n;
  float acc = 0.f;
  for (int c = l * VN; c < n; c += 64 * VN) {
    float a[VN];
    ld16(xr + c, a);
#pragma unroll
    for (int e = 0; e < VN; ++e) acc += a[e] * a[e];
  }
  acc = wave_sum(acc);
  if (l == 0) {
    const float vm = acc / (float)n;
    const float vv = beta2 * v[r] + (1.0f - beta2) * vm;
    v[r] = vv;
    vmean[r] = vm;
    step[r] = 1.0f / sqrtf(fmaxf(vv, 1e-10f));
  }
}

// One workgroup per item: v_norm = sqrt(sum vmean), v_norm_new =
// sqrt(sum vmean*step^2) over the item's m rows (fixed order), then the row
// factors fs = step * v_norm / max(v_norm_new, 1e-10).
__global__ __launch_bounds__(OPT_NT) void normuon_final_k(const float* __restrict__ vmean,
                                                          const float* __restrict__ step, int m,
                                                          float* __restrict__ fs) {
  __shared__ float red[OPT_NT / 64];
  const size_t o = (size_t)blockIdx.x * m;
  float a = 0.f, b = 0.f;
  for (int r = threadIdx.x; r < m; r += OPT_NT) {
    const float vm = vmean[o + r], st = step[o + r];
    a += vm;
    b += vm * st * st;
  }
  a = block_sum<OPT_NT>(a, red);
  b = block_sum<OPT_NT>(b, red);
  const float ratio = sqrtf(a) / fmaxf(sqrtf(b), 1e-10f);
  for (int r = threadIdx.x; r < m; r += OPT_NT) fs[o + r] = step[o + r] * ratio;
}

// p = p*decay - step*fs[row]*x, rows of n elements; optional bf16 copy of p
template <typename T>
__global__ __launch_bounds__(OPT_NT) void normuon_apply_k(float* __restrict__ p, const T* __restrict__ x,
                                                          const float* __restrict__ fs, bf16* __restrict__ plow,
                                                          size_t n4, int n, float decay, float step) {
  for (size_t i = (size_t)blockIdx.x * OPT_NT + threadIdx.x; i < n4; i += (size_t)gridDim.x * OPT_NT) {
    const float f = step * fs[(4 * i) / n];  // n is a multiple of 4: the 4 elements share a row
    f32x4 pv = ((f32x4*)p)[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) pv[e] = pv[e] * decay - f * to_f(x[4 * i + e]);
    ((f32x4*)p)[i] = pv;
    if (plow) {
#pragma unroll
      for (int e = 0; e < 4; ++e) plow[4 * i + e] = (bf16)pv[e];
    }
  }
}

// AdamW with bias correction: rc1 = 1/(1 - beta1^t), rc2 = 1/(1 - beta2^t)
__global__ __launch_bounds__(OPT_NT) void adamw_k(float* __restrict__ p, const float* __restrict__ g,
                                                 float* __restrict__ m, float* __restrict__ v,
                                                 bf16* __restrict__ plow, size_t n4, float lr, float b1, float b2,
                                                 float eps, float decay, float rc1, float rc2) {
  for (size_t i = (size_t)blockIdx.x * OPT_NT + threadIdx.x; i < n4; i += (size_t)gridDim.x * OPT_NT) {
    // every operand is streamed once: non-temporal accesses
    const f32x4 gv = __builtin_nontemporal_load((const f32x4*)g + i);
    f32x4 pv = __builtin_nontemporal_load((const f32x4*)p + i), mv = __builtin_nontemporal_load((const f32x4*)m + i),
          vv = __builtin_nontemporal_load((const f32x4*)v + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mv[e] = b1 * mv[e] + (1.0f - b1) * gv[e];
      vv[e] = b2 * vv[e] + (1.0f - b2) * gv[e] * gv[e];
      pv[e] = pv[e] * decay - lr * (mv[e] * rc1) / (sqrtf(vv[e] * rc2) + eps);
    }
    __builtin_nontemporal_store(pv, (f32x4*)p + i);
    __builtin_nontemporal_store(mv, (f32x4*)m + i);
    __builtin_nontemporal_store(vv, (f32x4*)v + i);
    if (plow) {
#pragma unroll
      for (int e = 0; e < 4; ++e) plow[4 * i + e] = (bf16)pv[e];
    }
  }
}

unsigned grid_for(size_t n4) {
  const size_t b = (n4 + OPT_NT - 1) / OPT_NT;
  return (unsigned)(b < (size_t)OPT_PART ? (b ? b : 1) : (size_t)OPT_PART);
}

}  // namespace

hipError_t sumsq_partials(const float* x, size_t n, int count, float* part, int* np, hipStream_t s) {
  *np = (int)grid_for(n / 4);
  hipLaunchKernelGGL(sumsq_part_k, dim3(*np, count), dim3(OPT_NT), 0, s, x, n / 4, part);
  return hipGetLastError();
}

hipError_t muon_momentum(const float* g, float* buf, float* u, size_t n, int count, float mu, int nesterov,
                         float* part, int* np, hipStream_t s) {
  *np = (int)grid_for(n / 4);
  hipLaunchKernelGGL(muon_momentum_k, dim3(*np, count), dim3(OPT_NT), 0, s, g, buf, u, n / 4, mu, nesterov, part);
  return hipGetLastError();
}

hipError_t norm_final(const float* part, int np, int count, float norm_scale, float eps, float* inv, hipStream_t s) {
  hipLaunchKernelGGL(norm_final_k, dim3(count), dim3(OPT_NT), 0, s, part, np, norm_scale, eps, inv);
  return hipGetLastError();
}

hipError_t scale_cast(int dt, const float* g, const float* inv, void* x, size_t n, int count, hipStream_t s) {
  const dim3 grid(grid_for(n / 4), count);
  if (dt == BF16) hipLaunchKernelGGL(scale_cast_k<bf16>, grid, dim3(OPT_NT), 0, s, g, inv, (bf16*)x, n / 4);
  else hipLaunchKernelGGL(scale_cast_k<float>, grid, dim3(OPT_NT), 0, s, g, inv, (float*)x, n / 4);
  return hipGetLastError();
}

hipError_t splitk_axpby(int dt, const float* part, int splits, size_t n, float alpha, float beta, const void* R,
                        void* out, hipStream_t s) {
  if (dt == BF16)
    hipLaunchKernelGGL(splitk_axpby_k<bf16>, dim3(grid_for(n / 4)), dim3(OPT_NT), 0, s, part, splits, n / 4, alpha,
                       beta, (const bf16*)R, (bf16*)out);
  else
    hipLaunchKernelGGL(splitk_axpby_k<float>, dim3(grid_for(n / 4)), dim3(OPT_NT), 0, s, part, splits, n / 4, alpha,
                       beta, (const float*)R, (float*)out);
  return hipGetLastError();
}

hipError_t muon_apply(int dt, float* p, const void* x, bf16* plow, size_t n, float decay, float step, hipStream_t s) {
  if (dt == BF16)
    hipLaunchKernelGGL(muon_apply_k<bf16>, dim3(grid_for(n / 4)), dim3(OPT_NT), 0, s, p, (const bf16*)x, plow, n / 4,
                       decay, step);
  else
    hipLaunchKernelGGL(muon_apply_k<float>, dim3(grid_for(n / 4)), dim3(OPT_NT), 0, s, p, (const float*)x, plow,
                       n / 4, decay, step);
  return hipGetLastError();
}

hipError_t normuon_scale(int dt, const void* x, int count, int m, int n, float* v, float beta2, float* stat, float* fs,
                         hipStream_t s) {
  const size_t rows = (size_t)count * m;
  float* vmean = stat;
  float* step = stat + rows;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (dt == BF16)
    hipLaunchKernelGGL(normuon_rows_k<bf16>, grid, dim3(256), 0, s, (const bf16*)x, rows, n, v, beta2, vmean, step);
  else
    hipLaunchKernelGGL(normuon_rows_k<float>, grid, dim3(256), 0, s, (const float*)x, rows, n, v, beta2, vmean, step);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(normuon_final_k, dim3(count), dim3(OPT_NT), 0, s, vmean, step, m, fs);
  return hipGetLastError();
}

hipError_t normuon_apply(int dt, float* p, const void* x, const float* fs, bf16* plow, size_t rows, int n, float decay,
                         float step, hipStream_t s) {
  const size_t n4 = rows * n / 4;
  if (dt == BF16)
    hipLaunchKernelGGL(normuon_apply_k<bf16>, dim3(grid_for(n4)), dim3(OPT_NT), 0, s, p, (const bf16*)x, fs, plow, n4,
                       n, decay, step);
  else
    hipLaunchKernelGGL(normuon_apply_k<float>, dim3(grid_for(n4)), dim3(OPT_NT), 0, s, p, (const float*)x, fs, plow,
                       n4, n, decay, step);
  return hipGetLastError();
}

hipError_t adamw(float* p, const float* g, float* m, float* v, bf16* plow, size_t n, float lr, float b1, float b2,
                 float eps, float wd, int t, hipStream_t s) {
  const float rc1 = (float)(1.0 / (1.0 - std::pow((double)b1, (double)t)));
  const float rc2 = (float)(1.0 / (1.0 - std::pow((double)b2, (double)t)));
  hipLaunchKernelGGL(adamw_k, dim3(grid_for(n / 4)), dim3(OPT_NT), 0, s, p, g, m, v, plow, n / 4, lr, b1, b2, eps,
                     1.0f - lr * wd, rc1, rc2);
  return hipGetLastError();
}

}  // namespace gdb
