// The extras of the largest model in "Comment Entraîner Votre Propre ChatGPT
// Pour 50€ ?", section "1. Le modèle GPT (nanochat/gpt.py)": per-layer residual
// mixing x <- a*x + b*x0, value embeddings added to V through a per-head
// sigmoid gate, smear (the previous token's embedding mixed in through a gate
// on the first channels) and backout (a scaled mid-stack residual subtracted
// before the head).
//
// All of it is bandwidth-bound: one wavefront per token row, 16-byte accesses,
// fp32 arithmetic.  Gradients of the scalars and small parameters are reduced
// deterministically: each workgroup writes a partial sum, then one workgroup
// adds the partials in a fixed order.  Kernels that produce partials run a
// grid-stride loop over rows with at most EXTRA_PBLK workgroups, so their
// partial buffers have a fixed bound.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace gdb {

namespace {

__device__ __forceinline__ float sigm(float x) { return 1.0f / (1.0f + __expf(-x)); }

// g[0..VN) += p[0..VN) for an fp32 addend chunk (16-byte aligned).
template <int VN>
__device__ __forceinline__ void add_f32(const float* __restrict__ p, float* g) {
#pragma unroll
  for (int e = 0; e < VN; e += 4) {
    const f32x4 q = *(const f32x4*)(p + e);
    g[e] += q[0]; g[e + 1] += q[1]; g[e + 2] += q[2]; g[e + 3] += q[3];
  }
}

// out(k) (+)= sum over workgroups i of part[i*K + k], added in a fixed order;
// out(0) is out0[0], out(k > 0) is out1[k-1].  One workgroup.
__global__ __launch_bounds__(256) void reduce_cols_k(const float* __restrict__ part, int nblk, int K,
                                                      float* out0, float* out1, int accumulate) {
  __shared__ float red[4];
  for (int k = 0; k < K; ++k) {
    float s = 0.f;
    for (int i = threadIdx.x; i < nblk; i += 256) s += part[(size_t)i * K + k];
    s = block_sum<256>(s, red);
    if (threadIdx.x == 0) {
      float* o = k == 0 ? out0 : out1 + (k - 1);
      *o = accumulate ? *o + s : s;
    }
  }
}

// The same sums for many columns (the value-embedding gate's Hkv*nc): a
// workgroup of 16 waves per 64 columns, lane = column, so every partial row
// is read as whole 256-byte segments; wave w adds rows w, w + 16, w + 32, ...
// in that order (eight loads in flight), then the 16 wave sums are added in
// wave order.  One workgroup walking the columns one at a time took ~260 us
// for the d26 gate's 416 columns of 512 partials.
__global__ __launch_bounds__(1024) void reduce_cols_wide_k(const float* __restrict__ part, int nblk, int K,
                                                           float* out0, float* out1, int accumulate) {
  __shared__ float red[16][64];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int k = blockIdx.x * 64 + l;
  const int kc = k < K ? k : K - 1;  // lanes past the last column read a valid one and store nothing
  float s = 0.f;
  for (int i0 = w; i0 < nblk; i0 += 16 * 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + 16 * u;
      v[u] = i < nblk ? part[(size_t)i * K + kc] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  red[w][l] = s;
  __syncthreads();
  if (w == 0 && k < K) {
    float t = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) t += red[j][l];
    float* o = k == 0 ? out0 : out1 + (k - 1);
    *o = accumulate ? *o + t : t;
  }
}

hipError_t reduce_cols(const float* part, int nblk, int K, float* out0, float* out1, int accumulate, hipStream_t s) {
  if (K > 8)
    hipLaunchKernelGGL(reduce_cols_wide_k, dim3((K + 63) / 64), dim3(1024), 0, s, part, nblk, K, out0, out1,
                       accumulate);
  else
    hipLaunchKernelGGL(reduce_cols_k, dim3(1), dim3(256), 0, s, part, nblk, K, out0, out1, accumulate);
  return hipGetLastError();
}

// ------------------------------------------------------------------- mixing
// y = lam[0]*x + lam[1]*x0 over n elements (n a multiple of the vector width).
template <typename T>
__global__ __launch_bounds__(256) void mix_fwd_k(const T* __restrict__ x, const T* __restrict__ x0,
                                                  const float* __restrict__ lam, T* __restrict__ y, size_t n) {
  constexpr int VN = V16<T>::n;
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * VN;
  if (i >= n) return;
  const float a = lam[0], b = lam[1];
  float u[VN], v[VN];
  ld16(x + i, u);
  ld16(x0 + i, v);
#pragma unroll
  for (int e = 0; e < VN; ++e) u[e] = a * u[e] + b * v[e];
  st16(y + i, u);
}

// dy is the gradient w.r.t. the mixed stream:
//   dx = a*dy (dx may alias dy);  dx0 = (acc ? dx0 : 0) + b*dy  (fp32);
//   per-workgroup partials of sum(dy*x) and sum(dy*x0).
template <typename T>
__global__ __launch_bounds__(256) void mix_bwd_k(const T* dy, const T* __restrict__ x, const T* __restrict__ x0,
                                                  const float* __restrict__ lam, T* dx, float* __restrict__ dx0,
                                                  int acc_dx0, float* __restrict__ part, int N, int C) {
  constexpr int VN = V16<T>::n;
  __shared__ float red[2][4];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const float a = lam[0], b = lam[1];
  float sa = 0.f, sb = 0.f;
  for (int row = blockIdx.x * 4 + w; row < N; row += gridDim.x * 4) {
    const size_t off = (size_t)row * C;
    for (int vi = l; vi < C / VN; vi += 64) {
      const size_t o = off + (size_t)vi * VN;
      float g[VN], u[VN], z[VN], d0[VN];
      ld16(dy + o, g);
      ld16(x + o, u);
      ld16(x0 + o, z);
#pragma unroll
      for (int e = 0; e < VN; ++e) d0[e] = 0.f;
      if (acc_dx0) add_f32<VN>(dx0 + o, d0);
#pragma unroll
      for (int e = 0; e < VN; ++e) {
        sa += g[e] * u[e];
        sb += g[e] * z[e];
        d0[e] += b * g[e];
        g[e] *= a;
      }
      st16(dx + o, g);
#pragma unroll
      for (int e = 0; e < VN; e += 4) *(f32x4*)(dx0 + o + e) = f32x4{d0[e], d0[e + 1], d0[e + 2], d0[e + 3]};
    }
  }
  sa = wave_sum(sa);
  sb = wave_sum(sb);
  if (l == 0) { red[0][w] = sa; red[1][w] = sb; }
  __syncthreads();
  if (threadIdx.x == 0) {
    part[blockIdx.x * 2] = red[0][0] + red[0][1] + red[0][2] + red[0][3];
    part[blockIdx.x * 2 + 1] = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  }
}

// ------------------------------------------------------- value embeddings
// One wave per token n.  s_g = xn[n, :nc] . Wg[g, :];  gate_g = 3*sigmoid(s_g);
// v[n, g, :] += gate_g * VE[ids[n], g, :], in place on the raw qkv row (the v
// columns start at voff).  s is saved for the backward; lane g holds s_g.
template <typename T>
__global__ __launch_bounds__(256) void ve_fwd_k(T* qkv, int ldq, int voff, const T* __restrict__ xn, int C,
                                                 const int32_t* __restrict__ ids, const T* __restrict__ ve,
                                                 const T* __restrict__ wg, int nc, int Hkv, int D, int V,
                                                 float* __restrict__ s_save, int N) {
  constexpr int VN = V16<T>::n;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + w;
  if (n >= N) return;  // wave-uniform
  int id = ids[n];
  id = id < 0 ? 0 : (id >= V ? V - 1 : id);
  // gate logits: lane l takes head g0 + l/LP and channels 8(l % LP) .. +7 of
  // the nc, the LP lanes of a head are summed by a butterfly, and lane g ends
  // with s_g (LP = 4 for nc = 32: all 16 heads of a pass at once, where one
  // 64-lane sum per head took Hkv six-step butterflies)
  const int LP = nc <= 8 ? 1 : nc <= 16 ? 2 : nc <= 32 ? 4 : 8, HPP = 64 / LP;
  float s_mine = 0.f;
  for (int g0 = 0; g0 < Hkv; g0 += HPP) {
    const int g = g0 + l / LP, c0 = 8 * (l % LP);
    float acc = 0.f;
    if (g < Hkv) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (c0 + i < nc) acc += to_f(xn[(size_t)n * C + c0 + i]) * to_f(wg[g * nc + c0 + i]);
    }
    for (int o = LP / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    const int j = l - g0;  // lane l takes head l's sum, held by lane (l - g0) * LP
    const bool mine = j >= 0 && j < HPP;
    const float sj = __shfl(acc, (mine ? j : 0) * LP, 64);
    if (mine) s_mine = sj;
  }
  if (l < Hkv) s_save[(size_t)n * Hkv + l] = s_mine;
  const float gate_mine = 3.0f * sigm(s_mine);
  T* vrow = qkv + (size_t)n * ldq + voff;
  const T* erow = ve + (size_t)id * Hkv * D;
  const int G = D / VN;  // lanes per head
  const int nchunk = Hkv * G;
  for (int base = 0; base < nchunk; base += 64) {  // same trip count on every lane: the shuffle sees all of them
    const int ci = base + l;
    const float gate = __shfl(gate_mine, min(ci / G, Hkv - 1), 64);
    if (ci < nchunk) {
      float a[VN], e[VN];
      ld16(vrow + ci * VN, a);
      ld16(erow + ci * VN, e);
#pragma unroll
      for (int q = 0; q < VN; ++q) a[q] += gate * e[q];
      st16(vrow + ci * VN, a);
    }
  }
}

// One wave per token n; dv = the v columns of dqkv (the addition passes the
// gradient to v unchanged):
//   dgate_g = dv[n,g,:] . VE[id,g,:];  ds[n,g] = dgate_g * 3*sig(s)*(1 - sig(s));
//   dVE[id,g,:] += gate_g * dv[n,g,:]  (fp32 atomics: ids repeat; skipped when
//   dve is null, the deterministic path sums the rows in a fixed order instead).
// Lane l takes columns l, l+64, ... of each head, so one atomic instruction
// covers 256 contiguous bytes (two cache lines) of the dVE row; dgate_g is a
// butterfly over the wave.
template <typename T>
__global__ __launch_bounds__(256) void ve_bwd_k(const T* __restrict__ dqkv, int ldq, int voff,
                                                 const int32_t* __restrict__ ids, const T* __restrict__ ve,
                                                 const float* __restrict__ s_save, int Hkv, int D, int V,
                                                 float* __restrict__ ds, float* __restrict__ dve, int N) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + w;
  if (n >= N) return;  // wave-uniform
  int id = ids[n];
  id = id < 0 ? 0 : (id >= V ? V - 1 : id);
  const float sg_mine = sigm(l < Hkv ? s_save[(size_t)n * Hkv + l] : 0.f);
  const float gate_mine = 3.0f * sg_mine;
  const T* dv = dqkv + (size_t)n * ldq + voff;
  const T* erow = ve + (size_t)id * Hkv * D;
  float* drow = dve ? dve + (size_t)id * Hkv * D : nullptr;
  float dg_mine = 0.f;
  for (int h = 0; h < Hkv; ++h) {
    const float gate = __shfl(gate_mine, h, 64);
    float p = 0.f;
#pragma unroll 2
    for (int c = h * D + l; c < (h + 1) * D; c += 64) {
      const float g = to_f(dv[c]);
      p += g * to_f(erow[c]);
      if (drow) unsafeAtomicAdd(drow + c, gate * g);  // kernel-argument test: uniform
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) p += __shfl_xor(p, o, 64);
    if (l == h) dg_mine = p;
  }
  if (l < Hkv) ds[(size_t)n * Hkv + l] = dg_mine * 3.0f * sg_mine * (1.0f - sg_mine);
}

// dxn[n, :nc] += ds[n, :] @ Wg (in place) and per-workgroup partials of
// dWg[g, c] = sum_n ds[n, g] * xn[n, c] over the workgroup's 64 tokens.
template <typename T>
__global__ __launch_bounds__(256) void ve_gate_bwd_k(const float* __restrict__ ds, const T* __restrict__ xn, T* dxn,
                                                      int C, const T* __restrict__ wg, int nc, int Hkv,
                                                      float* __restrict__ part, int N) {
  // the block's 64 rows of ds and of xn's first nc channels, and wg, are
  // staged in LDS with coalesced loads; the sums below then read LDS only
  // (the same products added in the same order as from memory)
  __shared__ float ds_s[64][65], xn_s[64][65], wg_s[64][65];
  const int n0 = blockIdx.x * 64, n1 = min(N, n0 + 64), nn = n1 - n0;
  for (int e = threadIdx.x; e < nn * Hkv; e += 256) ds_s[e / Hkv][e % Hkv] = ds[(size_t)n0 * Hkv + e];
  for (int e = threadIdx.x; e < nn * nc; e += 256) xn_s[e / nc][e % nc] = to_f(xn[(size_t)(n0 + e / nc) * C + e % nc]);
  for (int e = threadIdx.x; e < Hkv * nc; e += 256) wg_s[e / nc][e % nc] = to_f(wg[e]);
  __syncthreads();
  for (int e = threadIdx.x; e < nn * nc; e += 256) {
    const int r = e / nc, c = e % nc;
    float acc = 0.f;
    for (int g = 0; g < Hkv; ++g) acc += ds_s[r][g] * wg_s[g][c];
    T* p = dxn + (size_t)(n0 + r) * C + c;
    *p = from_f<T>(to_f(*p) + acc);
  }
  for (int e = threadIdx.x; e < Hkv * nc; e += 256) {
    const int g = e / nc, c = e % nc;
    float acc = 0.f;
    for (int r = 0; r < nn; ++r) acc += ds_s[r][g] * xn_s[r][c];
    part[(size_t)blockIdx.x * Hkv * nc + e] = acc;
  }
}

// --------------------------------------------------------------------- smear
// One wave per token (b, t): s = e[t, :ng] . w;  x[t] = e[t] + lam*sigmoid(s)*e[t-1]
// for t >= 1 and x[0] = e[0].  s is saved for the backward.
template <typename T>
__global__ __launch_bounds__(256) void smear_fwd_k(const T* __restrict__ e, const T* __restrict__ wgt, int ng,
                                                    const float* __restrict__ lam, T* __restrict__ x,
                                                    float* __restrict__ s_save, int N, int T_, int C) {
  constexpr int VN = V16<T>::n;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + w;
  if (n >= N) return;  // wave-uniform
  const int t = n % T_;
  const T* er = e + (size_t)n * C;
  const float s = wave_sum(l < ng ? to_f(er[l]) * to_f(wgt[l]) : 0.f);
  if (l == 0) s_save[n] = s;
  const float gate = t >= 1 ? lam[0] * sigm(s) : 0.f;
  const T* ep = t >= 1 ? er - C : er;
  for (int vi = l; vi < C / VN; vi += 64) {
    float a[VN], b[VN];
    ld16(er + vi * VN, a);
    ld16(ep + vi * VN, b);
#pragma unroll
    for (int q = 0; q < VN; ++q) a[q] += gate * b[q];
    st16(x + (size_t)n * C + vi * VN, a);
  }
}

// g = dx + dxa (dxa an optional fp32 addend) is the gradient w.r.t. x:
//   de[t] = g[t] + gate[t+1]*g[t+1];  dgate[t] = g[t] . e[t-1] (t >= 1, else 0);
//   ds = lam*sig'(s_t)*dgate;  de[t, :ng] += ds*w;
//   per-workgroup partials: dlam = sum sig(s_t)*dgate, dw[c] = sum ds*e[t, c].
template <typename T>
__global__ __launch_bounds__(256) void smear_bwd_k(const T* __restrict__ e, const T* __restrict__ wgt, int ng,
                                                    const float* __restrict__ lam, const float* __restrict__ s_save,
                                                    const T* __restrict__ dx, const float* __restrict__ dxa,
                                                    T* __restrict__ de, float* __restrict__ part, int N, int T_,
                                                    int C) {
  constexpr int VN = V16<T>::n;
  __shared__ float red[4][64];  // [wave][dlam, dw[0..ng)]
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const float lm = lam[0];
  float dlam_p = 0.f, dw_p = 0.f;  // lane l < ng accumulates dw[l]
  for (int n = blockIdx.x * 4 + w; n < N; n += gridDim.x * 4) {
    const int t = n % T_;
    const bool has_next = t + 1 < T_;
    const float gn = has_next ? lm * sigm(s_save[n + 1]) : 0.f;
    const float sg = sigm(s_save[n]);
    const size_t off = (size_t)n * C;
    float dg = 0.f;
    if (t >= 1) {
      for (int vi = l; vi < C / VN; vi += 64) {
        float g[VN], p[VN];
        ld16(dx + off + vi * VN, g);
        if (dxa) add_f32<VN>(dxa + off + vi * VN, g);
        ld16(e + off - C + vi * VN, p);
#pragma unroll
        for (int q = 0; q < VN; ++q) dg += g[q] * p[q];
      }
      dg = wave_sum(dg);
    }
    const float ds = lm * sg * (1.0f - sg) * dg;
    dlam_p += sg * dg;
    for (int vi = l; vi < C / VN; vi += 64) {
      float g[VN];
      ld16(dx + off + vi * VN, g);
      if (dxa) add_f32<VN>(dxa + off + vi * VN, g);
      if (has_next) {
        float h[VN];
        ld16(dx + off + C + vi * VN, h);
        if (dxa) add_f32<VN>(dxa + off + C + vi * VN, h);
#pragma unroll
        for (int q = 0; q < VN; ++q) g[q] += gn * h[q];
      }
      if (vi * VN < ng) {
#pragma unroll
        for (int q = 0; q < VN; ++q)
          if (vi * VN + q < ng) g[q] += ds * to_f(wgt[vi * VN + q]);
      }
      st16(de + off + vi * VN, g);
    }
    if (l < ng) dw_p += ds * to_f(e[off + l]);
  }
  if (l == 0) red[w][0] = dlam_p;
  if (l < ng) red[w][1 + l] = dw_p;
  __syncthreads();
  if (threadIdx.x <= ng) {
    const int k = threadIdx.x;
    part[(size_t)blockIdx.x * (ng + 1) + k] = red[0][k] + red[1][k] + red[2][k] + red[3][k];
  }
}

// ------------------------------------------------------------------- backout
// y = x - lam*xb (y may alias x: each element is read before it is written, by one thread)
template <typename T>
__global__ __launch_bounds__(256) void backout_fwd_k(const T* x, const T* __restrict__ xb,
                                                      const float* __restrict__ lam, T* y, size_t n) {
  constexpr int VN = V16<T>::n;
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * VN;
  if (i >= n) return;
  const float a = lam[0];
  float u[VN], v[VN];
  ld16(x + i, u);
  ld16(xb + i, v);
#pragma unroll
  for (int e = 0; e < VN; ++e) u[e] -= a * v[e];
  st16(y + i, u);
}

// dxb += -lam*dy (in place); per-workgroup partials of -sum(dy*xb).
template <typename T>
__global__ __launch_bounds__(256) void backout_bwd_k(const T* __restrict__ dy, const T* __restrict__ xb,
                                                      const float* __restrict__ lam, T* dxb,
                                                      float* __restrict__ part, int N, int C) {
  constexpr int VN = V16<T>::n;
  __shared__ float red[4];
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const float a = lam[0];
  float s = 0.f;
  for (int row = blockIdx.x * 4 + w; row < N; row += gridDim.x * 4) {
    const size_t off = (size_t)row * C;
    for (int vi = l; vi < C / VN; vi += 64) {
      const size_t o = off + (size_t)vi * VN;
      float g[VN], u[VN], d[VN];
      ld16(dy + o, g);
      ld16(xb + o, u);
      ld16(dxb + o, d);
#pragma unroll
      for (int e = 0; e < VN; ++e) {
        s += g[e] * u[e];
        d[e] -= a * g[e];
      }
      st16(dxb + o, d);
    }
  }
  s = wave_sum(s);
  if (l == 0) red[w] = s;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = -(red[0] + red[1] + red[2] + red[3]);
}

int rows_grid(int N) { return std::max(1, std::min((N + 3) / 4, EXTRA_PBLK)); }
unsigned vec_grid(size_t n, int dt) { return (unsigned)((n / (dt == BF16 ? 8 : 4) + 255) / 256); }

}  // namespace

int mix_partials(int N) { return rows_grid(N); }
int ve_gate_partials(int N) { return (N + 63) / 64; }
int smear_partials(int N) { return rows_grid(N); }
int backout_partials(int N) { return rows_grid(N); }

hipError_t mix_fwd(int dt, const void* x, const void* x0, const float* lam, void* y, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (dt == BF16)
    hipLaunchKernelGGL(mix_fwd_k<bf16>, dim3(vec_grid(n, dt)), dim3(256), 0, s, (const bf16*)x, (const bf16*)x0, lam,
                       (bf16*)y, n);
  else
    hipLaunchKernelGGL(mix_fwd_k<float>, dim3(vec_grid(n, dt)), dim3(256), 0, s, (const float*)x, (const float*)x0,
                       lam, (float*)y, n);
  return hipGetLastError();
}

hipError_t mix_bwd(int dt, const void* dy, const void* x, const void* x0, const float* lam, void* dx, float* dx0,
                   int acc_dx0, float* part, float* dlam, int accumulate, int N, int C, hipStream_t s) {
  const int nb = rows_grid(N);
  if (dt == BF16)
    hipLaunchKernelGGL(mix_bwd_k<bf16>, dim3(nb), dim3(256), 0, s, (const bf16*)dy, (const bf16*)x, (const bf16*)x0,
                       lam, (bf16*)dx, dx0, acc_dx0, part, N, C);
  else
    hipLaunchKernelGGL(mix_bwd_k<float>, dim3(nb), dim3(256), 0, s, (const float*)dy, (const float*)x,
                       (const float*)x0, lam, (float*)dx, dx0, acc_dx0, part, N, C);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return reduce_cols(part, nb, 2, dlam, dlam + 1, accumulate, s);
}

hipError_t ve_fwd(int dt, void* qkv, int ldq, int voff, const void* xn, int C, const int32_t* ids, const void* ve,
                  const void* wg, int nc, int Hkv, int D, int V, float* s_save, int N, hipStream_t s) {
  const dim3 grid((N + 3) / 4);
  if (dt == BF16)
    hipLaunchKernelGGL(ve_fwd_k<bf16>, grid, dim3(256), 0, s, (bf16*)qkv, ldq, voff, (const bf16*)xn, C, ids,
                       (const bf16*)ve, (const bf16*)wg, nc, Hkv, D, V, s_save, N);
  else
    hipLaunchKernelGGL(ve_fwd_k<float>, grid, dim3(256), 0, s, (float*)qkv, ldq, voff, (const float*)xn, C, ids,
                       (const float*)ve, (const float*)wg, nc, Hkv, D, V, s_save, N);
  return hipGetLastError();
}

hipError_t ve_bwd(int dt, const void* dqkv, int ldq, int voff, const int32_t* ids, const void* ve,
                  const float* s_save, int Hkv, int D, int V, float* ds, float* dve, int N, hipStream_t s) {
  const dim3 grid((N + 3) / 4);
  if (dt == BF16)
    hipLaunchKernelGGL(ve_bwd_k<bf16>, grid, dim3(256), 0, s, (const bf16*)dqkv, ldq, voff, ids, (const bf16*)ve,
                       s_save, Hkv, D, V, ds, dve, N);
  else
    hipLaunchKernelGGL(ve_bwd_k<float>, grid, dim3(256), 0, s, (const float*)dqkv, ldq, voff, ids,
                       (const float*)ve, s_save, Hkv, D, V, ds, dve, N);
  return hipGetLastError();
}

hipError_t ve_gate_bwd(int dt, const float* ds, const void* xn, void* dxn, int C, const void* wg, int nc, int Hkv,
                       float* part, float* dwg, int accumulate, int N, hipStream_t s) {
  const int nb = ve_gate_partials(N);
  if (dt == BF16)
    hipLaunchKernelGGL(ve_gate_bwd_k<bf16>, dim3(nb), dim3(256), 0, s, ds, (const bf16*)xn, (bf16*)dxn, C,
                       (const bf16*)wg, nc, Hkv, part, N);
  else
    hipLaunchKernelGGL(ve_gate_bwd_k<float>, dim3(nb), dim3(256), 0, s, ds, (const float*)xn, (float*)dxn, C,
                       (const float*)wg, nc, Hkv, part, N);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return reduce_cols(part, nb, Hkv * nc, dwg, dwg + 1, accumulate, s);
}

hipError_t smear_fwd(int dt, const void* e, const void* w, int ng, const float* lam, void* x, float* s_save, int N,
                     int T, int C, hipStream_t s) {
  const dim3 grid((N + 3) / 4);
  if (dt == BF16)
    hipLaunchKernelGGL(smear_fwd_k<bf16>, grid, dim3(256), 0, s, (const bf16*)e, (const bf16*)w, ng, lam, (bf16*)x,
                       s_save, N, T, C);
  else
    hipLaunchKernelGGL(smear_fwd_k<float>, grid, dim3(256), 0, s, (const float*)e, (const float*)w, ng, lam,
                       (float*)x, s_save, N, T, C);
  return hipGetLastError();
}

hipError_t smear_bwd(int dt, const void* e, const void* w, int ng, const float* lam, const float* s_save,
                     const void* dx, const float* dxa, void* de, float* part, float* dlam, float* dw, int accumulate,
                     int N, int T, int C, hipStream_t s) {
  const int nb = rows_grid(N);
  if (dt == BF16)
    hipLaunchKernelGGL(smear_bwd_k<bf16>, dim3(nb), dim3(256), 0, s, (const bf16*)e, (const bf16*)w, ng, lam, s_save,
                       (const bf16*)dx, dxa, (bf16*)de, part, N, T, C);
  else
    hipLaunchKernelGGL(smear_bwd_k<float>, dim3(nb), dim3(256), 0, s, (const float*)e, (const float*)w, ng, lam,
                       s_save, (const float*)dx, dxa, (float*)de, part, N, T, C);
  hipError_t er = hipGetLastError();
  if (er != hipSuccess) return er;
  return reduce_cols(part, nb, ng + 1, dlam, dw, accumulate, s);
}

hipError_t backout_fwd(int dt, const void* x, const void* xb, const float* lam, void* y, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (dt == BF16)
    hipLaunchKernelGGL(backout_fwd_k<bf16>, dim3(vec_grid(n, dt)), dim3(256), 0, s, (const bf16*)x, (const bf16*)xb,
                       lam, (bf16*)y, n);
  else
    hipLaunchKernelGGL(backout_fwd_k<float>, dim3(vec_grid(n, dt)), dim3(256), 0, s, (const float*)x,
                       (const float*)xb, lam, (float*)y, n);
  return hipGetLastError();
}

hipError_t backout_bwd(int dt, const void* dy, const void* xb, const float* lam, void* dxb, float* part, float* dlam,
                       int accumulate, int N, int C, hipStream_t s) {
  const int nb = rows_grid(N);
  if (dt == BF16)
    hipLaunchKernelGGL(backout_bwd_k<bf16>, dim3(nb), dim3(256), 0, s, (const bf16*)dy, (const bf16*)xb, lam,
                       (bf16*)dxb, part, N, C);
  else
    hipLaunchKernelGGL(backout_bwd_k<float>, dim3(nb), dim3(256), 0, s, (const float*)dy, (const float*)xb, lam,
                       (float*)dxb, part, N, C);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return reduce_cols(part, nb, 1, dlam, dlam, accumulate, s);
}

}  // namespace gdb
