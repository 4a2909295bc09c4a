// Fixed-order scatter-adds over token ids, for the deterministic backward.
//
// The embedding table's gradient (untied token embedding, "Comment Entraîner
// Votre Propre ChatGPT Pour 50€ ?", section "1. Le modèle GPT") and the value
// embedding tables' gradients (the value-embedding snippet of the same
// section) add one row per token into the row of its id; ids repeat.  With
// float atomics the order of those additions, and so the rounding, changes
// from run to run.  Here the tokens are first sorted by id (a stable LSD radix
// sort on 8-bit digits, so tokens of one id stay in token order), then one
// wavefront per table row and block of columns adds that row's tokens in
// sorted order: the result is the same bits on every run.
//
// Radix pass (digit = 8 bits of the clamped id):
//   hist:    each workgroup counts the digits of its tile of ORD_TILE keys;
//   scan:    one workgroup turns the digit-major counts into start offsets;
//   scatter: each workgroup walks its tile in 256-key rounds in key order and
//            ranks each key among equal digits (wave ballots on the 8 digit
//            bits, then the waves in order), so equal digits keep their order.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace gdb {

namespace {

constexpr int ORD_THREADS = 256;
constexpr int ORD_ITEMS = 8;
constexpr int ORD_TILE = ORD_THREADS * ORD_ITEMS;

__device__ __forceinline__ int clamp_id(int id, int V) { return id < 0 ? 0 : (id >= V ? V - 1 : id); }

__global__ __launch_bounds__(ORD_THREADS) void ord_hist_k(const int32_t* __restrict__ keys, int N, int V, int shift,
                                                           int first, int* __restrict__ hist, int nblk) {
  __shared__ int h[256];
  h[threadIdx.x] = 0;
  __syncthreads();
  const int base = blockIdx.x * ORD_TILE;
#pragma unroll
  for (int r = 0; r < ORD_ITEMS; ++r) {
    const int i = base + r * ORD_THREADS + threadIdx.x;
    if (i < N) {
      const int k = first ? clamp_id(keys[i], V) : keys[i];
      atomicAdd(&h[(k >> shift) & 255], 1);  // integer counts: exact whatever the order
    }
  }
  __syncthreads();
  hist[threadIdx.x * nblk + blockIdx.x] = h[threadIdx.x];
}

// exclusive scan of n ints in place, one workgroup of 1024 threads, chunk by chunk
__global__ __launch_bounds__(1024) void ord_scan_k(int* __restrict__ a, int n) {
  __shared__ int wsum[16];
  __shared__ int carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int base = 0; base < n; base += 1024) {
    const int i = base + threadIdx.x;
    const int v = i < n ? a[i] : 0;
    // inclusive scan within the wave
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    int pre = carry;
    for (int j = 0; j < w; ++j) pre += wsum[j];
    if (i < n) a[i] = pre + x - v;
    __syncthreads();
    if (threadIdx.x == 1023) carry = pre + x;
    __syncthreads();
  }
}

__global__ __launch_bounds__(ORD_THREADS) void ord_scatter_k(const int32_t* __restrict__ keys,
                                                              const int32_t* __restrict__ vals, int N, int V,
                                                              int shift, int first, const int* __restrict__ offs,
                                                              int nblk, int32_t* __restrict__ keys_out,
                                                              int32_t* __restrict__ vals_out) {
  __shared__ int base_d[256];
  __shared__ int run[256];
  __shared__ int wcnt[ORD_THREADS / 64][256];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  base_d[t] = offs[t * nblk + blockIdx.x];
  run[t] = 0;
#pragma unroll
  for (int j = 0; j < ORD_THREADS / 64; ++j) wcnt[j][t] = 0;
  __syncthreads();
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int r = 0; r < ORD_ITEMS; ++r) {
    const int i = blockIdx.x * ORD_TILE + r * ORD_THREADS + t;
    const bool valid = i < N;
    int k = 0, v = 0;
    if (valid) {
      k = first ? clamp_id(keys[i], V) : keys[i];
      v = first ? i : vals[i];
    }
    const int d = (k >> shift) & 255;
    // lanes of this wave holding the same digit
    unsigned long long m = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (d >> b) & 1;
      const unsigned long long bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    const int rank = __popcll(m & below);
    if (valid && rank == 0) wcnt[w][d] = __popcll(m);
    __syncthreads();
    if (valid) {
      int pos = base_d[d] + run[d] + rank;
      for (int j = 0; j < w; ++j) pos += wcnt[j][d];
      keys_out[pos] = k;
      vals_out[pos] = v;
    }
    __syncthreads();
    int add = 0;
#pragma unroll
    for (int j = 0; j < ORD_THREADS / 64; ++j) {
      add += wcnt[j][t];
      wcnt[j][t] = 0;
    }
    run[t] += add;
    __syncthreads();
  }
}

// Lanes 0-31 find the first index j in [0, N) with key[j] >= t0, lanes 32-63
// the first with key[j] >= t1 (keys sorted ascending), both at once: each
// round, a half's 32 lanes probe 32 evenly spaced keys of its remaining range
// and its first probe at or above the target narrows the range to one gap; a
// range of at most 32 keys is settled in one round.  N = 32768 takes four
// rounds of one load per lane (binary searches by one lane: two chains of
// fifteen dependent loads).  Each half returns its own index.
__device__ __forceinline__ int wave_bounds(const int32_t* __restrict__ key, int N, int t0, int t1, int l) {
  const int h = l >> 5, ll = l & 31;
  const int t = h ? t1 : t0;
  int lo = 0, hi = N;  // the half's answer lies in [lo, hi]
  while (__any(lo < hi)) {
    const int len = hi - lo;
    const int step = len > 32 ? (len + 31) >> 5 : 1;
    const int p = lo + ll * step;
    const unsigned long long m = __ballot(p >= hi || key[p] >= t);
    const unsigned mh = (unsigned)(m >> (32 * h));
    const int f = mh ? __ffs((int)mh) - 1 : 32;  // the half's first probe at or above t
    if (len > 32) {
      const int nlo = f == 0 ? lo : lo + (f - 1) * step + 1;
      hi = f == 0 ? lo : (f < 32 ? min(hi, lo + f * step) : hi);
      lo = nlo;
    } else {
      lo = hi = f < 32 ? lo + f : hi;
    }
  }
  return lo;
}

// One wavefront per (table row v, block of 64*VN columns): out[v, c] (+)= the
// sum over the row's tokens n, in sorted (token) order, of
// g(n, c) * x[n*ldx + xoff + c], c < width, with g = 3*sigmoid(s[n*G + c/D])
// when gate logits s are given, else 1.  The rows of SEG_U tokens are loaded
// together and then added one after another, so a row that many tokens share
// (natural text's frequent ids) costs one memory latency per SEG_U tokens
// rather than per token; the rest of a row goes in batches of 4.  The
// additions keep the token order whatever the batching.
constexpr int SEG_U = 16;
template <typename T, bool GATE, int U>
__device__ __forceinline__ void seg_batch(int myn, int cnt, const T* __restrict__ x, int ldx, int xoff, int cl,
                                          const float* __restrict__ s, int G, int D, float* acc) {
  constexpr int VN = V16<T>::n;
  typedef typename std::conditional<sizeof(T) == 2, bf16x8, f32x4>::type Raw;
  Raw raw[U];
  float gs[U];
  // every load issued before the first addition (tokens past cnt re-read the
  // batch's first row and are not added)
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int n = __shfl(myn, u < cnt ? u : 0, 64);
    raw[u] = *(const Raw*)(x + (size_t)n * ldx + xoff + cl);
    if (GATE) gs[u] = s[(size_t)n * G + cl / D];
  }
  __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of every addition
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u < cnt) {  // wave-uniform
      const float g = GATE ? 3.0f / (1.0f + __expf(-gs[u])) : 1.0f;
#pragma unroll
      for (int e = 0; e < VN; ++e) acc[e] += g * (float)raw[u][e];
    }
  }
}

template <typename T, bool GATE>
__global__ __launch_bounds__(256) void segsum_k(const int32_t* __restrict__ skey, const int32_t* __restrict__ perm,
                                                int N, const T* __restrict__ x, int ldx, int xoff, int width,
                                                const float* __restrict__ s, int G, int D, float* __restrict__ out,
                                                int V, int accumulate, int ncb) {
  constexpr int VN = V16<T>::n;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
  const int v = gw / ncb, cb = gw - v * ncb;
  if (v >= V) return;  // wave-uniform
  const int c0 = (cb * 64 + l) * VN;
  const bool on = c0 < width;
  const int cl = on ? c0 : 0;  // lanes past the row's end load column 0 and store nothing
  const int bnd = wave_bounds(skey, N, v, v + 1, l);
  const int lo = __builtin_amdgcn_readlane(bnd, 0), hi = __builtin_amdgcn_readlane(bnd, 32);
  float acc[VN];
#pragma unroll
  for (int e = 0; e < VN; ++e) acc[e] = 0.f;
  // the gated form holds a gate logit per token too: half the batch
  constexpr int BU = GATE ? SEG_U / 2 : SEG_U;
  int j0 = lo;
  if (hi - j0 >= BU) {
    // lane u < BU holds the batch's u-th token index; the next batch's
    // indices are loaded while this batch's rows are in flight
    int myn = perm[j0 + (l < BU ? l : 0)];
    for (; hi - j0 >= BU; j0 += BU) {
      const int j1 = j0 + BU;
      const int nxt = perm[hi - j1 >= BU ? j1 + (l < BU ? l : 0) : j0];
      seg_batch<T, GATE, BU>(myn, BU, x, ldx, xoff, cl, s, G, D, acc);
      myn = nxt;
    }
  }
  for (; j0 < hi; j0 += 4) {
    const int cnt = min(4, hi - j0);
    seg_batch<T, GATE, 4>(perm[j0 + (l < cnt ? l : 0)], cnt, x, ldx, xoff, cl, s, G, D, acc);
  }
  if (!on) return;
  float* orow = out + (size_t)v * width + c0;
  if (accumulate) {
#pragma unroll
    for (int e = 0; e < VN; e += 4) {
      const f32x4 o = *(const f32x4*)(orow + e);
      acc[e] += o[0]; acc[e + 1] += o[1]; acc[e + 2] += o[2]; acc[e + 3] += o[3];
    }
  }
#pragma unroll
  for (int e = 0; e < VN; e += 4) *(f32x4*)(orow + e) = f32x4{acc[e], acc[e + 1], acc[e + 2], acc[e + 3]};
}

template <typename T>
void launch_segsum(dim3 grid, hipStream_t st, const int32_t* sk, const int32_t* perm, int N, const void* x, int ldx,
                   int xoff, int width, const float* gs, int G, int D, float* out, int V, int accumulate, int ncb) {
  if (gs)
    hipLaunchKernelGGL((segsum_k<T, true>), grid, dim3(256), 0, st, sk, perm, N, (const T*)x, ldx, xoff, width, gs, G, D,
                       out, V, accumulate, ncb);
  else
    hipLaunchKernelGGL((segsum_k<T, false>), grid, dim3(256), 0, st, sk, perm, N, (const T*)x, ldx, xoff, width, gs, G,
                       D, out, V, accumulate, ncb);
}

int ord_blocks(int N) { return std::max(1, (N + ORD_TILE - 1) / ORD_TILE); }
int ord_passes(int V) {
  int bits = 1;
  while (bits < 31 && (1LL << bits) < (long long)V) ++bits;
  return (bits + 7) / 8;
}
size_t al256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace

size_t token_order_ws_bytes(int N) {
  const size_t n = (size_t)std::max(N, 1);
  return 4 * al256(n * 4) + al256((size_t)256 * ord_blocks(N) * 4);
}

hipError_t token_order(const int32_t* ids, int N, int V, void* ws, const int32_t** sorted_ids, const int32_t** perm,
                       hipStream_t s) {
  char* b = (char*)ws;
  const size_t n4 = al256((size_t)std::max(N, 1) * 4);
  int32_t* k[2] = {(int32_t*)b, (int32_t*)(b + 2 * n4)};
  int32_t* p[2] = {(int32_t*)(b + n4), (int32_t*)(b + 3 * n4)};
  int* hist = (int*)(b + 4 * n4);
  const int nblk = ord_blocks(N), np = ord_passes(V);
  int cur = 0;
  for (int pass = 0; pass < np; ++pass) {
    const int first = pass == 0;
    const int32_t* kin = first ? ids : k[cur];
    const int32_t* pin = first ? nullptr : p[cur];
    const int dst = first ? 0 : cur ^ 1;
    hipLaunchKernelGGL(ord_hist_k, dim3(nblk), dim3(ORD_THREADS), 0, s, kin, N, V, 8 * pass, first, hist, nblk);
    hipLaunchKernelGGL(ord_scan_k, dim3(1), dim3(1024), 0, s, hist, 256 * nblk);
    hipLaunchKernelGGL(ord_scatter_k, dim3(nblk), dim3(ORD_THREADS), 0, s, kin, pin, N, V, 8 * pass, first, hist,
                       nblk, k[dst], p[dst]);
    cur = dst;
  }
  *sorted_ids = k[cur];
  *perm = p[cur];
  return hipGetLastError();
}

hipError_t rows_segsum(int dt, const int32_t* sorted_ids, const int32_t* perm, int N, const void* x, int ldx, int xoff,
                       int width, const float* gate_s, int G, int D, float* out, int V, int accumulate, hipStream_t s) {
  const int vn = dt == BF16 ? 8 : 4;
  const int ncb = (width + 64 * vn - 1) / (64 * vn);  // column blocks per row
  const dim3 grid((unsigned)(((size_t)V * ncb + 3) / 4));
  if (dt == BF16) launch_segsum<bf16>(grid, s, sorted_ids, perm, N, x, ldx, xoff, width, gate_s, G, D, out, V, accumulate, ncb);
  else launch_segsum<float>(grid, s, sorted_ids, perm, N, x, ldx, xoff, width, gate_s, G, D, out, V, accumulate, ncb);
  return hipGetLastError();
}

}  // namespace gdb
