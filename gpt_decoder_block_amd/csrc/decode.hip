// Decode attention against a key/value cache: one new query per sequence, the
// step the inference engine of "Comment Entraîner Votre Propre ChatGPT Pour
// 50€ ?" (section "6. Moteur d'inférence") runs after the prompt has been
// prefilled into the cache.  The query of sequence b sits at position
// i = len_b - 1 and sees key j iff j <= i and (window < 0 or i - j <= window),
// the causal sliding-window rule of the training attention (section "5.
// Unification de Flash Attention": causal=True with a window_size); query
// head h reads K/V head h / (H / Hkv).
//
// The work is a stream over the cache (HBM bound: every visible K and V row
// is read once; one query row per head does 4·D flops per key).  Split-KV
// ("flash decoding"): workgroup (b, kv head g, split s) takes a chunk of the
// visible keys for all G = H / Hkv query heads that share g, so each K/V row
// is fetched once for the whole group.  A key row of D elements is spread
// over D*esize/16 lanes (16 bytes each); one wave instruction covers several
// rows; the dot products finish with a butterfly inside each row's lanes and
// every row group keeps its own online softmax (running max, sum and
// unnormalised output in the base-2 domain).  Row groups, then waves, merge
// their partial states; with one split the workgroup writes the output, else
// it writes (o, m, l) to the workspace and a second kernel merges the splits.
#include <algorithm>
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace gdb {

// Split-KV partials of the allocation-free decode entry point: a fixed
// device array instead of a caller workspace.  decode_plan keeps
// B*H*nsplit below 2048*(H/Hkv) <= 16384 whenever it splits, i.e. at most
// 16384 * (128 + 4) * 4 bytes = 8.65 MB, so 16 MiB holds every plan.  Each
// GPU the library runs on holds its own copy until the process ends.
constexpr size_t DECODE_SCRATCH_BYTES = (size_t)16 << 20;
static __device__ __align__(256) char scratch[DECODE_SCRATCH_BYTES];

namespace {

constexpr int DEC_NW = 4;  // waves per workgroup
constexpr int DEC_U = 4;   // key rows per row group in flight
// floats per split partial: o[D], m, l, padded to 16 bytes
constexpr int part_stride(int D) { return D + 4; }

// merge a second online-softmax state (m2, l2, o2) into (m, l, o)
template <int EPL>
__device__ __forceinline__ void merge_state(float& m, float& l, float* o, float m2, float l2, const float* o2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;  // both empty
  const float a1 = __builtin_amdgcn_exp2f(m - mn), a2 = __builtin_amdgcn_exp2f(m2 - mn);
  l = l * a1 + l2 * a2;
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = o[e] * a1 + o2[e] * a2;
  m = mn;
}

template <typename T, int D, int G>
__global__ __launch_bounds__(64 * DEC_NW) void attn_decode_k(DecodeArgs a, float scale_log2) {
  constexpr int EPL = 16 / (int)sizeof(T);  // elements per lane of a key row
  constexpr int LPR = D / EPL;              // lanes per key row
  constexpr int KPW = 64 / LPR;             // key rows per wave instruction
  constexpr int STRIDE = DEC_NW * KPW;      // rows between a row group's consecutive keys
  __shared__ float red[DEC_NW][G][D + 2];
  const int b = blockIdx.x / a.Hkv, g = blockIdx.x % a.Hkv;
  const int split = blockIdx.y, nsplit = gridDim.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int grp = lane / LPR, sl = lane % LPR;
  const int len = min(max(a.lens[b], 0), a.max_len);
  const int qi = len - 1;
  const int lo = a.window >= 0 ? max(0, qi - a.window) : 0;
  const int k0 = lo + split * a.chunk;
  const int k1 = min(len, k0 + a.chunk);

  const T* kb = (const T*)a.k + (size_t)b * a.bstride + (size_t)g * D + sl * EPL;
  const T* vb = (const T*)a.v + (size_t)b * a.bstride + (size_t)g * D + sl * EPL;
  float q[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    ld16((const T*)a.q + (size_t)b * a.ldq + (size_t)(g * G + h) * D + sl * EPL, q[h]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) q[h][e] *= scale_log2;
  }
  float m[G], l[G], o[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] = 0.f;
  }

  for (int j0 = k0 + w * KPW + grp; j0 < k1; j0 += STRIDE * DEC_U) {
    float kr[DEC_U][EPL], vr[DEC_U][EPL];
#pragma unroll
    for (int u = 0; u < DEC_U; ++u) {
      const int j = min(j0 + u * STRIDE, k1 - 1);  // clamped: rows past k1 are loaded but not used
      ld16(kb + (size_t)j * a.ldk, kr[u]);
      ld16(vb + (size_t)j * a.ldk, vr[u]);
    }
#pragma unroll
    for (int u = 0; u < DEC_U; ++u) {
      const bool ok = j0 + u * STRIDE < k1;  // uniform within the row group
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) s = fmaf(q[h][e], kr[u][e], s);
#pragma unroll
        for (int off = LPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
        if (ok) {
          const float mn = fmaxf(m[h], s);
          const float al = __builtin_amdgcn_exp2f(m[h] - mn);
          const float p = __builtin_amdgcn_exp2f(s - mn);
          l[h] = l[h] * al + p;
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[h][e] = fmaf(p, vr[u][e], o[h][e] * al);
          m[h] = mn;
        }
      }
    }
  }
  // merge the row groups of the wave (lanes sl, sl + LPR, ...)
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float o2[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) o2[e] = __shfl_xor(o[h][e], off, 64);
      const float m2 = __shfl_xor(m[h], off, 64), l2 = __shfl_xor(l[h], off, 64);
      merge_state<EPL>(m[h], l[h], o[h], m2, l2, o2);
    }
  }
  // merge the waves through LDS (row group 0 of each wave holds its state)
  if (grp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) red[w][h][sl * EPL + e] = o[h][e];
      if (sl == 0) {
        red[w][h][D] = m[h];
        red[w][h][D + 1] = l[h];
      }
    }
  }
  __syncthreads();
  if (w != 0 || grp != 0) return;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    for (int ww = 1; ww < DEC_NW; ++ww) {
      float o2[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) o2[e] = red[ww][h][sl * EPL + e];
      merge_state<EPL>(m[h], l[h], o[h], red[ww][h][D], red[ww][h][D + 1], o2);
    }
    const int hh = g * G + h;
    if (nsplit == 1) {
      const float inv = l[h] > 0.f ? 1.0f / l[h] : 0.f;
      float r[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) r[e] = o[h][e] * inv;
      st16((T*)a.o + (size_t)b * a.ldo + (size_t)hh * D + sl * EPL, r);
      if (a.lse && sl == 0)
        a.lse[(size_t)b * a.H + hh] = l[h] > 0.f ? (m[h] + __log2f(l[h])) * 0.6931471805599453f : -INFINITY;
    } else {
      float* pp = a.part + (((size_t)b * a.H + hh) * nsplit + split) * part_stride(D);
#pragma unroll
      for (int e = 0; e < EPL; e += 4) *(f32x4*)(pp + sl * EPL + e) = f32x4{o[h][e], o[h][e + 1], o[h][e + 2], o[h][e + 3]};
      if (sl == 0) {
        pp[D] = m[h];
        pp[D + 1] = l[h];
      }
    }
  }
}

// one wave per (b, h): merge the splits' (o, m, l); lane s holds split s's
// m and l (nsplit <= 64), so the weights come from one max and one sum over
// the wave and the output loads of all splits are independent
template <typename T, int D>
__global__ __launch_bounds__(64) void attn_decode_merge_k(DecodeArgs a, int nsplit) {
  constexpr int DPL = D / 64;  // dims per lane
  constexpr int PD = part_stride(D);
  const int bh = blockIdx.x, b = bh / a.H, hh = bh % a.H, lane = threadIdx.x;
  const float* pp = a.part + (size_t)bh * nsplit * PD;
  const float ms = lane < nsplit ? pp[(size_t)lane * PD + D] : -INFINITY;
  const float ls = lane < nsplit ? pp[(size_t)lane * PD + D + 1] : 0.f;
  const float mx = wave_max(ms);
  const float ws = mx != -INFINITY ? __builtin_amdgcn_exp2f(ms - mx) : 0.f;  // 0 for an empty split
  const float l = wave_sum(ls * ws);
  float o[DPL] = {};
#pragma unroll 8
  for (int s = 0; s < nsplit; ++s) {
    const float wgt = __shfl(ws, s, 64);
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] = fmaf(pp[(size_t)s * PD + lane * DPL + e], wgt, o[e]);
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  T* out = (T*)a.o + (size_t)b * a.ldo + (size_t)hh * D + lane * DPL;
#pragma unroll
  for (int e = 0; e < DPL; ++e) out[e] = from_f<T>(o[e] * inv);
  if (a.lse && lane == 0) a.lse[(size_t)b * a.H + hh] = l > 0.f ? (mx + __log2f(l)) * 0.6931471805599453f : -INFINITY;
}

template <typename T, int D, int G>
void launch_decode(const DecodeArgs& a, int nsplit, float scale_log2, hipStream_t s) {
  hipLaunchKernelGGL((attn_decode_k<T, D, G>), dim3(a.B * a.Hkv, nsplit), dim3(64 * DEC_NW), 0, s, a, scale_log2);
  if (nsplit > 1) hipLaunchKernelGGL((attn_decode_merge_k<T, D>), dim3(a.B * a.H), dim3(64), 0, s, a, nsplit);
}

template <typename T, int D>
hipError_t decode_g(const DecodeArgs& a, int nsplit, float scale_log2, hipStream_t s) {
  switch (a.H / a.Hkv) {
    case 1: launch_decode<T, D, 1>(a, nsplit, scale_log2, s); break;
    case 2: launch_decode<T, D, 2>(a, nsplit, scale_log2, s); break;
    case 3: launch_decode<T, D, 3>(a, nsplit, scale_log2, s); break;
    case 4: launch_decode<T, D, 4>(a, nsplit, scale_log2, s); break;
    case 6: launch_decode<T, D, 6>(a, nsplit, scale_log2, s); break;
    case 8: launch_decode<T, D, 8>(a, nsplit, scale_log2, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

size_t decode_scratch_bytes() { return DECODE_SCRATCH_BYTES; }

// Device address of the current device's copy of `scratch`, looked up with
// hipGetSymbolAddress on the first call made with that device current and
// kept per device (the array's name is a host-side stand-in, never a device
// address).
hipError_t decode_scratch(void** out) {
  constexpr int MAXDEV = 64;
  static std::mutex mu;
  static void* ptrs[MAXDEV] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAXDEV) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return hipSuccess;
}

bool decode_group_supported(int G) { return G == 1 || G == 2 || G == 3 || G == 4 || G == 6 || G == 8; }

void decode_plan(int B, int Hkv, int max_len, int window, int* chunk, int* nsplit) {
  // visible keys of the longest sequence, in chunks of a multiple of 64 keys
  // sized for about 1024 workgroups in all, at least 128 keys (two passes of
  // a workgroup's loads) and at most 64 chunks (one per lane of the merge)
  const int nvis = window >= 0 ? std::min(max_len, window + 1) : max_len;
  long long c = ((long long)nvis * B * Hkv + 1023) / 1024;
  c = std::max(c, 128LL);
  c = std::max(c, ((long long)nvis + 63) / 64);
  c = (c + 63) / 64 * 64;
  *chunk = (int)c;
  *nsplit = nvis > 0 ? (int)((nvis + c - 1) / c) : 1;
}

hipError_t attn_decode(int dt, const DecodeArgs& a, hipStream_t s) {
  int chunk = 0, nsplit = 1;
  decode_plan(a.B, a.Hkv, a.max_len, a.window, &chunk, &nsplit);
  DecodeArgs b = a;
  b.chunk = chunk;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)a.D);
  if (dt == BF16) return a.D == 128 ? decode_g<bf16, 128>(b, nsplit, scale_log2, s)
                                    : decode_g<bf16, 64>(b, nsplit, scale_log2, s);
  return a.D == 128 ? decode_g<float, 128>(b, nsplit, scale_log2, s) : decode_g<float, 64>(b, nsplit, scale_log2, s);
}

}  // namespace gdb
