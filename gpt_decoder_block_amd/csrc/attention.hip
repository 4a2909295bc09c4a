// Causal / sliding-window grouped-query attention, forward and backward.
//
// Semantics ("Comment Entraîner Votre Propre ChatGPT Pour 50€ ?", sections
// "1. Le modèle GPT" and "5. Unification de Flash Attention": causal attention
// with an optional window, fewer K/V heads than query heads, (B, T, H, D)
// tensors, default 1/sqrt(D) scale):
//   o_i = sum_j softmax_j(q_i . k_j / sqrt(D)) v_j over visible j:
//   j <= i and (window < 0 or i - j <= window); query head h reads K/V head
//   h / (H / Hkv).
//
// bf16 path, D = 128, gfx950 MFMA (v_mfma_f32_32x32x16_bf16), flash-style:
//   forward: a workgroup owns 128 query rows of one (b, h), 32 per wave, and
//     streams 64-key tiles of K (row-major in LDS) and V (transposed in LDS)
//     through two LDS stages; only tiles that intersect the causal band or the
//     window are visited.  Each lane owns one query row: S^T = K Q^T puts a
//     query in a lane, so the online-softmax max/sum need one exchange with
//     the partner lane (lane ^ 32) only; O^T = V^T P^T keeps the same lane ->
//     query map for the rescale.  P goes from the S accumulators into the
//     second MFMA's operand registers directly, with a relabelling of the
//     contraction index that both operands share.  Writes O (bf16) and the
//     row log-sum-exp (fp32).
//   backward: delta_i = dO_i . O_i; then two deterministic kernels that each
//     recompute P from the saved log-sum-exp:
//       dK/dV: a workgroup owns 128 keys of one (b, kv head) and loops over
//         the query heads of its group and the visible 64-row query tiles,
//         accumulating dV^T += dO^T P and dK^T += Q^T dS in registers
//         (the GQA head reduction happens in registers, no atomics);
//       dQ: a workgroup owns 128 query rows and loops over the visible key
//         tiles, dQ^T += K^T dS^T.
// fp32 path: one thread per query (or key) row; slow, exact reference-order
// kernels for the fp32 mode.
#include "common.h"
#include "kernels.h"

namespace gdb {

namespace {

constexpr int HD = 128;  // head_dim of the MFMA path

// Row-major tile [rows][128] bf16: 16 chunks of 8 per row, XOR-swizzled.
__device__ __forceinline__ int kswz(int row, int chunk) { return chunk ^ (row & 15); }
// Transposed tile [128 d][64 j] bf16: 16 units of 4 per row, XOR-swizzled.
__device__ __forceinline__ int tswz(int d, int unit) { return unit ^ ((d ^ (d >> 3)) & 15); }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// read the A-operand of a 32x32x16 MFMA from a transposed tile: row `d`,
// contraction slots e -> key 16ks + 8(e/4) + 4lh + e%4
__device__ __forceinline__ bf16x8 ld_t_frag(const bf16* S, int d, int ks, int lh) {
  const bf16x4 lo = *(const bf16x4*)(S + d * 64 + tswz(d, 4 * ks + lh) * 4);
  const bf16x4 hi = *(const bf16x4*)(S + d * 64 + tswz(d, 4 * ks + 2 + lh) * 4);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// pack the accumulator values of keys (or queries) 16ks..16ks+15 held by this
// lane into the matching contraction slots (same relabelling as ld_t_frag)
__device__ __forceinline__ bf16x8 pack_p(const f32x16* s, int ks) {
  const f32x16& x = s[ks >> 1];
  const int b = 8 * (ks & 1);
  return bf16x8{(bf16)x[b + 0], (bf16)x[b + 1], (bf16)x[b + 2], (bf16)x[b + 3],
                (bf16)x[b + 4], (bf16)x[b + 5], (bf16)x[b + 6], (bf16)x[b + 7]};
}

// Global -> registers for a 64-row x 128-d tile: each thread loads 4
// consecutive rows of one 16-byte chunk (row (t>>4)*4 + i, chunk t & 15).
struct TileRegs {
  bf16x8 r[4];
  __device__ __forceinline__ void load(const bf16* base, size_t ld, int row0, int nrows) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row0 + (t >> 4) * 4 + i;
      r[i] = row < nrows ? *(const bf16x8*)(base + (size_t)row * ld + (t & 15) * 8) : bf16x8{};
    }
  }
  __device__ __forceinline__ void store_rows(bf16* S) const {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (t >> 4) * 4 + i;
      *(bf16x8*)(S + row * HD + kswz(row, t & 15) * 8) = r[i];
    }
  }
  __device__ __forceinline__ void store_trans(bf16* S) const {
    const int t = threadIdx.x;
    const int unit = t >> 4;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int d = (t & 15) * 8 + jj;
      *(bf16x4*)(S + d * 64 + tswz(d, unit) * 4) = bf16x4{r[0][jj], r[1][jj], r[2][jj], r[3][jj]};
    }
  }
};

__device__ __forceinline__ bool visible(int i, int j, int T, int W) {
  return j < T && j <= i && (W < 0 || i - j <= W);
}

// ----------------------------------------------------------------- forward
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_k(AttnArgs a, float scale_log2) {
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][64 * HD];
  __shared__ __attribute__((aligned(16))) bf16 Vt[2][HD * 64];
  const int T = a.T, H = a.H, Hkv = a.Hkv, W = a.window;
  const int nqb = (T + 127) / 128;
  const int qb = nqb - 1 - (int)blockIdx.x;  // heaviest query blocks first
  const int b = blockIdx.y / H, h = blockIdx.y % H, g = h / (H / Hkv);
  const int q0 = qb * 128;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, lr = lane & 31, lh = lane >> 5;
  const int qi = q0 + w * 32 + lr;
  const bf16* base = (const bf16*)a.qkv + (size_t)b * T * a.ld;
  const bf16* kbase = base + (H + g) * HD;
  const bf16* vbase = base + (H + Hkv + g) * HD;

  bf16x8 qf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
    qf[kk] = qi < T ? *(const bf16x8*)(base + (size_t)qi * a.ld + h * HD + kk * 16 + lh * 8) : bf16x8{};

  int kv_lo = W >= 0 ? max(0, q0 - W) : 0;
  kv_lo &= ~63;
  const int kv_hi = min(T, q0 + 128);
  const int ntile = (kv_hi - kv_lo + 63) / 64;

  TileRegs kr, vr;
  kr.load(kbase, a.ld, kv_lo, T);
  vr.load(vbase, a.ld, kv_lo, T);
  kr.store_rows(Ks[0]);
  vr.store_trans(Vt[0]);
  __syncthreads();

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16{};
  float m = -INFINITY, l = 0.f;

  for (int it = 0; it < ntile; ++it) {
    const int st = it & 1;
    const int kv0 = kv_lo + it * 64;
    const bool more = it + 1 < ntile;
    if (more) {
      kr.load(kbase, a.ld, kv0 + 64, T);
      vr.load(vbase, a.ld, kv0 + 64, T);
    }
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        const int row = jb * 32 + lr;
        const bf16x8 kf = *(const bf16x8*)(Ks[st] + row * HD + kswz(row, 2 * kk + lh) * 8);
        s[jb] = mfma32(kf, qf[kk], s[jb]);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int j = kv0 + jb * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
        const float x = visible(qi, j, T, W) ? s[jb][v] * scale_log2 : -INFINITY;
        s[jb][v] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = fmaxf(m, mx);
    const float msafe = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(m - msafe);
    l *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db) o[db] *= alpha;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = __builtin_amdgcn_exp2f(s[jb][v] - msafe);
        s[jb][v] = p;
        l += p;
      }
    m = mnew;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 pf = pack_p(s, ks);
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] = mfma32(ld_t_frag(Vt[st], db * 32 + lr, ks, lh), pf, o[db]);
    }
    if (more) {
      kr.store_rows(Ks[st ^ 1]);
      vr.store_trans(Vt[st ^ 1]);
    }
    __syncthreads();
  }

  const float lt = l + __shfl_xor(l, 32, 64);
  if (qi < T) {
    const float inv = 1.0f / lt;
    bf16* orow = (bf16*)a.o + ((size_t)b * T + qi) * a.ldo + h * HD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = db * 32 + 8 * gq + 4 * lh;
        *(bf16x4*)(orow + d) = bf16x4{(bf16)(o[db][4 * gq] * inv), (bf16)(o[db][4 * gq + 1] * inv),
                                      (bf16)(o[db][4 * gq + 2] * inv), (bf16)(o[db][4 * gq + 3] * inv)};
      }
    if (lh == 0) a.lse[((size_t)b * H + h) * T + qi] = (m + __log2f(lt)) * 0.69314718055994531f;
  }
}

// ------------------------------------------------------- backward: delta
template <typename T_>
__global__ __launch_bounds__(256) void attn_delta_k(AttnArgs a) {
  // one wave per (token, head); lanes stride over D
  const int idx = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
  const int N = a.B * a.T;
  if (idx >= N * a.H) return;
  const int n = idx / a.H, h = idx % a.H;
  const T_* o = (const T_*)a.o + (size_t)n * a.ldo + h * a.D;
  const T_* d = (const T_*)a.dout + (size_t)n * a.lddo + h * a.D;
  float s = 0.f;
  for (int e = l; e < a.D; e += 64) s += to_f(o[e]) * to_f(d[e]);
  s = wave_sum(s);
  const int b = n / a.T, t = n % a.T;
  if (l == 0) a.delta[((size_t)b * a.H + h) * a.T + t] = s;
}

// ------------------------------------------------------ backward: dK, dV
__global__ __launch_bounds__(256, 1) void attn_bwd_dkv_bf16_k(AttnArgs a, float scale_log2, float scale) {
  __shared__ __attribute__((aligned(16))) bf16 Qs[2][64 * HD];
  __shared__ __attribute__((aligned(16))) bf16 Qt[2][HD * 64];
  __shared__ __attribute__((aligned(16))) bf16 Ds[2][64 * HD];
  __shared__ __attribute__((aligned(16))) bf16 Dt[2][HD * 64];
  __shared__ __attribute__((aligned(16))) float Ls[2][64];
  __shared__ __attribute__((aligned(16))) float Dl[2][64];
  const int T = a.T, H = a.H, Hkv = a.Hkv, W = a.window, G = H / Hkv;
  const int b = blockIdx.y / Hkv, g = blockIdx.y % Hkv;
  const int kv0 = blockIdx.x * 128;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, lr = lane & 31, lh = lane >> 5;
  const int kj = kv0 + w * 32 + lr;  // this lane's key
  const bf16* base = (const bf16*)a.qkv + (size_t)b * T * a.ld;
  const bf16* dbase = (const bf16*)a.dout + (size_t)b * T * a.lddo;

  bf16x8 kf[8], vf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const size_t roff = (size_t)kj * a.ld + kk * 16 + lh * 8;
    kf[kk] = kj < T ? *(const bf16x8*)(base + roff + (H + g) * HD) : bf16x8{};
    vf[kk] = kj < T ? *(const bf16x8*)(base + roff + (H + Hkv + g) * HD) : bf16x8{};
  }
  f32x16 dk[4], dv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { dk[i] = f32x16{}; dv[i] = f32x16{}; }

  const int q_lo = kv0;  // multiple of 64
  const int q_hi = W >= 0 ? min(T, kv0 + 128 + W) : T;
  const int nqt = q_hi > q_lo ? (q_hi - q_lo + 63) / 64 : 0;
  const int total = nqt * G;

  TileRegs qr, dr;
  float lsev = 0.f, delv = 0.f;
  auto gload = [&](int it) {
    const int hh = g * G + it / nqt;
    const int i0 = q_lo + (it % nqt) * 64;
    qr.load(base + hh * HD, a.ld, i0, T);
    dr.load(dbase + hh * HD, a.lddo, i0, T);
    if (t < 64) {
      const int i = i0 + t;
      const size_t li = ((size_t)b * H + hh) * T + i;
      lsev = i < T ? a.lse[li] * 1.4426950408889634f : 0.f;
      delv = i < T ? a.delta[li] : 0.f;
    }
  };
  auto sstore = [&](int st) {
    qr.store_rows(Qs[st]);
    qr.store_trans(Qt[st]);
    dr.store_rows(Ds[st]);
    dr.store_trans(Dt[st]);
    if (t < 64) { Ls[st][t] = lsev; Dl[st][t] = delv; }
  };
  if (total > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();

  for (int it = 0; it < total; ++it) {
    const int st = it & 1;
    const int i0 = q_lo + (it % nqt) * 64;
    const bool more = it + 1 < total;
    if (more) gload(it + 1);
    // S[i][j] and dP[i][j]: lane = key j, registers = queries
    f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
        const int row = ib * 32 + lr;
        const bf16x8 qa = *(const bf16x8*)(Qs[st] + row * HD + kswz(row, 2 * kk + lh) * 8);
        const bf16x8 da = *(const bf16x8*)(Ds[st] + row * HD + kswz(row, 2 * kk + lh) * 8);
        s[ib] = mfma32(qa, kf[kk], s[ib]);
        dp[ib] = mfma32(da, vf[kk], dp[ib]);
      }
    }
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int il = ib * 32 + 8 * gq + 4 * lh;
        const f32x4 L4 = *(const f32x4*)(&Ls[st][il]);
        const f32x4 D4 = *(const f32x4*)(&Dl[st][il]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int v = 4 * gq + r;
          const int i = i0 + il + r;
          const float p = visible(i, kj, T, W) && i < T ? __builtin_amdgcn_exp2f(s[ib][v] * scale_log2 - L4[r]) : 0.f;
          s[ib][v] = p;
          dp[ib][v] = p * (dp[ib][v] - D4[r]);
        }
      }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 pf = pack_p(s, ks);
      const bf16x8 sf = pack_p(dp, ks);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        dv[db] = mfma32(ld_t_frag(Dt[st], db * 32 + lr, ks, lh), pf, dv[db]);
        dk[db] = mfma32(ld_t_frag(Qt[st], db * 32 + lr, ks, lh), sf, dk[db]);
      }
    }
    if (more) sstore(st ^ 1);
    __syncthreads();
  }

  if (kj < T) {
    bf16* row = (bf16*)a.dqkv + ((size_t)b * T + kj) * a.lddq;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = db * 32 + 8 * gq + 4 * lh;
        *(bf16x4*)(row + (H + g) * HD + d) =
            bf16x4{(bf16)(dk[db][4 * gq] * scale), (bf16)(dk[db][4 * gq + 1] * scale),
                   (bf16)(dk[db][4 * gq + 2] * scale), (bf16)(dk[db][4 * gq + 3] * scale)};
        *(bf16x4*)(row + (H + Hkv + g) * HD + d) =
            bf16x4{(bf16)dv[db][4 * gq], (bf16)dv[db][4 * gq + 1], (bf16)dv[db][4 * gq + 2], (bf16)dv[db][4 * gq + 3]};
      }
  }
}

// ------------------------------------------------------------ backward: dQ
__global__ __launch_bounds__(256, 1) void attn_bwd_dq_bf16_k(AttnArgs a, float scale_log2, float scale) {
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][64 * HD];
  __shared__ __attribute__((aligned(16))) bf16 Kt[2][HD * 64];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][64 * HD];
  const int T = a.T, H = a.H, Hkv = a.Hkv, W = a.window;
  const int nqb = (T + 127) / 128;
  const int qb = nqb - 1 - (int)blockIdx.x;
  const int b = blockIdx.y / H, h = blockIdx.y % H, g = h / (H / Hkv);
  const int q0 = qb * 128;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, lr = lane & 31, lh = lane >> 5;
  const int qi = q0 + w * 32 + lr;
  const bf16* base = (const bf16*)a.qkv + (size_t)b * T * a.ld;
  const bf16* kbase = base + (H + g) * HD;
  const bf16* vbase = base + (H + Hkv + g) * HD;

  bf16x8 qf[8], df[8];
  const bf16* drow = (const bf16*)a.dout + ((size_t)b * T + qi) * a.lddo + h * HD;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    qf[kk] = qi < T ? *(const bf16x8*)(base + (size_t)qi * a.ld + h * HD + kk * 16 + lh * 8) : bf16x8{};
    df[kk] = qi < T ? *(const bf16x8*)(drow + kk * 16 + lh * 8) : bf16x8{};
  }
  const size_t li = ((size_t)b * H + h) * T + qi;
  const float lse2 = qi < T ? a.lse[li] * 1.4426950408889634f : 0.f;
  const float dlt = qi < T ? a.delta[li] : 0.f;

  int kv_lo = W >= 0 ? max(0, q0 - W) : 0;
  kv_lo &= ~63;
  const int kv_hi = min(T, q0 + 128);
  const int ntile = (kv_hi - kv_lo + 63) / 64;

  TileRegs kr, vr;
  kr.load(kbase, a.ld, kv_lo, T);
  vr.load(vbase, a.ld, kv_lo, T);
  kr.store_rows(Ks[0]);
  kr.store_trans(Kt[0]);
  vr.store_rows(Vs[0]);
  __syncthreads();

  f32x16 dq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) dq[i] = f32x16{};

  for (int it = 0; it < ntile; ++it) {
    const int st = it & 1;
    const int kv0 = kv_lo + it * 64;
    const bool more = it + 1 < ntile;
    if (more) {
      kr.load(kbase, a.ld, kv0 + 64, T);
      vr.load(vbase, a.ld, kv0 + 64, T);
    }
    f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        const int row = jb * 32 + lr;
        const int off = row * HD + kswz(row, 2 * kk + lh) * 8;
        s[jb] = mfma32(*(const bf16x8*)(Ks[st] + off), qf[kk], s[jb]);
        dp[jb] = mfma32(*(const bf16x8*)(Vs[st] + off), df[kk], dp[jb]);
      }
    }
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int j = kv0 + jb * 32 + 8 * (v >> 2) + 4 * lh + (v & 3);
        const float p = visible(qi, j, T, W) ? __builtin_amdgcn_exp2f(s[jb][v] * scale_log2 - lse2) : 0.f;
        dp[jb][v] = p * (dp[jb][v] - dlt);
      }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 sf = pack_p(dp, ks);
#pragma unroll
      for (int db = 0; db < 4; ++db) dq[db] = mfma32(ld_t_frag(Kt[st], db * 32 + lr, ks, lh), sf, dq[db]);
    }
    if (more) {
      kr.store_rows(Ks[st ^ 1]);
      kr.store_trans(Kt[st ^ 1]);
      vr.store_rows(Vs[st ^ 1]);
    }
    __syncthreads();
  }
  if (qi < T) {
    bf16* row = (bf16*)a.dqkv + ((size_t)b * T + qi) * a.lddq + h * HD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = db * 32 + 8 * gq + 4 * lh;
        *(bf16x4*)(row + d) = bf16x4{(bf16)(dq[db][4 * gq] * scale), (bf16)(dq[db][4 * gq + 1] * scale),
                                     (bf16)(dq[db][4 * gq + 2] * scale), (bf16)(dq[db][4 * gq + 3] * scale)};
      }
  }
}

// ---------------------------------------------------------------- fp32 path
template <int D>
__global__ __launch_bounds__(64) void attn_fwd_f32_k(AttnArgs a, float scale) {
  const int idx = blockIdx.x * 64 + threadIdx.x;
  const int T = a.T, H = a.H, Hkv = a.Hkv, W = a.window;
  if (idx >= a.B * H * T) return;
  const int i = idx % T, h = (idx / T) % H, b = idx / (T * H);
  const int g = h / (H / Hkv);
  const float* base = (const float*)a.qkv + (size_t)b * T * a.ld;
  float q[D], o[D];
  for (int d = 0; d < D; ++d) { q[d] = base[(size_t)i * a.ld + h * D + d]; o[d] = 0.f; }
  float m = -INFINITY, l = 0.f;
  const int j0 = W >= 0 ? max(0, i - W) : 0;
  for (int j = j0; j <= i; ++j) {
    const float* k = base + (size_t)j * a.ld + (H + g) * D;
    const float* v = base + (size_t)j * a.ld + (H + Hkv + g) * D;
    float s = 0.f;
    for (int d = 0; d < D; ++d) s = fmaf(q[d], k[d], s);
    s *= scale;
    const float mn = fmaxf(m, s);
    const float al = expf(m - mn), p = expf(s - mn);
    l = l * al + p;
    for (int d = 0; d < D; ++d) o[d] = o[d] * al + p * v[d];
    m = mn;
  }
  float* orow = (float*)a.o + ((size_t)b * T + i) * a.ldo + h * D;
  for (int d = 0; d < D; ++d) orow[d] = o[d] / l;
  a.lse[((size_t)b * H + h) * T + i] = m + logf(l);
}

template <int D>
__global__ __launch_bounds__(64) void attn_bwd_dq_f32_k(AttnArgs a, float scale) {
  const int idx = blockIdx.x * 64 + threadIdx.x;
  const int T = a.T, H = a.H, Hkv = a.Hkv, W = a.window;
  if (idx >= a.B * H * T) return;
  const int i = idx % T, h = (idx / T) % H, b = idx / (T * H);
  const int g = h / (H / Hkv);
  const float* base = (const float*)a.qkv + (size_t)b * T * a.ld;
  const float* dor = (const float*)a.dout + ((size_t)b * T + i) * a.lddo + h * D;
  float q[D], dq[D], dov[D];
  for (int d = 0; d < D; ++d) { q[d] = base[(size_t)i * a.ld + h * D + d]; dq[d] = 0.f; dov[d] = dor[d]; }
  const size_t li = ((size_t)b * H + h) * T + i;
  const float lse = a.lse[li], dl = a.delta[li];
  const int j0 = W >= 0 ? max(0, i - W) : 0;
  for (int j = j0; j <= i; ++j) {
    const float* k = base + (size_t)j * a.ld + (H + g) * D;
    const float* v = base + (size_t)j * a.ld + (H + Hkv + g) * D;
    float s = 0.f, dp = 0.f;
    for (int d = 0; d < D; ++d) { s = fmaf(q[d], k[d], s); dp = fmaf(dov[d], v[d], dp); }
    const float p = expf(s * scale - lse);
    const float ds = p * (dp - dl);
    for (int d = 0; d < D; ++d) dq[d] = fmaf(ds, k[d], dq[d]);
  }
  float* out = (float*)a.dqkv + ((size_t)b * T + i) * a.lddq + h * D;
  for (int d = 0; d < D; ++d) out[d] = dq[d] * scale;
}

template <int D>
__global__ __launch_bounds__(64) void attn_bwd_dkv_f32_k(AttnArgs a, float scale) {
  const int idx = blockIdx.x * 64 + threadIdx.x;
  const int T = a.T, H = a.H, Hkv = a.Hkv, W = a.window, G = H / Hkv;
  if (idx >= a.B * Hkv * T) return;
  const int j = idx % T, g = (idx / T) % Hkv, b = idx / (T * Hkv);
  const float* base = (const float*)a.qkv + (size_t)b * T * a.ld;
  float k[D], v[D], dk[D], dv[D];
  for (int d = 0; d < D; ++d) {
    k[d] = base[(size_t)j * a.ld + (H + g) * D + d];
    v[d] = base[(size_t)j * a.ld + (H + Hkv + g) * D + d];
    dk[d] = 0.f;
    dv[d] = 0.f;
  }
  const int i1 = W >= 0 ? min(T - 1, j + W) : T - 1;
  for (int hh = g * G; hh < (g + 1) * G; ++hh) {
    for (int i = j; i <= i1; ++i) {
      const float* q = base + (size_t)i * a.ld + hh * D;
      const float* dor = (const float*)a.dout + ((size_t)b * T + i) * a.lddo + hh * D;
      const size_t li = ((size_t)b * H + hh) * T + i;
      float s = 0.f, dp = 0.f;
      for (int d = 0; d < D; ++d) { s = fmaf(q[d], k[d], s); dp = fmaf(dor[d], v[d], dp); }
      const float p = expf(s * scale - a.lse[li]);
      const float ds = p * (dp - a.delta[li]);
      for (int d = 0; d < D; ++d) { dv[d] = fmaf(p, dor[d], dv[d]); dk[d] = fmaf(ds, q[d], dk[d]); }
    }
  }
  float* out = (float*)a.dqkv + ((size_t)b * T + j) * a.lddq;
  for (int d = 0; d < D; ++d) {
    out[(H + g) * D + d] = dk[d] * scale;
    out[(H + Hkv + g) * D + d] = dv[d];
  }
}

}  // namespace

hipError_t attn_fwd(int dt, const AttnArgs& a, hipStream_t s) {
  if (a.B * a.T == 0) return hipSuccess;
  const float scale = 1.0f / sqrtf((float)a.D);
  if (dt == BF16) {
    dim3 g((a.T + 127) / 128, a.B * a.H);
    hipLaunchKernelGGL(attn_fwd_bf16_k, g, dim3(256), 0, s, a, scale * 1.4426950408889634f);
  } else {
    dim3 g((a.B * a.H * a.T + 63) / 64);
    if (a.D == 64) hipLaunchKernelGGL(attn_fwd_f32_k<64>, g, dim3(64), 0, s, a, scale);
    else hipLaunchKernelGGL(attn_fwd_f32_k<128>, g, dim3(64), 0, s, a, scale);
  }
  return hipGetLastError();
}

hipError_t attn_bwd(int dt, const AttnArgs& a, hipStream_t s) {
  if (a.B * a.T == 0) return hipSuccess;
  const float scale = 1.0f / sqrtf((float)a.D);
  const int rows = a.B * a.T * a.H;
  if (dt == BF16) hipLaunchKernelGGL(attn_delta_k<bf16>, dim3((rows + 3) / 4), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(attn_delta_k<float>, dim3((rows + 3) / 4), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dt == BF16) {
    hipLaunchKernelGGL(attn_bwd_dkv_bf16_k, dim3((a.T + 127) / 128, a.B * a.Hkv), dim3(256), 0, s, a,
                       scale * 1.4426950408889634f, scale);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_bwd_dq_bf16_k, dim3((a.T + 127) / 128, a.B * a.H), dim3(256), 0, s, a,
                       scale * 1.4426950408889634f, scale);
  } else {
    dim3 gq((a.B * a.H * a.T + 63) / 64), gk((a.B * a.Hkv * a.T + 63) / 64);
    if (a.D == 64) {
      hipLaunchKernelGGL(attn_bwd_dq_f32_k<64>, gq, dim3(64), 0, s, a, scale);
      hipLaunchKernelGGL(attn_bwd_dkv_f32_k<64>, gk, dim3(64), 0, s, a, scale);
    } else {
      hipLaunchKernelGGL(attn_bwd_dq_f32_k<128>, gq, dim3(64), 0, s, a, scale);
      hipLaunchKernelGGL(attn_bwd_dkv_f32_k<128>, gk, dim3(64), 0, s, a, scale);
    }
  }
  return hipGetLastError();
}

}  // namespace gdb
