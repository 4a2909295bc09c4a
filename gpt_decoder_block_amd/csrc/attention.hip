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
//   backward: two deterministic kernels that each recompute P from the saved
//     log-sum-exp:
//       dQ: a workgroup of 8 waves owns 256 query rows and loops over the
//         visible key tiles, dQ^T += K^T dS^T; it also forms
//         delta_i = dO_i . O_i from the dO rows it holds and writes it;
//       dK/dV (after dQ): a workgroup of 4 waves owns 128 keys of one
//         (b, kv head) and loops over the query heads of its group and the
//         visible query rows, 32 at a time through two LDS stages,
//         accumulating dV^T += dO^T P and
//         dK^T += Q^T dS in registers (the GQA head reduction happens in
//         registers, no atomics).
// fp32 path: one thread per query (or key) row; slow, exact reference-order
// kernels for the fp32 mode.
#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace gdb {

namespace {

constexpr int HD = 128;  // head_dim of the MFMA path
// Two waves on every SIMD, so that one wave's softmax overlaps the other's
// MFMAs: the forward and dK/dV run two workgroups of 4 waves per CU (the
// workgroups synchronise independently, so the two waves of a SIMD are not
// held in step by a shared barrier), dQ one workgroup of 8 waves (measured
// faster for it).
#ifndef ATTN_NW
#define ATTN_NW 4
#define ATTN_IB 1
#endif
#ifndef ATTN_NS
#define ATTN_NS 2
#endif
#ifndef ATTN_DQ_NW
#define ATTN_DQ_NW 8
#endif
#ifndef ATTN_DQ_NS
#define ATTN_DQ_NS 3
#endif
#ifndef ATTN_DKV_NW
#define ATTN_DKV_NW 4
#endif
#ifndef ATTN_DKV_NS
#define ATTN_DKV_NS 2
#endif
#ifndef ATTN_DKV_SR
#define ATTN_DKV_SR 32
#endif
constexpr int ATTN_FQ = 32 * ATTN_IB * ATTN_NW;  // query rows per forward workgroup
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;

// Tiles are [64 rows][128] bf16 in LDS, row-major (256 B per row), with the
// 16-byte chunk index XOR-swizzled by f(row) = 4(row & 3) + ((row >> 2) & 3).
// f is a bijection on any 16 consecutive aligned rows, so a row-fragment read
// (16 lanes, 16 rows, one logical chunk) touches 16 distinct chunks; and in a
// transposed read (32 lanes: 4 rows x 2 adjacent chunk pairs) the row term
// lands in chunk bits 2-3 while the column term stays in bits 0-1, so those
// 32 lanes also hit 16 distinct chunks: both are free of bank conflicts.
// Tiles are filled by direct global->LDS loads (no staging registers): in
// each wave instruction, lane L writes the 16 bytes at LDS base + 16L, so
// lane L fetches the logical chunk that belongs at physical chunk L%16 of
// row L/16.
__device__ __forceinline__ int kswz(int row, int chunk) { return chunk ^ (((row & 3) << 2) | ((row >> 2) & 3)); }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Issue the direct loads of a 64-row tile, 16/NW per wave of an NW-wave
// workgroup (one load = 4 rows); rows past nrows are clamped to the last row
// (finite values that every use masks out).
template <int NW = 4>
__device__ __forceinline__ void tile_async(const bf16* base, size_t ld, int row0, int nrows, bf16* S) {
  constexpr int RW = 64 / NW;  // rows per wave
  const int t = threadIdx.x, w = t >> 6, L = t & 63;
#pragma unroll
  for (int i = 0; i < RW / 4; ++i) {
    const int r = w * RW + i * 4 + (L >> 4);
    const int c = kswz(r, L & 15);
    int row = row0 + r;
    row = row < nrows ? row : nrows - 1;
    __builtin_amdgcn_global_load_lds((const void*)(base + (size_t)row * ld + c * 8), (lds_ptr)(S + (w * RW + i * 4) * HD),
                                     16, 0, 0);
  }
}

// The same copy through a buffer resource over the operand (32-bit byte
// offsets; the host checks that a sequence's rows fit), for the forward and
// dQ loops that keep copies in flight while they read another stage.  The
// compiler inserts a wait for pending LDS copies before any LDS read that may
// alias them, and with global_load_lds into a stage array it could not tell
// the stages apart: a vmcnt(0) before every other tile's reads drained the
// prefetch.  Here the destination's origin is hidden, so no such wait is
// inserted; the kernels wait for their own copies explicitly before the
// barrier that publishes a stage.  dK/dV copies Q and dO this way too: the
// base sits in scalar registers and each lane adds a 32-bit offset, about 24
// fewer vector instructions per query tile than 64-bit lane addresses (the
// whole backward 1.5-2% faster).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const bf16* base, size_t ld, int nrows) {
  const size_t bytes = nrows > 0 ? ((size_t)(nrows - 1) * ld + HD) * 2 : 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(base), (short)0, (int)min(bytes, (size_t)0x7FFFFFF0),
                                           0x00020000);
}
template <int NW = 4, int ROWS = 64>
__device__ __forceinline__ void tile_async(__amdgpu_buffer_rsrc_t rs, size_t ld, int row0, int nrows, bf16* S) {
  static_assert(ROWS % (4 * NW) == 0, "whole 4-row loads per wave");
  constexpr int RW = ROWS / NW;  // rows per wave
  const int t = threadIdx.x, w = __builtin_amdgcn_readfirstlane(t >> 6), L = t & 63;
#pragma unroll
  for (int i = 0; i < RW / 4; ++i) {
    const int r = w * RW + i * 4 + (L >> 4);
    const int c = kswz(r, L & 15);
    int row = row0 + r;
    row = row < nrows ? row : nrows - 1;
    lds_ptr d = (lds_ptr)(S + (w * RW + i * 4) * HD);
    asm volatile("" : "+s"(d));  // hide the destination's origin from the alias analysis
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, ((unsigned)row * (unsigned)ld + c * 8) * 2u, 0, 0, 0);
  }
}

// 64 floats (one per lane) straight into LDS; index clamped to n - 1.  The
// destination's origin is hidden like the buffer copies' above: otherwise
// the compiler waits for every copy in flight (vmcnt(0)) before the first
// read of any LDS array these rows might alias, which in dK/dV drained the
// next stage's Q/dO copies right after the S products.
__device__ __forceinline__ void vec64_async(const float* src, int i0, int n, float* S) {
  const int L = threadIdx.x & 63;
  int i = i0 + L;
  i = i < n ? i : n - 1;
  lds_ptr d = (lds_ptr)S;
  asm volatile("" : "+s"(d));  // hide the destination's origin from the alias analysis
  __builtin_amdgcn_global_load_lds((const void*)(src + i), d, 4, 0, 0);
}

// MFMA operand with rows = tile rows (A of S = K Q^T etc.): lane (row lr of
// block rb, half lh) reads columns kk*16 + 8lh .. +7.
__device__ __forceinline__ bf16x8 row_frag(const bf16* S, int rb, int kk, int lr, int lh) {
  const int row = rb * 32 + lr;
  return *(const bf16x8*)(S + row * HD + kswz(row, 2 * kk + lh) * 8);
}

__device__ __forceinline__ bf16x4 tr_read(const bf16* p) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p));
}

// Transposed operand read with the gfx950 LDS transpose load: the MFMA A
// operand with rows = tile columns d (block db) and contraction over tile
// rows: lane (d = 32db + lane%32, lh) gets rows 16ks + 8(e/4) + 4lh + e%4,
// e = 0..7.  In each 16-lane group the hardware returns to lane i element i%4
// of the 8 bytes addressed by lane 4j + i/4 (j = 0..3), so source lane s
// addresses row k0 + s/4, columns dbase + 4(s%4) .. +3.
__device__ __forceinline__ bf16x8 tr_frag(const bf16* S, int db, int ks, int lane) {
  const int G = lane >> 4, sl = lane & 15;
  const int lh = G >> 1;
  const int col = 32 * db + 16 * (G & 1) + 4 * (sl & 3);
  const int r0 = 16 * ks + 4 * lh + (sl >> 2);
  const int r1 = r0 + 8;
  const bf16x4 lo = tr_read(S + r0 * HD + (kswz(r0, col >> 3) << 3) + (col & 7));
  const bf16x4 hi = tr_read(S + r1 * HD + (kswz(r1, col >> 3) << 3) + (col & 7));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// written with non-short-circuit operators so that it compiles to compares
// and a select, never to a branch per element
__device__ __forceinline__ bool visible(int i, int j, int T, int W) {
  return (j < T) & (j <= i) & ((W < 0) | (i - j <= W));
}

// wait until at most N vector-memory operations of this wave are in flight
// (the builtin, so that the compiler's own wait insertion knows which loads
// are complete; gfx9 encoding: vmcnt in bits 3:0, expcnt 7, lgkmcnt 15)
#define WAIT_VM(N) __builtin_amdgcn_s_waitcnt(0xF70 | (N))
// workgroup barrier that waits for this wave's LDS accesses but leaves its
// copies into LDS in flight (__syncthreads waits for every one: vmcnt(0))
#define LDS_BARRIER() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")

// ----------------------------------------------------------------- forward
// Workgroup: 32*IB*NW query rows of one (b, h); wave w owns IB blocks of 32
// rows (the K and V fragments read from LDS serve every block of the wave).
// Lane (lr, lh) of block ib holds query q0 + 32*IB*w + 32ib + lr.  K and V
// tiles of 64 keys stream through NS LDS stages, NS - 1 tiles ahead.
//
// BOUNDED: q^ and k^ come out of the QK RMS-norm (no affine), so each has
// norm <= sqrt(D) and every score q^.k^/sqrt(D) lies in [-sqrt(D), sqrt(D)].
// Softmax is invariant to a shift, so the fixed offset M = sqrt(D) (with 1%
// margin for bf16 rounding of q^, k^) replaces the running row max: no max
// reduction, no rescaling of O, and exp never overflows.  Otherwise the usual
// online max with rescaling.

// Scores the lane may not see become -inf in place, so the exponentials
// that follow give exactly 0; called on tiles that cross the band's edge
// only.  Register v of block jb holds the pair (fixed, var0 + 32jb +
// 8(v>>2) + 4lh + (v&3)), the fixed index being the lane's own query (forward,
// dQ: var = key) or key (dK/dV: var = query).
template <bool VAR_IS_KEY, int NB>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[NB], int fixed, int var0, int lh, int T, int W) {
  // visible iff lo <= c <= hi for the register's compile-time offset
  // c = 32jb + 8(v>>2) + (v&3) from this lane's first index var0 + 4lh
  const int base = var0 + 4 * lh;
  constexpr int FAR = 1 << 29;  // beyond any offset, no overflow
  int lo, hi;
  if (VAR_IS_KEY) {  // fixed = query i, var = key j: j <= i, j < T, i - j <= W
    hi = min(fixed, T - 1) - base;
    lo = W >= 0 ? fixed - W - base : -FAR;
  } else {           // fixed = key j, var = query i: j <= i, i < T, i - j <= W, j < T
    lo = fixed - base;
    hi = (W >= 0 ? min(T - 1, fixed + W) : T - 1) - base;
    if (fixed >= T) hi = -FAR;
  }
#pragma unroll
  for (int jb = 0; jb < NB; ++jb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int c = jb * 32 + 8 * (v >> 2) + (v & 3);
      s[jb][v] = ((c >= lo) & (c <= hi)) ? s[jb][v] : -INFINITY;
    }
}

// Probabilities of one 32-query x 64-key tile for this lane's query (hidden
// keys already at -inf), written straight into the bf16 operand registers of
// the P V^T MFMA (pk[ks] = keys 16ks..16ks+15 in contraction-slot order).
// The row sum l accumulates the bf16-rounded weights (v_dot2 with ones), so
// O is an exact convex combination of V rows whatever the rounding of P.
template <bool BOUNDED>
__device__ __forceinline__ void softmax_pack(const f32x16 (&s)[2], bf16x8 (&pk)[4], float scale_log2, float& m,
                                             float& l, float& alpha) {
  float msafe;
  if (BOUNDED) {
    msafe = m;
    alpha = 1.0f;
  } else {
    float mx = -INFINITY;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[jb][v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // running max in the log2 domain (scores scaled by scale*log2(e))
    const float mnew = fmaxf(m, mx * scale_log2);
    msafe = mnew == -INFINITY ? 0.f : mnew;
    alpha = __builtin_amdgcn_exp2f(m - msafe);  // exactly 1 when the max did not move
    l *= alpha;
    m = mnew;
  }
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    bf16x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int jb = ks >> 1, v = 8 * (ks & 1) + e;
      out[e] = (bf16)__builtin_amdgcn_exp2f(fmaf(s[jb][v], scale_log2, -msafe));
    }
    pk[ks] = out;
    typedef bf16x2 bf16x2x4[4];
    const auto& pairs = *reinterpret_cast<const bf16x2x4*>(&pk[ks]);
#pragma unroll
    for (int q = 0; q < 4; ++q) l = __builtin_amdgcn_fdot2_f32_bf16(pairs[q], ones, l, false);
  }
}

template <int IB, bool BOUNDED, int NW, int NS>
__global__ __launch_bounds__(64 * NW) void attn_fwd_bf16_k(AttnArgs a, float scale_log2) {
  static_assert(NS == 2 || NS == 3, "two or three K/V stages");
  constexpr int FQ = 32 * IB * NW;
  __shared__ __attribute__((aligned(16))) bf16 Ks[NS][64 * HD];
  __shared__ __attribute__((aligned(16))) bf16 Vs[NS][64 * HD];
  const int T = a.T, H = a.H, Hkv = a.Hkv, W = a.window;
  // grid (B*H, query blocks): every head's heaviest query block is dispatched first
  const int nqb = (T + FQ - 1) / FQ;
  const int qb = nqb - 1 - (int)blockIdx.y;
  const int b = blockIdx.x / H, h = blockIdx.x % H, g = h / (H / Hkv);
  const int q0 = qb * FQ;
  const int t = threadIdx.x, lane = t & 63, lr = lane & 31, lh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform: tile tests become scalar branches
  const int qw0 = q0 + w * 32 * IB;          // first query of this wave
  const bf16* base = (const bf16*)a.qkv + (size_t)b * T * a.ld;
  const bf16* kbase = base + (H + g) * HD;
  const bf16* vbase = base + (H + Hkv + g) * HD;
  const auto krs = tile_rsrc(kbase, a.ld, T), vrs = tile_rsrc(vbase, a.ld, T);

  int kv_lo = W >= 0 ? max(0, q0 - W) : 0;
  kv_lo &= ~63;
  const int kv_hi = min(T, q0 + FQ);
  const int ntile = (kv_hi - kv_lo + 63) / 64;
  // this wave's visible key range
  const int wq_hi = min(qw0 + 32 * IB - 1, T - 1);
  const int wk_lo = W >= 0 ? max(0, qw0 - W) : 0;

  tile_async<NW>(krs, a.ld, kv_lo, T, Ks[0]);
  tile_async<NW>(vrs, a.ld, kv_lo, T, Vs[0]);
  if (NS == 3 && ntile > 1) {
    tile_async<NW>(krs, a.ld, kv_lo + 64, T, Ks[1]);
    tile_async<NW>(vrs, a.ld, kv_lo + 64, T, Vs[1]);
  }

  bf16x8 qf[IB][8];
#pragma unroll
  for (int ib = 0; ib < IB; ++ib) {
    const int qi = min(qw0 + ib * 32 + lr, T - 1);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qf[ib][kk] = *(const bf16x8*)(base + (size_t)qi * a.ld + h * HD + kk * 16 + lh * 8);
  }
  f32x16 o[IB][4];
  float m[IB], l[IB];
#pragma unroll
  for (int ib = 0; ib < IB; ++ib) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[ib][i] = f32x16{};
    m[ib] = BOUNDED ? 1.01f * sqrtf((float)HD) * scale_log2 : -INFINITY;
    l[ib] = 0.f;
  }
  WAIT_VM(0);
  __syncthreads();

  // the stage index is a compile-time constant in each copy of the tile
  // step, so every LDS address is a per-lane base plus an immediate offset
  auto tile_step = [&](int it, auto stc) {
    constexpr int ST = decltype(stc)::value;
    constexpr int st = ST;
    const int kv0 = kv_lo + it * 64;
    // NS = 3: tile it+2 goes into the stage read two steps ago; NS = 2: tile
    // it+1 into the stage read in the previous step (both freed by its barrier)
    const bool ahead = it + NS - 1 < ntile;
    if (ahead) {
      constexpr int sn = (ST + NS - 1) % NS;
      tile_async<NW>(krs, a.ld, kv0 + 64 * (NS - 1), T, Ks[sn]);
      tile_async<NW>(vrs, a.ld, kv0 + 64 * (NS - 1), T, Vs[sn]);
    }
    // wave-uniform: does the tile touch this wave's rows, and is it fully visible?
    const bool any = qw0 < T && kv0 <= wq_hi && kv0 + 63 >= wk_lo;
    if (any) {
      const bool full = kv0 + 63 <= qw0 && kv0 + 63 < T && (W < 0 || wq_hi - kv0 <= W);
      f32x16 s[IB][2];
#pragma unroll
      for (int ib = 0; ib < IB; ++ib) s[ib][0] = s[ib][1] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
          const bf16x8 kf = row_frag(Ks[st], jb, kk, lr, lh);
#pragma unroll
          for (int ib = 0; ib < IB; ++ib) s[ib][jb] = mfma32(kf, qf[ib][kk], s[ib][jb]);
        }
      }
      bf16x8 pk[IB][4];
#pragma unroll
      for (int ib = 0; ib < IB; ++ib) {
        const int qi = qw0 + ib * 32 + lr;
        float alpha;
        if (!full) mask_tile<true>(s[ib], qi, kv0, lh, T, W);
        softmax_pack<BOUNDED>(s[ib], pk[ib], scale_log2, m[ib], l[ib], alpha);
        if (!BOUNDED && __any(alpha != 1.0f)) {
#pragma unroll
          for (int db = 0; db < 4; ++db) o[ib][db] *= alpha;
        }
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16x8 vf = tr_frag(Vs[st], db, ks, lane);
#pragma unroll
          for (int ib = 0; ib < IB; ++ib) o[ib][db] = mfma32(vf, pk[ib][ks], o[ib][db]);
        }
      }
    }
    if (NS == 3 && ahead) {  // tile it+1 landed; tile it+2 may still be in flight
      if constexpr (NW == 8) WAIT_VM(4);
      else WAIT_VM(8);
    } else {
      WAIT_VM(0);
    }
    __syncthreads();
  };
  for (int it = 0; it < ntile; it += NS) {
    tile_step(it, std::integral_constant<int, 0>{});
    if (it + 1 < ntile) tile_step(it + 1, std::integral_constant<int, 1>{});
    if constexpr (NS == 3) {
      if (it + 2 < ntile) tile_step(it + 2, std::integral_constant<int, 2 % NS>{});
    }
  }

#pragma unroll
  for (int ib = 0; ib < IB; ++ib) {
    const int qi = qw0 + ib * 32 + lr;
    const float lt = l[ib] + __shfl_xor(l[ib], 32, 64);
    if (qi < T) {
      const float inv = 1.0f / lt;
      bf16* orow = (bf16*)a.o + ((size_t)b * T + qi) * a.ldo + h * HD;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int d = db * 32 + 8 * gq + 4 * lh;
          *(bf16x4*)(orow + d) = bf16x4{(bf16)(o[ib][db][4 * gq] * inv), (bf16)(o[ib][db][4 * gq + 1] * inv),
                                        (bf16)(o[ib][db][4 * gq + 2] * inv), (bf16)(o[ib][db][4 * gq + 3] * inv)};
        }
      if (lh == 0) a.lse[((size_t)b * H + h) * T + qi] = (m[ib] + __log2f(lt)) * 0.69314718055994531f;
    }
  }
}

// ------------------------------------------------------- backward: delta
template <typename T_>
__global__ __launch_bounds__(256) void attn_delta_k(AttnArgs a) {
  // one wave per token: 16-byte vectors of O and dO, a head's D elements on
  // G = D/VN consecutive lanes, summed by a butterfly over those lanes
  constexpr int VN = V16<T_>::n;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6), l = threadIdx.x & 63;
  const int N = a.B * a.T;
  if (n >= N) return;  // wave-uniform
  const int G = a.D / VN, nchunk = a.H * G;
  const T_* o = (const T_*)a.o + (size_t)n * a.ldo;
  const T_* d = (const T_*)a.dout + (size_t)n * a.lddo;
  const int b = n / a.T, t = n % a.T;
  for (int base = 0; base < nchunk; base += 64) {
    const int ci = base + l;
    float s = 0.f;
    if (ci < nchunk) {
      float x[VN], y[VN];
      ld16(o + ci * VN, x);
      ld16(d + ci * VN, y);
#pragma unroll
      for (int e = 0; e < VN; ++e) s += x[e] * y[e];
    }
    for (int off = G / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    const int h = ci / G;
    if (ci < nchunk && (l % G) == 0) a.delta[((size_t)b * a.H + h) * a.T + t] = s;
  }
}

// Backward of y = rope(rms(x)) for one head row held by a lane pair (lh = 0,
// 1), in the accumulator layout of the backward kernels: register 4gq + e of
// block db is d = 32db + 8gq + 4lh + e.  g = gscale * acc is dL/dy; with
// m = (g . y) / D, u = g - m y (the radial part removed), dL/dx is the inverse
// rotation of u times rinv.  Rotary pair (j, j + 64) is (block db, block
// db + 2) of the same lane.  y is the saved row, cs the (cos, sin) row of the
// position; the result goes to out at the same d.
__device__ __forceinline__ void qknorm_rope_bwd_row(const f32x16 (&acc)[4], float gscale, const bf16* __restrict__ y,
                                                    float rinv, const float* __restrict__ cs, int lh,
                                                    bf16* __restrict__ out) {
  bf16x4 yv[4][4];
  float dot = 0.f;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      yv[db][gq] = *(const bf16x4*)(y + db * 32 + 8 * gq + 4 * lh);
#pragma unroll
      for (int e = 0; e < 4; ++e) dot += acc[db][4 * gq + e] * gscale * (float)yv[db][gq][e];
    }
  dot += __shfl_xor(dot, 32, 64);
  const float m = dot * (1.0f / HD);
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int j0 = db * 32 + 8 * gq + 4 * lh;
      const f32x4 c0 = *(const f32x4*)(cs + 2 * j0), c1 = *(const f32x4*)(cs + 2 * j0 + 4);
      const float c[4] = {c0[0], c0[2], c1[0], c1[2]}, sn[4] = {c0[1], c0[3], c1[1], c1[3]};
      bf16x4 oa, ob;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ua = acc[db][4 * gq + e] * gscale - (float)yv[db][gq][e] * m;
        const float ub = acc[db + 2][4 * gq + e] * gscale - (float)yv[db + 2][gq][e] * m;
        oa[e] = (bf16)(rinv * (ua * c[e] + ub * sn[e]));
        ob[e] = (bf16)(rinv * (-ua * sn[e] + ub * c[e]));
      }
      *(bf16x4*)(out + j0) = oa;
      *(bf16x4*)(out + j0 + 64) = ob;
    }
}

// ------------------------------------------------------ backward: dK, dV
// Workgroup: 32*NW keys of one (b, kv head), 32 per wave (lane = key).  Two
// 4-wave workgroups share a CU (NW = 4, 78 KiB of LDS each), so the two
// waves of a SIMD belong to different workgroups and one's exp/convert work
// overlaps the other's MFMAs without a common barrier.  The workgroup's V
// rows sit in LDS for the whole kernel (the wave's K rows stay in
// registers).  Loops over the query heads of the group and the visible
// 64-row query tiles; Q, dO (row-major) and the rows' log-sum-exp and delta
// go through NS LDS stages of SR rows (SR = 64, NS = 1: the next tile is
// copied once every wave has read this one, the other workgroup computing
// meanwhile; SR = 32, NS = 2, the default: each stage holds half a tile and
// the next half is in flight while this one is used, in the same LDS).
// Each tile is taken as two 32-query halves: S, then P (kept in fp32 in
// place of S) into dV^T += dO^T P, then dP and dS into dK^T += Q^T dS, so
// at most S and dP of one half are live; the transposed operands come from
// the LDS transpose load.  A wave has 256 registers; the accumulators take
// 128, so KX of its eight K fragments wait in LDS rather than in scratch,
// whose reloads would also wait for copies in flight (vector-memory counts
// retire in order): at NW = 4, KX = 3 the kernel needs 247 registers and
// no scratch (SR = 64, NS = 1: 256 registers and an 8-byte spill).
template <int NW, int KX = 3, int NS = 2, int SR = 64>
__global__ __launch_bounds__(64 * NW, NW == 4 ? 2 : 1) void attn_bwd_dkv_bf16_k(AttnArgs a, float scale_log2,
                                                                               float scale) {
  static_assert(NS == 1 || NS == 2, "one or two Q/dO stages");
  static_assert(SR == 64 || (SR == 32 && NS == 2), "a stage holds a 64-row query tile or half of one");
  constexpr int FK = 32 * NW;
  constexpr int HPT = 64 / SR;  // stages per 64-row query tile
  __shared__ __attribute__((aligned(16))) bf16 Vs[FK * HD];
  __shared__ __attribute__((aligned(16))) bf16 Qs[NS][SR * HD];
  __shared__ __attribute__((aligned(16))) bf16 Ds[NS][SR * HD];
  __shared__ __attribute__((aligned(16))) float Ls[NS][NW][64];  // [stage][wave: lse (even), delta (odd)][row]
  // the last KX of the wave's eight K fragments, parked in LDS (private to
  // the wave) to free registers
  __shared__ __attribute__((aligned(16))) bf16x8 Kx[NW][KX > 0 ? KX : 1][64];
  const int T = a.T, H = a.H, Hkv = a.Hkv, W = a.window, G = H / Hkv;
  const int b = blockIdx.x / Hkv, g = blockIdx.x % Hkv;   // grid (B*Hkv, key blocks)
  const int kv0 = blockIdx.y * FK;
  const int t = threadIdx.x, lane = t & 63, lr = lane & 31, lh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform: tile tests become scalar branches
  const int kj = kv0 + w * 32 + lr;  // this lane's key
  const bf16* base = (const bf16*)a.qkv + (size_t)b * T * a.ld;
  const bf16* dbase = (const bf16*)a.dout + (size_t)b * T * a.lddo;

  const int q_lo = kv0;  // multiple of 64
  const int q_hi = W >= 0 ? min(T, kv0 + FK + W) : T;
  const int nqt = q_hi > q_lo ? (q_hi - q_lo + 63) / 64 : 0;
  const int total = nqt * G * HPT;  // stage fills: (query head, query tile, part of the tile)
  // wave's keys
  const int wk0 = kv0 + w * 32, wk_hi = min(wk0 + 31, T - 1);
  // first query row of stage fill `it`
  auto row0 = [&](int it) { return q_lo + ((it / HPT) % nqt) * 64 + (it % HPT) * SR; };

  // every wave issues the same number of loads per fill (2 x SR/(4 NW) + 1)
  auto issue = [&](int it, int stg) {
    const int hh = g * G + it / (HPT * nqt);
    const int i0 = row0(it);
    tile_async<NW, SR>(tile_rsrc(base + hh * HD, a.ld, T), a.ld, i0, T, Qs[stg]);
    tile_async<NW, SR>(tile_rsrc(dbase + hh * HD, a.lddo, T), a.lddo, i0, T, Ds[stg]);
    const size_t lo = ((size_t)b * H + hh) * T;
    vec64_async((w & 1) ? a.delta + lo : a.lse + lo, i0, T, Ls[stg][w]);
  };
#pragma unroll
  for (int r = 0; r < FK; r += 64) tile_async<NW>(base + (H + Hkv + g) * HD, a.ld, kv0 + r, T, Vs + r * HD);
  if (total > 0) issue(0, 0);

  bf16x8 kf[8 - KX];
  {
    const int kc = min(kj, T - 1);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const bf16x8 v = *(const bf16x8*)(base + (size_t)kc * a.ld + (H + g) * HD + kk * 16 + lh * 8);
      if (kk < 8 - KX) kf[kk < 8 - KX ? kk : 0] = v;
      else Kx[w][kk >= 8 - KX ? kk - (8 - KX) : 0][lane] = v;
    }
  }
  f32x16 dk[4], dv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { dk[i] = f32x16{}; dv[i] = f32x16{}; }
  WAIT_VM(0);
  __syncthreads();

  for (int it = 0; it < total; ++it) {
    const int st = NS == 2 ? it & 1 : 0;
    const int i0 = row0(it);
    // two stages: the other stage was last read in iteration it-1, which
    // every wave has left; one stage: the next tile is copied after this one
    // has been read (the other workgroup on the CU computes meanwhile)
    if (NS == 2 && it + 1 < total) issue(it + 1, st ^ 1);
    // wave-uniform visibility of this stage's query rows for the wave's 32 keys
    const int iq_hi = min(i0 + SR - 1, T - 1);
    const bool any = wk0 < T && i0 + SR - 1 >= wk0 && (W < 0 || i0 - wk_hi <= W);
    if (any) {
      const bool full = i0 >= wk_hi && iq_hi < T && (W < 0 || iq_hi - wk0 <= W) && i0 + SR - 1 < T;
#pragma unroll
      for (int ib = 0; ib < SR / 32; ++ib) {
        // query rows 32ib..32ib+31: lane = key j, registers = queries.  S
        // first; P (kept in fp32 in place of S) feeds dV before dP is
        // computed, so P's bf16 copy and dP are never live together
        f32x16 sv = f32x16{};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk)
          sv = mfma32(row_frag(Qs[st], ib, kk, lr, lh), kk < 8 - KX ? kf[kk < 8 - KX ? kk : 0] : Kx[w][kk >= 8 - KX ? kk - (8 - KX) : 0][lane], sv);
        if (!full) {
          f32x16 sm[1] = {sv};
          mask_tile<false>(sm, kj, i0 + ib * 32, lh, T, W);
          sv = sm[0];
        }
        // P straight into bf16 operand registers (slot order of tr_frag)
        bf16x8 pf[2];
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const f32x4 L4 = *(const f32x4*)(&Ls[st][0][ib * 32 + 8 * gq + 4 * lh]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int v = 4 * gq + r;
            sv[v] = __builtin_amdgcn_exp2f(fmaf(sv[v], scale_log2, -L4[r] * 1.4426950408889634f));
            pf[gq >> 1][4 * (gq & 1) + r] = (bf16)sv[v];
          }
        }
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int db = 0; db < 4; ++db) dv[db] = mfma32(tr_frag(Ds[st], db, 2 * ib + k2, lane), pf[k2], dv[db]);
        f32x16 dpv = f32x16{};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) dpv = mfma32(row_frag(Ds[st], ib, kk, lr, lh), row_frag(Vs, w, kk, lr, lh), dpv);
        bf16x8 sf[2];
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const f32x4 D4 = *(const f32x4*)(&Ls[st][1][ib * 32 + 8 * gq + 4 * lh]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int v = 4 * gq + r;
            sf[gq >> 1][4 * (gq & 1) + r] = (bf16)(sv[v] * (dpv[v] - D4[r]));
          }
        }
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int db = 0; db < 4; ++db) dk[db] = mfma32(tr_frag(Qs[st], db, 2 * ib + k2, lane), sf[k2], dk[db]);
      }
    }
    if (NS == 1) {
      __syncthreads();  // every wave has read the stage
      if (it + 1 < total) issue(it + 1, 0);
    }
    WAIT_VM(0);  // tile it+1 has landed
    __syncthreads();
  }

  if (kj < T) {
    bf16* row = (bf16*)a.dqkv + ((size_t)b * T + kj) * a.lddq;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = db * 32 + 8 * gq + 4 * lh;
        if (!a.rope)
          *(bf16x4*)(row + (H + g) * HD + d) =
              bf16x4{(bf16)(dk[db][4 * gq] * scale), (bf16)(dk[db][4 * gq + 1] * scale),
                     (bf16)(dk[db][4 * gq + 2] * scale), (bf16)(dk[db][4 * gq + 3] * scale)};
        *(bf16x4*)(row + (H + Hkv + g) * HD + d) =
            bf16x4{(bf16)dv[db][4 * gq], (bf16)dv[db][4 * gq + 1], (bf16)dv[db][4 * gq + 2], (bf16)dv[db][4 * gq + 3]};
      }
    if (a.rope)
      qknorm_rope_bwd_row(dk, scale, base + (size_t)kj * a.ld + (H + g) * HD,
                          a.rinv[((size_t)b * T + kj) * (H + Hkv) + H + g], a.rope + (size_t)kj * HD, lh,
                          row + (H + g) * HD);
  }
}

// ------------------------------------------------------------ backward: dQ
// Workgroup: 32*NW query rows of one (b, h), 32 per wave (lane = query).  K
// and V tiles of 64 keys stream through NS LDS stages, NS - 1 tiles ahead;
// dQ^T += K^T dS^T with K^T read by the LDS transpose load.
template <int NW, int NS>
__global__ __launch_bounds__(64 * NW, NW == 4 ? 2 : 1) void attn_bwd_dq_bf16_k(AttnArgs a, float scale_log2,
                                                                              float scale) {
  static_assert(NS == 2 || NS == 3, "two or three K/V stages");
  constexpr int FQ = 32 * NW;
  __shared__ __attribute__((aligned(16))) bf16 Ks[NS][64 * HD];
  __shared__ __attribute__((aligned(16))) bf16 Vs[NS][64 * HD];
  const int T = a.T, H = a.H, Hkv = a.Hkv, W = a.window;
  const int nqb = (T + FQ - 1) / FQ;
  const int qb = nqb - 1 - (int)blockIdx.y;   // grid (B*H, query blocks), heaviest first
  const int b = blockIdx.x / H, h = blockIdx.x % H, g = h / (H / Hkv);
  const int q0 = qb * FQ;
  const int t = threadIdx.x, lane = t & 63, lr = lane & 31, lh = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform: tile tests become scalar branches
  const int qi = q0 + w * 32 + lr;
  const int qw0 = q0 + w * 32, wq_hi = min(qw0 + 31, T - 1);
  const int wk_lo = W >= 0 ? max(0, qw0 - W) : 0;
  const bf16* base = (const bf16*)a.qkv + (size_t)b * T * a.ld;
  const bf16* kbase = base + (H + g) * HD;
  const bf16* vbase = base + (H + Hkv + g) * HD;
  const auto krs = tile_rsrc(kbase, a.ld, T), vrs = tile_rsrc(vbase, a.ld, T);

  int kv_lo = W >= 0 ? max(0, q0 - W) : 0;
  kv_lo &= ~63;
  const int kv_hi = min(T, q0 + FQ);
  const int ntile = (kv_hi - kv_lo + 63) / 64;

  tile_async<NW>(krs, a.ld, kv_lo, T, Ks[0]);
  tile_async<NW>(vrs, a.ld, kv_lo, T, Vs[0]);
  if (NS == 3 && ntile > 1) {
    tile_async<NW>(krs, a.ld, kv_lo + 64, T, Ks[1]);
    tile_async<NW>(vrs, a.ld, kv_lo + 64, T, Vs[1]);
  }
  bf16x8 qf[8], df[8];
  const int qc = min(qi, T - 1);
  const bf16* drow = (const bf16*)a.dout + ((size_t)b * T + qc) * a.lddo + h * HD;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    qf[kk] = *(const bf16x8*)(base + (size_t)qc * a.ld + h * HD + kk * 16 + lh * 8);
    df[kk] = *(const bf16x8*)(drow + kk * 16 + lh * 8);
  }
  const size_t li = ((size_t)b * H + h) * T + qc;
  const float lse2 = a.lse[li] * 1.4426950408889634f;
  // delta_i = dO_i . O_i from the dO fragments held here (each lane of the
  // pair has half of the row); written for the dK/dV kernel, which runs next
  float dlt;
  {
    const bf16* orow = (const bf16*)a.o + ((size_t)b * T + qc) * a.ldo + h * HD;
    float pd = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const bf16x8 ov = *(const bf16x8*)(orow + kk * 16 + lh * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) pd = fmaf((float)ov[e], (float)df[kk][e], pd);
    }
    dlt = pd + __shfl_xor(pd, 32, 64);
    if (lh == 0 && qi < T) a.delta[li] = dlt;
  }
  f32x16 dq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) dq[i] = f32x16{};
  WAIT_VM(0);
  __syncthreads();

  // the stage index is a compile-time constant in each copy of the tile
  // step, so every LDS address is a per-lane base plus an immediate offset
  auto tile_step = [&](int it, auto stc) {
    constexpr int ST = decltype(stc)::value;
    constexpr int st = ST;
    const int kv0 = kv_lo + it * 64;
    // the next copy goes into the stage freed by the previous step's barrier
    const bool ahead = it + NS - 1 < ntile;
    if (ahead) {
      constexpr int sn = (ST + NS - 1) % NS;
      tile_async<NW>(krs, a.ld, kv0 + 64 * (NS - 1), T, Ks[sn]);
      tile_async<NW>(vrs, a.ld, kv0 + 64 * (NS - 1), T, Vs[sn]);
    }
    const bool any = qw0 < T && kv0 <= wq_hi && kv0 + 63 >= wk_lo;
    if (any) {
      const bool full = kv0 + 63 <= qw0 && kv0 + 63 < T && (W < 0 || wq_hi - kv0 <= W);
      f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
          s[jb] = mfma32(row_frag(Ks[st], jb, kk, lr, lh), qf[kk], s[jb]);
          dp[jb] = mfma32(row_frag(Vs[st], jb, kk, lr, lh), df[kk], dp[jb]);
        }
      }
      if (!full) mask_tile<true>(s, qi, kv0, lh, T, W);
      bf16x8 sf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int jb = ks >> 1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int v = 8 * (ks & 1) + e;
          const float p = __builtin_amdgcn_exp2f(fmaf(s[jb][v], scale_log2, -lse2));
          sf[ks][e] = (bf16)(p * (dp[jb][v] - dlt));
        }
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int db = 0; db < 4; ++db) dq[db] = mfma32(tr_frag(Ks[st], db, ks, lane), sf[ks], dq[db]);
      }
    }
    if (NS == 3 && ahead) {
      if constexpr (NW == 8) WAIT_VM(4);
      else WAIT_VM(8);
    } else {
      WAIT_VM(0);
    }
    LDS_BARRIER();
  };
  for (int it = 0; it < ntile; it += NS) {
    tile_step(it, std::integral_constant<int, 0>{});
    if (it + 1 < ntile) tile_step(it + 1, std::integral_constant<int, 1>{});
    if constexpr (NS == 3) {
      if (it + 2 < ntile) tile_step(it + 2, std::integral_constant<int, 2 % NS>{});
    }
  }
  if (qi < T) {
    bf16* row = (bf16*)a.dqkv + ((size_t)b * T + qi) * a.lddq + h * HD;
    if (a.rope) {
      qknorm_rope_bwd_row(dq, scale, base + (size_t)qi * a.ld + h * HD,
                          a.rinv[((size_t)b * T + qi) * (H + Hkv) + h], a.rope + (size_t)qi * HD, lh, row);
    } else {
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

// the bf16 kernels address a sequence's rows of qkv (and, in the backward,
// of dO) by 32-bit byte offsets
static bool offsets_fit(const AttnArgs& a) { return (size_t)a.T * a.ld * 2 <= 0x7FFFFF00ull; }
static bool bwd_offsets_fit(const AttnArgs& a) { return offsets_fit(a) && (size_t)a.T * a.lddo * 2 <= 0x7FFFFF00ull; }

hipError_t attn_fwd(int dt, const AttnArgs& a, hipStream_t s) {
  if (a.B * a.T == 0) return hipSuccess;
  if (dt == BF16 && !offsets_fit(a)) return hipErrorInvalidValue;
  const float scale = 1.0f / sqrtf((float)a.D);
  if (dt == BF16) {
    if (a.qk_normed) {
      dim3 g(a.B * a.H, (a.T + ATTN_FQ - 1) / ATTN_FQ);
      hipLaunchKernelGGL((attn_fwd_bf16_k<ATTN_IB, true, ATTN_NW, ATTN_NS>), g, dim3(64 * ATTN_NW), 0, s, a,
                         scale * 1.4426950408889634f);
    } else {
      dim3 g(a.B * a.H, (a.T + 127) / 128);
      hipLaunchKernelGGL((attn_fwd_bf16_k<1, false, 4, 3>), g, dim3(256), 0, s, a, scale * 1.4426950408889634f);
    }
  } else {
    dim3 g((a.B * a.H * a.T + 63) / 64);
    if (a.D == 64) hipLaunchKernelGGL(attn_fwd_f32_k<64>, g, dim3(64), 0, s, a, scale);
    else hipLaunchKernelGGL(attn_fwd_f32_k<128>, g, dim3(64), 0, s, a, scale);
  }
  return hipGetLastError();
}

hipError_t attn_bwd(int dt, const AttnArgs& a, hipStream_t s) {
  if (a.B * a.T == 0) return hipSuccess;
  if (dt == BF16 && !bwd_offsets_fit(a)) return hipErrorInvalidValue;
  const float scale = 1.0f / sqrtf((float)a.D);
  if (dt == BF16) {
    // dQ first: it also writes delta, which dK/dV reads
    hipLaunchKernelGGL((attn_bwd_dq_bf16_k<ATTN_DQ_NW, ATTN_DQ_NS>), dim3(a.B * a.H, (a.T + 32 * ATTN_DQ_NW - 1) / (32 * ATTN_DQ_NW)),
                       dim3(64 * ATTN_DQ_NW), 0, s, a,
                       scale * 1.4426950408889634f, scale);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_bwd_dkv_bf16_k<ATTN_DKV_NW, 3, ATTN_DKV_NS, ATTN_DKV_SR>), dim3(a.B * a.Hkv, (a.T + 32 * ATTN_DKV_NW - 1) / (32 * ATTN_DKV_NW)),
                       dim3(64 * ATTN_DKV_NW), 0, s, a, scale * 1.4426950408889634f, scale);
  } else {
    const int rows = a.B * a.T;  // one wave per token
    hipLaunchKernelGGL(attn_delta_k<float>, dim3((rows + 3) / 4), dim3(256), 0, s, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
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
