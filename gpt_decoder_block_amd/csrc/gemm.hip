// GEMMs of the block and the lm_head: C[m, n] = sum_k A(m, k) * B(n, k) with
// either operand stored K-contiguous or M/N-contiguous, fused epilogues
// (residual add, ReLU² with its saved pre-activation, ReLU² backward, fp32
// weight-gradient output with split-K).
//
// bf16 path (gfx950 MFMA, v_mfma_f32_32x32x16_bf16):
//   * 256x256 output tile per workgroup, K step 64, 256 threads = 4 waves in a
//     2x2 grid, each wave a 128x128 sub-tile = 4x4 MFMA blocks of 32x32;
//   * both operands are staged in LDS K-contiguous ([row][64 k], 128 B rows)
//     with the 16-byte chunk index XOR-swizzled by (row ^ row>>3) & 7, so the
//     fragment reads (32 consecutive rows, one chunk) and the stores of both
//     loaders are bank-conflict free;
//   * an operand stored M- (or N-) contiguous is read as 8x8 blocks (eight
//     16-byte loads along m at eight consecutive k) and transposed in
//     registers before the LDS store, so every global access is a coalesced
//     16-byte load and the MFMA loop never sees the layout;
//   * two LDS stages: the next K tile is fetched into registers while the MFMAs
//     run on the current stage, one barrier per K step;
//   * the MFMA is issued with the B fragment as its first operand, so each lane
//     ends up holding 4 consecutive n of one output row m (8-byte bf16 or
//     16-byte fp32 stores);
//   * tile ids are remapped so that each XCD (blocks are dealt round-robin to
//     the 8 XCDs) works on a contiguous, grouped range of tiles and reuses
//     A rows / B columns in its own L2.
// fp32 path: plain LDS-tiled FMA GEMM (64x64 tile, 4x4 per thread).
#include "common.h"
#include "kernels.h"

namespace gdb {

namespace {

constexpr int BM = 256, BN = 256, BK = 64, NTHR = 256;
constexpr int TILE_ELEMS = BM * BK;  // elements of one operand tile

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over [base, base + bytes): loads at offsets >= bytes return
// zero, which implements the ragged-edge predication without branches.
constexpr unsigned OOB = 0xFFFFFFF0u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, size_t bytes) {
  const unsigned n = bytes > 0xFFFFFF00ull ? 0xFFFFFF00u : (unsigned)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}
__device__ __forceinline__ bf16x8 bload(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// Global -> registers: 8 vectors of 8 bf16 per thread and operand, then
// registers -> LDS (K-contiguous, swizzled).  The resource is rebased at the
// tile's first row (K-major) or at (kbeg, first row) (M-major), so offsets
// stay far below 4 GiB; rows past the operand's end and k past the split's
// end read as zero.
template <bool KMAJ>
struct Loader {
  bf16x8 r[8];
  __amdgpu_buffer_rsrc_t rs;
  unsigned off0;      // byte offset of this thread's first vector at k step 0
  unsigned step;      // bytes to advance per K step
  unsigned rowstep;   // bytes between the thread's consecutive vectors
  int kcol, kend_rel; // K-major: this thread's k within a step; split end (relative)
  __device__ __forceinline__ void init(const bf16* P, int ld, int rows, int r0, int kbeg, int kend) {
    const int t = threadIdx.x;
    if (KMAJ) {
      const int c = t & 7, rr = t >> 3;
      const bf16* base = P + (size_t)r0 * ld + kbeg;
      const size_t bytes = rows > r0 ? ((size_t)(rows - r0) * ld - kbeg) * 2 : 0;
      rs = make_rsrc(base, bytes);
      off0 = (unsigned)((rr * ld + c * 8) * 2);
      step = BK * 2;
      rowstep = (unsigned)(32 * ld * 2);
      kcol = c * 8;
      kend_rel = kend - kbeg;
    } else {
      const int mc = t & 31, kb = t >> 5;
      const bf16* base = P + (size_t)kbeg * ld + r0;
      const size_t bytes = (size_t)(kend - kbeg) * ld * 2;
      rs = make_rsrc(base, bytes);
      const bool mvalid = r0 + mc * 8 < rows;
      off0 = mvalid ? (unsigned)(((kb * 8) * ld + mc * 8) * 2) : OOB;
      step = (unsigned)(BK * ld * 2);
      rowstep = (unsigned)(ld * 2);
      kcol = 0;
      kend_rel = kend - kbeg;
    }
  }
  __device__ __forceinline__ void load(int kt) {
    // invalid vectors get an offset >= 0xFFFFFFF0 (past any resource size):
    // an OR with an all-ones mask, so the compiler cannot turn it into a branch
    unsigned bad;
    if (KMAJ) bad = 0u - (unsigned)(kt * BK + kcol >= kend_rel);
    else bad = 0u - (unsigned)(off0 == OOB);
    const unsigned o = (off0 + kt * step) | (bad & OOB);
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = bload(rs, (o + i * rowstep) | (bad & OOB));
  }
  __device__ __forceinline__ void store(bf16* __restrict__ S) {
    const int t = threadIdx.x;
    if (KMAJ) {
      const int c = t & 7, rr = t >> 3;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = rr + 32 * i;
        *(bf16x8*)(S + row * BK + ((c ^ swz(row)) * 8)) = r[i];
      }
    } else {
      const int mc = t & 31, kb = t >> 5;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        bf16x8 w;
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = r[i][j];
        const int row = mc * 8 + j;
        *(bf16x8*)(S + row * BK + ((kb ^ swz(row)) * 8)) = w;
      }
    }
  }
};

__device__ __forceinline__ void tile_coords(int bid, int nbm, int nbn, int& tm, int& tn) {
  const int total = nbm * nbn;
  const int full = (total / 8) * 8;
  int logical = bid;
  if (bid < full) logical = (bid % 8) * (full / 8) + bid / 8;
  constexpr int GROUP = 8;
  const int per_group = GROUP * nbn;
  const int g = logical / per_group;
  const int first_m = g * GROUP;
  const int gsize = min(nbm - first_m, GROUP);
  const int in = logical % per_group;
  tm = first_m + in % gsize;
  tn = in / gsize;
}

// MFMA fragments of one 16-wide k sub-step: 4 row blocks of A, 4 of B.
__device__ __forceinline__ void load_frags(const bf16* As, const bf16* Bs, int kk, int wm, int wn, int lr,
                                           int lh, bf16x8* af, bf16x8* bfr) {
  const int ch = kk * 2 + lh;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = wm * 128 + i * 32 + lr;
    af[i] = *(const bf16x8*)(As + row * BK + ((ch ^ swz(row)) * 8));
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = wn * 128 + j * 32 + lr;
    bfr[j] = *(const bf16x8*)(Bs + row * BK + ((ch ^ swz(row)) * 8));
  }
}

template <bool AK, bool BK_, int EPI>
__global__ __launch_bounds__(NTHR, 1) void gemm_bf16_k(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) bf16 smem[2][2][TILE_ELEMS];  // [stage][A|B]
  const int nbm = (p.M + BM - 1) / BM, nbn = (p.N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, nbm, nbn, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  // split-K range
  const int ksplit = ((p.K + p.splits * BK - 1) / (p.splits * BK)) * BK;
  const int kbeg = min(p.K, (int)blockIdx.y * ksplit);
  const int kend = min(p.K, kbeg + ksplit);
  const int nk = (kend - kbeg + BK - 1) / BK;

  Loader<AK> la;
  Loader<BK_> lb;
  la.init((const bf16*)p.A, p.lda, p.M, m0, kbeg, kend);
  lb.init((const bf16*)p.B, p.ldb, p.N, n0, kbeg, kend);

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int lr = lane & 31, lh = lane >> 5;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  la.load(0);
  lb.load(0);
  la.store(smem[0][0]);
  lb.store(smem[0][1]);
  __syncthreads();
  bf16x8 af[2][4], bfr[2][4];
  load_frags(smem[0][0], smem[0][1], 0, wm, wn, lr, lh, af[0], bfr[0]);

  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    // next tile (zeros past the end: harmless, the stage it lands in is not read)
    la.load(kt + 1);
    lb.load(kt + 1);
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch at the top of the step
    const bf16* As = smem[st][0];
    const bf16* Bs = smem[st][1];
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int cb = kk & 1;
      if (kk + 1 < BK / 16) load_frags(As, Bs, kk + 1, wm, wn, lr, lh, af[cb ^ 1], bfr[cb ^ 1]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[cb][j], af[cb][i], acc[i][j], 0, 0, 0);
      if (kk + 1 < BK / 16) {
        // interleave the next sub-step's 8 LDS reads among the 16 MFMAs
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
    }
    la.store(smem[st ^ 1][0]);
    lb.store(smem[st ^ 1][1]);
    __syncthreads();
    load_frags(smem[st ^ 1][0], smem[st ^ 1][1], 0, wm, wn, lr, lh, af[0], bfr[0]);
  }

  // Epilogue through LDS, in two passes of 128 rows (the 128 KiB of operand
  // stages hold a [128][256] fp32 half tile).  Pass q: the waves with wm == q
  // write their accumulators (lane: 4 consecutive n of row m, 16-byte chunk
  // XOR-swizzled by the row), then every wave writes whole rows to memory:
  // 64 lanes x 4 columns = one 256-column row per instruction.
  float* stage = (float*)&smem[0][0][0];
  const int ncols = min(BN, p.N - n0);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    if (wm == q) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = i * 32 + lr;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int c = (wn * 128 + j * 32 + 8 * g + 4 * lh) >> 2;  // 16-byte chunk (4 floats)
            *(f32x4*)(stage + r * 256 + ((c ^ (r & 15)) << 2)) =
                f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
          }
      }
    }
    __syncthreads();
    const int c = lane;            // this lane's 4-column chunk of the row
    const int n = n0 + c * 4;
    const bool cok = c * 4 < ncols;
    constexpr int RPW = 128 / (NTHR / 64);  // rows per wave per pass
    // residual / saved-u operand for all of this wave's rows, loaded up front
    bf16x4 rv[RPW];
    if (EPI == EPI_RESID || EPI == EPI_DRELU2) {
#pragma unroll
      for (int k = 0; k < RPW; ++k) {
        const int m = m0 + q * 128 + w + k * (NTHR / 64);
        rv[k] = (cok && m < p.M) ? *(const bf16x4*)((const bf16*)p.R + (size_t)m * p.ldr + n) : bf16x4{};
      }
    }
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
      const int r = w + k * (NTHR / 64);
      const int m = m0 + q * 128 + r;
      if (cok && m < p.M) {
        const f32x4 v4 = *(const f32x4*)(stage + r * 256 + ((c ^ (r & 15)) << 2));
        float v[4] = {v4[0], v4[1], v4[2], v4[3]};
        if (EPI == EPI_F32) {
          float* C = (float*)p.C;
          size_t off = (size_t)m * p.ldc + n;
          if (p.splits > 1) {
            C = p.partial + (size_t)blockIdx.y * p.M * p.N;
            off = (size_t)m * p.N + n;
          } else if (p.accumulate) {
            const f32x4 o = *(const f32x4*)(C + off);
            v[0] += o[0]; v[1] += o[1]; v[2] += o[2]; v[3] += o[3];
          }
          *(f32x4*)(C + off) = f32x4{v[0], v[1], v[2], v[3]};
        } else {
          bf16* C = (bf16*)p.C;
          const size_t off = (size_t)m * p.ldc + n;
          bf16x4 o;
          if (EPI == EPI_RESID) {
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = (bf16)(v[e] + (float)rv[k][e]);
          } else if (EPI == EPI_DRELU2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = (bf16)(v[e] * 2.0f * fmaxf((float)rv[k][e], 0.f));
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = (bf16)v[e];
          }
          *(bf16x4*)(C + off) = o;
          if (EPI == EPI_RELU2) {
            bf16x4 h;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float rl = fmaxf(v[e], 0.f);
              h[e] = (bf16)(rl * rl);
            }
            *(bf16x4*)((bf16*)p.C2 + off) = h;
          }
        }
      }
    }
    if (q == 0) __syncthreads();
  }
}

// ------------------------------------------------------------ fp32 SIMT
constexpr int FT = 64, FK = 16;

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_k(GemmArgs p) {
  __shared__ float As[FK][FT + 4], Bs[FK][FT + 4];
  const float* A = (const float*)p.A;
  const float* B = (const float*)p.B;
  const int m0 = blockIdx.x * FT, n0 = blockIdx.y * FT;
  const int ksplit = ((p.K + p.splits * FK - 1) / (p.splits * FK)) * FK;
  const int kbeg = blockIdx.z * ksplit, kend = min(p.K, kbeg + ksplit);
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int k0 = kbeg; k0 < kend; k0 += FK) {
    for (int e = threadIdx.x; e < FT * FK; e += 256) {
      int mm, kk;
      if (p.a_kmajor) { mm = e / FK; kk = e % FK; } else { kk = e / FT; mm = e % FT; }
      const int m = m0 + mm, k = k0 + kk;
      As[kk][mm] = (m < p.M && k < kend) ? (p.a_kmajor ? A[(size_t)m * p.lda + k] : A[(size_t)k * p.lda + m]) : 0.f;
      int nn, kb;
      if (p.b_kmajor) { nn = e / FK; kb = e % FK; } else { kb = e / FT; nn = e % FT; }
      const int n = n0 + nn, k2 = k0 + kb;
      Bs[kb][nn] = (n < p.N && k2 < kend) ? (p.b_kmajor ? B[(size_t)n * p.ldb + k2] : B[(size_t)k2 * p.ldb + n]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= p.N) continue;
      const float v = acc[i][j];
      if (EPI == EPI_F32) {
        if (p.splits > 1) p.partial[(size_t)blockIdx.z * p.M * p.N + (size_t)m * p.N + n] = v;
        else {
          float* C = (float*)p.C + (size_t)m * p.ldc + n;
          *C = p.accumulate ? *C + v : v;
        }
      } else {
        float* C = (float*)p.C + (size_t)m * p.ldc + n;
        if (EPI == EPI_RESID) *C = ((const float*)p.R)[(size_t)m * p.ldr + n] + v;
        else if (EPI == EPI_DRELU2) *C = v * 2.0f * fmaxf(((const float*)p.R)[(size_t)m * p.ldr + n], 0.f);
        else *C = v;
        if (EPI == EPI_RELU2) {
          const float r = fmaxf(v, 0.f);
          ((float*)p.C2)[(size_t)m * p.ldc + n] = r * r;
        }
      }
    }
  }
}

template <bool AK, bool BKM>
hipError_t launch_bf16(const GemmArgs& a, dim3 g, hipStream_t s) {
  switch (a.epi) {
    case EPI_STORE: hipLaunchKernelGGL((gemm_bf16_k<AK, BKM, EPI_STORE>), g, dim3(NTHR), 0, s, a); break;
    case EPI_RESID: hipLaunchKernelGGL((gemm_bf16_k<AK, BKM, EPI_RESID>), g, dim3(NTHR), 0, s, a); break;
    case EPI_RELU2: hipLaunchKernelGGL((gemm_bf16_k<AK, BKM, EPI_RELU2>), g, dim3(NTHR), 0, s, a); break;
    case EPI_DRELU2: hipLaunchKernelGGL((gemm_bf16_k<AK, BKM, EPI_DRELU2>), g, dim3(NTHR), 0, s, a); break;
    case EPI_F32: hipLaunchKernelGGL((gemm_bf16_k<AK, BKM, EPI_F32>), g, dim3(NTHR), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int gemm_splits(int dt, int M, int N, int K, int epi) {
  if (epi != EPI_F32) return 1;
  const int tile = dt == BF16 ? BM : FT;
  const int tiles = ((M + tile - 1) / tile) * ((N + tile - 1) / tile);
  const int kstep = dt == BF16 ? BK : FK;
  int s = 1;
  // aim for >= 2 workgroups per CU on the 256-CU chip, keep >= 8 K steps per split
  while (tiles * s < 512 && (K / (kstep * (s * 2))) >= 8 && s < 32) s *= 2;
  return s;
}

hipError_t gemm(int dt, const GemmArgs& a, hipStream_t s) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  if (dt == BF16) {
    const int nbm = (a.M + BM - 1) / BM, nbn = (a.N + BN - 1) / BN;
    dim3 g(nbm * nbn, a.splits);
    if (a.a_kmajor && a.b_kmajor) return launch_bf16<true, true>(a, g, s);
    if (a.a_kmajor && !a.b_kmajor) return launch_bf16<true, false>(a, g, s);
    if (!a.a_kmajor && !a.b_kmajor) return launch_bf16<false, false>(a, g, s);
    return launch_bf16<false, true>(a, g, s);
  }
  dim3 g((a.M + FT - 1) / FT, (a.N + FT - 1) / FT, a.splits);
  switch (a.epi) {
    case EPI_STORE: hipLaunchKernelGGL(gemm_f32_k<EPI_STORE>, g, dim3(256), 0, s, a); break;
    case EPI_RESID: hipLaunchKernelGGL(gemm_f32_k<EPI_RESID>, g, dim3(256), 0, s, a); break;
    case EPI_RELU2: hipLaunchKernelGGL(gemm_f32_k<EPI_RELU2>, g, dim3(256), 0, s, a); break;
    case EPI_DRELU2: hipLaunchKernelGGL(gemm_f32_k<EPI_DRELU2>, g, dim3(256), 0, s, a); break;
    case EPI_F32: hipLaunchKernelGGL(gemm_f32_k<EPI_F32>, g, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gdb
