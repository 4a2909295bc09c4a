// GEMMs of the block, the lm_head and the optimizer's Newton-Schulz steps:
// C[m, n] = sum_k A(m, k) * B(n, k) with either operand stored K-contiguous or
// M/N-contiguous, fused epilogues (residual add, ReLU² with its saved
// pre-activation, ReLU² backward, fp32 output with split-K, alpha*acc + beta*R).
//
// bf16 path (gfx950 MFMA, v_mfma_f32_32x32x16_bf16):
//   * 256x256 output tile per workgroup, K step 64, 512 threads = 8 waves in a
//     2x4 grid, each wave a 128x64 sub-tile = 4x2 MFMA blocks of 32x32, two
//     waves per SIMD;
//   * both operands are staged in LDS K-contiguous ([row][64 k], 128 B rows)
//     with the 16-byte chunk index XOR-swizzled by (row ^ row>>3) & 7, so the
//     fragment reads (32 consecutive rows, one chunk) and the stores of both
//     loaders are bank-conflict free;
//   * an operand stored M- (or N-) contiguous is read as 8x8 blocks (16-byte
//     loads along m at consecutive k; with 8 waves each thread loads four of
//     them and stores half chunks) and transposed in registers before the LDS
//     store, so every global access is a coalesced 16-byte load and the MFMA
//     loop never sees the layout;
//   * two LDS stages, one barrier per K step: while the MFMAs run on one stage
//     the next K tile is copied into the other — a K-contiguous operand
//     straight from memory into LDS (buffer_load ... lds), the other through
//     registers;
//   * the MFMA is issued with the B fragment as its first operand, so each lane
//     ends up holding 4 consecutive n of one output row m (8-byte bf16 or
//     16-byte fp32 stores);
//   * tile ids are remapped so that each XCD (blocks are dealt round-robin to
//     the 8 XCDs) works on a contiguous, grouped range of tiles (groups of 4
//     tile rows) and reuses A rows / B columns in its own L2.
// fp8 path (v_mfma_f32_32x32x64_f8f6f4 on OCP e4m3 codes, both operands
// K-contiguous): the same tiles, LDS layout and loaders with a K step of 128
// codes (the same 128-byte LDS rows); each lane's fragment is 32 bytes (two
// swizzled chunks) and the per-tensor scales amax/448 of both operands
// multiply the fp32 accumulators in the epilogue.
// fp32 path: plain LDS-tiled FMA GEMM (64x64 tile, 4x4 per thread).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace gdb {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;
// waves per workgroup of the bf16 GEMM with both operands K-contiguous
// (the other layouts and the fp8 GEMM use 8 too)
#ifndef GEMM_NW
#define GEMM_NW 8
#endif
// both operands M/N-contiguous (the weight gradients): copied straight into
// LDS as [k][m] and read with the LDS transpose load (1), or loaded into
// registers and stored transposed (0)
#ifndef GEMM_TRD
#define GEMM_TRD 1
#endif
// both operands K-contiguous, splits of a multiple of 128 k: fed by a ring of
// four 32-k LDS stages with precomputed addresses (1), or by the two 64-k
// stages of the main kernel (0).  The ring removes every VALU instruction from
// the main loop but was 1-3% slower on the d24 shapes with 8 waves and 3-7%
// with 4 (one barrier per 32 k, 64-byte copy segments), so it is off.
#ifndef GEMM_RING
#define GEMM_RING 0
#endif
#ifndef RING_NW
#define RING_NW 8
#endif
constexpr int TILE_ELEMS = BM * BK;  // bf16 elements of one operand tile (128-byte rows)
constexpr int BK8 = 128;             // fp8 codes per K step (the same 128-byte rows)

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

// Global -> registers: 8 vectors of 16 bytes per thread and operand, then
// registers -> LDS (K-contiguous, swizzled).  ES is the element size (2: bf16,
// 1: fp8 codes; fp8 operands are always K-major).  The resource is rebased at
// the tile's first row (K-major) or at (kbeg, first row) (M-major), so offsets
// stay far below 4 GiB; rows past the operand's end and k past the split's
// end read as zero.
// HALF (M-contiguous only): 512 threads share the operand, each loads 4 of
// the 8 k rows of its 8x8 block and stores 8-byte half chunks (the 8-wave
// workgroup with both operands M-contiguous).
template <bool KMAJ, int ES = 2, bool HALF = false>
struct Loader {
  static_assert(ES == 2 || KMAJ, "fp8 operands are K-major");
  static_assert(!HALF || !KMAJ, "HALF: M-contiguous operands");
  static constexpr int VEC = 16 / ES;   // elements per 16-byte vector
  static constexpr int BKE = 128 / ES;  // elements per K step
  static constexpr int NV = HALF ? 4 : 8;  // vectors per thread and K step
  bf16x8 r[NV];       // 16-byte containers
  __amdgpu_buffer_rsrc_t rs;
  int tid;            // this thread's index among the 256 that load the operand
  // M-major: this thread's 8x8 block, m chunk mc (m = 8mc..8mc+7) and k group
  // kb (k = NV*kb ..).  HALF: in wave w, lane 16g + u takes mc = 8g + u%8 and
  // kb = 2w + u/8, so each 16 lanes of a transposed store write 16 different
  // 8-byte bank slots (row, chunk and half); the plain t%32, t/32 split wrote
  // only 8 and took twice the LDS cycles per store
  __device__ __forceinline__ void block_of(int t, int& mc, int& kb) const {
    if constexpr (HALF) {
      const int w = t >> 6, l = t & 63, g = l >> 4, u = l & 15;
      mc = (u & 7) + 8 * g;
      kb = 2 * w + (u >> 3);
    } else {
      mc = t & 31;
      kb = t >> 5;
    }
  }
  unsigned off0;      // byte offset of this thread's first vector at k step 0
  unsigned step;      // bytes to advance per K step
  unsigned rowstep;   // bytes between the thread's consecutive vectors
  int kcol, kend_rel; // K-major: this thread's k within a step; split end (relative)
  __device__ __forceinline__ void init(const void* P, int ld, int rows, int r0, int kbeg, int kend,
                                       int tid_ = -1) {
    tid = tid_ < 0 ? (int)threadIdx.x : tid_;
    const int t = tid;
    if (KMAJ) {
      const int c = t & 7, rr = t >> 3;
      const char* base = (const char*)P + ((size_t)r0 * ld + kbeg) * ES;
      const size_t bytes = rows > r0 ? ((size_t)(rows - r0) * ld - kbeg) * ES : 0;
      rs = make_rsrc(base, bytes);
      off0 = (unsigned)((rr * ld + c * VEC) * ES);
      step = 128;
      rowstep = (unsigned)(32 * ld * ES);
      kcol = c * VEC;
      kend_rel = kend - kbeg;
    } else {
      int mc, kb;
      block_of(t, mc, kb);
      const bf16* base = (const bf16*)P + (size_t)kbeg * ld + r0;
      const size_t bytes = (size_t)(kend - kbeg) * ld * 2;
      rs = make_rsrc(base, bytes);
      const bool mvalid = r0 + mc * 8 < rows;
      off0 = mvalid ? (unsigned)(((kb * NV) * ld + mc * 8) * 2) : OOB;
      step = (unsigned)(BK * ld * 2);
      rowstep = (unsigned)(ld * 2);
      kcol = 0;
      kend_rel = kend - kbeg;
    }
  }
  // vector i (0..7) of K step kt.  Invalid vectors get an offset >=
  // 0xFFFFFFF0 (past any resource size): an OR with an all-ones mask, so the
  // compiler cannot turn it into a branch
  __device__ __forceinline__ void load1(int kt, int i) {
    unsigned bad;
    if (KMAJ) bad = 0u - (unsigned)(kt * BKE + kcol >= kend_rel);
    else bad = 0u - (unsigned)(off0 == OOB);
    const unsigned o = (off0 + kt * step) | (bad & OOB);
    r[i] = bload(rs, (o + i * rowstep) | (bad & OOB));
  }
  __device__ __forceinline__ void load(int kt) {
#pragma unroll
    for (int i = 0; i < NV; ++i) load1(kt, i);
  }
  __device__ __forceinline__ void store(bf16* __restrict__ S) {
    const int t = tid;
    if constexpr (KMAJ) {
      const int c = t & 7, rr = t >> 3;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = rr + 32 * i;
        *(bf16x8*)(S + row * BK + ((c ^ swz(row)) * 8)) = r[i];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) store1(S, j);
    }
  }
  // M-major operand: the LDS row j of this thread's 8x8 block (column j of
  // the eight loaded vectors)
  __device__ __forceinline__ void store1(bf16* __restrict__ S, int j) {
    static_assert(!KMAJ, "K-major operands are stored whole");
    int mc, kb;
    block_of(tid, mc, kb);
    const int row = mc * 8 + j;
    if constexpr (HALF) {
      bf16x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = r[i][j];
      *(bf16x4*)(S + row * BK + (((kb >> 1) ^ swz(row)) * 8) + (kb & 1) * 4) = w;
    } else {
      bf16x8 w;
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = r[i][j];
      *(bf16x8*)(S + row * BK + ((kb ^ swz(row)) * 8)) = w;
    }
  }
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;
#define WAIT_VM0() asm volatile("s_waitcnt vmcnt(0)" ::: "memory")

// K-contiguous operand copied straight from memory into the swizzled LDS
// layout (no staging registers): in wave instruction q (rows 8q..8q+7) lane L
// writes LDS bytes 16L of that 1 KiB block, i.e. physical chunk L%8 of row
// 8q + L/8, so it fetches the logical chunk (L%8) ^ swz(row).
template <int ES = 2, int NW = 4>
struct DmaLoader {
  static constexpr int VEC = 16 / ES;   // elements per 16-byte chunk
  static constexpr int BKE = 128 / ES;  // elements per K step
  static constexpr int NI = 32 / NW;    // copies per wave (32 per operand and K step)
  __amdgpu_buffer_rsrc_t rs;
  unsigned off[NI];
  int kc[NI];
  int kend_rel;
  __device__ __forceinline__ void init(const void* P, int ld, int rows, int r0, int kbeg, int kend) {
    const int t = threadIdx.x, w = t >> 6, L = t & 63;
    const char* base = (const char*)P + ((size_t)r0 * ld + kbeg) * ES;
    const size_t bytes = rows > r0 ? ((size_t)(rows - r0) * ld - kbeg) * ES : 0;
    rs = make_rsrc(base, bytes);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = 8 * (i * NW + w) + (L >> 3);
      const int c = (L & 7) ^ swz(row);
      off[i] = (unsigned)((row * ld + c * VEC) * ES);
      kc[i] = c * VEC;
    }
    kend_rel = kend - kbeg;
  }
  // copy i (0..NI-1) of K step kt into stage S
  __device__ __forceinline__ void load1(int kt, bf16* S, int i) {
    // wave-uniform, so the LDS destination (M0) is computed on the scalar unit
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const unsigned bad = 0u - (unsigned)(kt * BKE + kc[i] >= kend_rel);
    const unsigned o = (off[i] + kt * 128) | (bad & OOB);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(S + (i * NW + w) * 8 * BK), 16, o, 0, 0, 0);
  }
  __device__ __forceinline__ void load(int kt, bf16* S) {
#pragma unroll
    for (int i = 0; i < NI; ++i) load1(kt, S, i);
  }
};

// M-contiguous operand copied straight from memory into LDS as [64 k][256 m]
// (512-byte rows), the 16-byte chunk index XOR-swizzled by 4(k & 7): in wave
// instruction q (k rows 2q, 2q + 1) lane L writes the 16 bytes at 16L, i.e.
// physical chunk L%32 of row 2q + L/32, so it fetches logical chunk
// (L%32) ^ 4(row & 7), m = 8 * chunk .. + 7.  The resource is rebased at
// (kbeg, first m) and ends at the split's last k row, so k rows past the
// split read as zero; chunks past the operand's m extent get an offset past
// any resource size (zero too).
template <int NW>
struct TrDma {
  static constexpr int NI = 32 / NW;  // copies per wave (32 per operand and K step)
  __amdgpu_buffer_rsrc_t rs;
  unsigned off[NI], bad[NI];
  unsigned step;  // bytes per K step (64 k rows)
  __device__ __forceinline__ void init(const void* P, int ld, int rows, int r0, int kbeg, int kend) {
    const int t = threadIdx.x, w = t >> 6, L = t & 63;
    const bf16* base = (const bf16*)P + (size_t)kbeg * ld + r0;
    rs = make_rsrc(base, (size_t)(kend - kbeg) * ld * 2);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = 2 * (i * NW + w) + (L >> 5);
      const int lc = (L & 31) ^ ((row & 7) << 2);
      const bool ok = r0 + 8 * lc < rows;
      off[i] = (unsigned)((row * ld + 8 * lc) * 2);
      bad[i] = ok ? 0u : OOB;
    }
    step = (unsigned)(BK * ld * 2);
  }
  // Issued as an asm statement: the compiler then cannot see an LDS store
  // that might alias the transposed fragment reads that follow (the
  // intrinsic made it wait for every copy in flight before each of them);
  // the kernel waits for its copies itself before the barrier that publishes
  // a stage.  No register is written; M0 carries the LDS destination.
  __device__ __forceinline__ void load1(int kt, bf16* S, int i) {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const unsigned d = (unsigned)(size_t)(lds_ptr_t)(S + (i * NW + w) * 512);
    const unsigned o = (off[i] + kt * step) | bad[i];
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(d), "v"(o), "s"(rs)
                 : "memory", "m0");
  }
};

// Both operands K-contiguous, 4 waves of 128x128: a ring of four LDS stages
// of 32 k per operand (64-byte rows, 16 KiB per 256-row tile; A stages in the
// first 64 KiB, B stages in the second), so copies run three steps ahead of
// the MFMAs.  Copy q (0..15) of a step fills rows 16q..16q+15 of a stage:
// lane L writes physical chunk L%4 of row 16q + L/4, so it fetches logical
// chunk (L%4) ^ ring_swz(row).  ring_swz takes a different value on each row
// of every aligned group of 4 rows with equal (row & 1) among 8, and of every
// aligned group of 4 rows with equal (row & 3) among 16, so the 8 or 16 lanes
// the LDS serves together in a 16-byte fragment read (32 consecutive rows,
// one chunk) hit distinct banks.  The resource is rebased on the scalar unit
// at every step (base + 64 bytes per step); steps past the end get an empty
// resource (their copies write zeros into a stage nobody reads).
__device__ __forceinline__ int ring_swz(int row) { return (((row >> 1) ^ (row >> 3)) & 1) | ((row >> 1) & 2); }

template <int NW>
struct RingDma {
  static constexpr int NI = 16 / NW;  // copies per wave (16 per operand and step)
  const char* base;
  unsigned bytes;
  unsigned off[NI];
  __device__ __forceinline__ void init(const void* P, int ld, int rows, int r0, int kbeg, int w, int L) {
    base = (const char*)P + ((size_t)r0 * ld + kbeg) * 2;
    const size_t b = rows > r0 ? ((size_t)(rows - r0) * ld - kbeg) * 2 : 0;
    bytes = b > 0xFFFFFF00ull ? 0xFFFFFF00u : (unsigned)b;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = 16 * (i * NW + w) + (L >> 2);
      const int lc = (L & 3) ^ ring_swz(row);
      off[i] = r0 + row < rows ? (unsigned)(row * ld * 2 + lc * 16) : OOB;
    }
  }
  // copy i (0..NI-1) of this wave for K step kt into the LDS bytes at d (the
  // wave's 1 KiB block of the stage); an asm statement, as for TrDma
  __device__ __forceinline__ void load1(int kt, int nk, unsigned d, int i) const {
    const unsigned adv = (unsigned)kt * 64u;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(base + adv), (short)0, kt < nk ? (int)(bytes - adv) : 0, 0x00020000);
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(d), "v"(off[i]), "s"(rs)
                 : "memory", "m0");
  }
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 tr_read(const bf16* p) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p));
}

#ifndef GEMM_XCD_SPLIT
#define GEMM_XCD_SPLIT 1
#endif
// Split-K launches (the weight gradients): the dispatcher hands workgroups to
// the 8 XCDs in turn, so with the tiles of one split numbered consecutively
// an XCD's concurrent workgroups would hold two or more splits' K ranges of
// scattered tiles.  xcd_rank gives workgroup i of a phase of n (the first at
// linear index base) its rank in an order where each XCD takes one contiguous
// run; the run is then read split-major and, within a split, in groups of 4
// tile rows (tile_order), so an XCD's workgroups share one K range and
// neighbouring operand panels in its L2.  Both are bijections.
__device__ __forceinline__ int xcd_rank(int i, int n, int base) {
  const int x = (base + i) & 7;
  int start = 0;
  for (int y = 0; y < x; ++y) {
    const int off = (y - base) & 7;  // the phase's first workgroup on XCD y
    start += off < n ? (n - off + 7) / 8 : 0;
  }
  return start + (i - ((x - base) & 7)) / 8;
}
__device__ __forceinline__ void tile_order(int idx, int nbm, int nbn, int& tm, int& tn) {
  constexpr int GROUP = 4;
  const int per_group = GROUP * nbn;
  const int g = idx / per_group;
  const int first_m = g * GROUP;
  const int gsize = min(nbm - first_m, GROUP);
  const int in = idx % per_group;
  tm = first_m + in % gsize;
  tn = in / gsize;
}

__device__ __forceinline__ void tile_coords(int bid, int nbm, int nbn, int& tm, int& tn) {
  const int total = nbm * nbn;
  const int full = (total / 8) * 8;
  int logical = bid;
  if (bid < full) logical = (bid % 8) * (full / 8) + bid / 8;
  // groups of 4 tile rows: an XCD's 32 concurrent tiles cover 4 A panels and
  // 8 B panels (2% faster on the d24 K-contiguous products than 8 x 4; 16 x 2
  // and 32 x 1 were 4-7% slower)
  constexpr int GROUP = 4;
  const int per_group = GROUP * nbn;
  const int g = logical / per_group;
  const int first_m = g * GROUP;
  const int gsize = min(nbm - first_m, GROUP);
  const int in = logical % per_group;
  tm = first_m + in % gsize;
  tn = in / gsize;
}

// MFMA fragments of one 16-wide k sub-step: 4 row blocks of A, JB of B (the
// wave's 128 x 32JB output block).
template <int JB = 4>
__device__ __forceinline__ void load_frags(const bf16* As, const bf16* Bs, int kk, int wm, int wn, int lr,
                                           int lh, bf16x8* af, bf16x8* bfr) {
  const int ch = kk * 2 + lh;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = wm * 128 + i * 32 + lr;
    af[i] = *(const bf16x8*)(As + row * BK + ((ch ^ swz(row)) * 8));
  }
#pragma unroll
  for (int j = 0; j < JB; ++j) {
    const int row = wn * 32 * JB + j * 32 + lr;
    bfr[j] = *(const bf16x8*)(Bs + row * BK + ((ch ^ swz(row)) * 8));
  }
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// fp8 fragments of one 64-code k sub-step (kk = 0, 1): lane half lh holds
// codes 32*lh .. 32*lh+31 of its row, i.e. the two chunks 4kk+2lh, 4kk+2lh+1.
__device__ __forceinline__ i32x8 frag8(const bf16* S, int row, int ch) {
  const u32x4 lo = *(const u32x4*)(S + row * BK + ((ch ^ swz(row)) * 8));
  const u32x4 hi = *(const u32x4*)(S + row * BK + (((ch + 1) ^ swz(row)) * 8));
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}
template <int JB = 4>
__device__ __forceinline__ void load_frags8(const bf16* As, const bf16* Bs, int kk, int wm, int wn, int lr,
                                            int lh, i32x8* af, i32x8* bfr) {
  const int ch = kk * 4 + lh * 2;
#pragma unroll
  for (int i = 0; i < 4; ++i) af[i] = frag8(As, wm * 128 + i * 32 + lr, ch);
#pragma unroll
  for (int j = 0; j < JB; ++j) bfr[j] = frag8(Bs, wn * 32 * JB + j * 32 + lr, ch);
}

template <typename T> struct V4;
template <> struct V4<bf16> { typedef bf16x4 t; };
template <> struct V4<float> { typedef f32x4 t; };

// OT: element type of C, C2 and R in the epilogues other than EPI_F32 (bf16;
// float for the fp8 products of an fp32 model)
// NW: waves per workgroup.  4: a 2x2 grid of 128x128 wave tiles (one wave
// per SIMD); 8: a 2x4 grid of 128x64 wave tiles, two waves per SIMD, so one
// wave's MFMAs run while the other waits on its copies or LDS reads.
template <bool AK, bool BK_, int EPI, bool F8 = false, typename OT = bf16, int NW = 4, bool RING = false>
__global__ __launch_bounds__(64 * NW, 1) void gemm_bf16_k(GemmArgs p) {
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  constexpr int NTH = 64 * NW;
  constexpr int WNN = NW / 2;         // waves along N
  constexpr int JB = BN / WNN / 32;   // 32-column blocks per wave (4 or 2)
  typedef typename V4<OT>::t OV;
  constexpr int ES = F8 ? 1 : 2;
  constexpr int KSTEP = F8 ? BK8 : BK;  // elements per K step
  __shared__ __attribute__((aligned(16))) bf16 smem[2][2][TILE_ELEMS];  // [stage][A|B]
  const int nbm = (p.M + BM - 1) / BM, nbn = (p.N + BN - 1) / BN;
  // tile and K range: one phase (blockIdx.x the tile, blockIdx.y the split)
  // or two (blockIdx.x runs over the first phase's pieces, split-major, then
  // the second's; each phase is a band of whole tile rows or columns)
  int tm, tn, split = blockIdx.y, nsplit = p.splits;
  if (p.splits2 > 0) {
    const int bid = blockIdx.x;
    const int r1 = p.split_cols ? nbm : p.first1, c1 = p.split_cols ? p.first1 : nbn;
    const int t1 = r1 * c1, n1 = t1 * p.splits;
    if (bid < n1) {
      if (GEMM_XCD_SPLIT) {
        const int g = xcd_rank(bid, n1, 0);
        split = g / t1;
        tile_order(g - split * t1, r1, c1, tm, tn);
      } else {
        split = bid / t1;
        tile_coords(bid - split * t1, r1, c1, tm, tn);
      }
    } else {
      const int r2 = p.split_cols ? nbm : nbm - p.first1, c2 = p.split_cols ? nbn - p.first1 : nbn;
      const int t2 = r2 * c2, b2 = bid - n1;
      if (GEMM_XCD_SPLIT) {
        const int g = xcd_rank(b2, t2 * p.splits2, n1);
        split = g / t2;
        tile_order(g - split * t2, r2, c2, tm, tn);
      } else {
        split = b2 / t2;
        tile_coords(b2 - split * t2, r2, c2, tm, tn);
      }
      if (p.split_cols) tn += p.first1;
      else tm += p.first1;
      nsplit = p.splits2;
    }
  } else if (GEMM_XCD_SPLIT && gridDim.y > 1) {
    const int nt = gridDim.x, n = nt * gridDim.y;
    const int g = xcd_rank(blockIdx.y * nt + blockIdx.x, n, (int)blockIdx.z * n);
    split = g / nt;
    tile_order(g - split * nt, nbm, nbn, tm, tn);
  } else {
    tile_coords(blockIdx.x, nbm, nbn, tm, tn);
  }
  const int m0 = tm * BM, n0 = tn * BN;
  if (blockIdx.z) {  // item of a batched launch
    const size_t z = blockIdx.z;
    p.A = (const char*)p.A + z * p.bsA * ES;
    p.B = (const char*)p.B + z * p.bsB * ES;
    p.C = (char*)p.C + z * p.bsC * (EPI == EPI_F32 ? sizeof(float) : sizeof(OT));
    if (p.R) p.R = (const char*)p.R + z * p.bsR * sizeof(OT);
  }
  // split-K range
  const int ksplit = ((p.K + nsplit * KSTEP - 1) / (nsplit * KSTEP)) * KSTEP;
  const int kbeg = min(p.K, split * ksplit);
  const int kend = min(p.K, kbeg + ksplit);
  const int nk = (kend - kbeg + KSTEP - 1) / KSTEP;

  // register loaders of M/N-contiguous operands: every thread takes part in
  // both; with 8 waves each thread loads half of its 8x8 block (HALF)
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  constexpr bool HALF = NW == 8;
  Loader<AK, ES, HALF && !AK> la;
  Loader<BK_, ES, HALF && !BK_> lb;
  la.init(p.A, p.lda, p.M, m0, kbeg, kend, HALF ? t : t & 255);
  lb.init(p.B, p.ldb, p.N, n0, kbeg, kend, HALF ? t : t & 255);

  const int wm = w / WNN, wn = w % WNN;
  const int lr = lane & 31, lh = lane >> 5;

  f32x16 acc[4][JB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < JB; ++j) acc[i][j] = f32x16{};

  if constexpr (F8) {
    // fp8 operands are K-contiguous: both copied straight into LDS
    constexpr int NDF = 32 / NW;        // copies per operand and wave
    constexpr int NM = 4 * JB;          // MFMAs per sub-step
    constexpr int CH = (4 + JB) * 2;    // 16-byte chunk reads of the next sub-step
    DmaLoader<1, NW> da, db;
    da.init(p.A, p.lda, p.M, m0, kbeg, kend);
    db.init(p.B, p.ldb, p.N, n0, kbeg, kend);
    da.load(0, smem[0][0]);
    db.load(0, smem[0][1]);
    WAIT_VM0();
    __syncthreads();
    i32x8 af[2][4], bfr[2][JB];
    load_frags8<JB>(smem[0][0], smem[0][1], 0, wm, wn, lr, lh, af[0], bfr[0]);
    for (int kt = 0; kt < nk; ++kt) {
      const int st = kt & 1;
      const bf16* As = smem[st][0];
      const bf16* Bs = smem[st][1];
      // first sub-step: the MFMAs interleaved with the next step's copies
      // and the second sub-step's chunk reads (fixed order)
#pragma unroll
      for (int q = 0; q < NM; ++q) {
        const int i = q / JB, j = q % JB;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[0][j], af[0][i], acc[i][j], 0, 0, 0, 0, 0, 0);
#pragma unroll
        for (int u = q * 2 * NDF / NM; u < (q + 1) * 2 * NDF / NM; ++u) {
          if (u < NDF) da.load1(kt + 1, smem[st ^ 1][0], u);
          else db.load1(kt + 1, smem[st ^ 1][1], u - NDF);
        }
        // chunk h of fragment r (A blocks 0-3, then B blocks) of sub-step 1
#pragma unroll
        for (int v = q * CH / NM; v < (q + 1) * CH / NM; ++v) {
          const int r = v >> 1, h = v & 1, ch = 4 + lh * 2 + h;
          const bool isa = r < 4;
          const int row = isa ? wm * 128 + r * 32 + lr : wn * 32 * JB + (r - 4) * 32 + lr;
          const u32x4 x = *(const u32x4*)((isa ? As : Bs) + row * BK + ((ch ^ swz(row)) * 8));
          i32x8& dst = isa ? af[1][r & 3] : bfr[1][(r - 4) & (JB - 1)];
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[4 * h + e] = (int)x[e];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < JB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[1][j], af[1][i], acc[i][j], 0, 0, 0, 0, 0, 0);
      WAIT_VM0();
      __syncthreads();
      load_frags8<JB>(smem[st ^ 1][0], smem[st ^ 1][1], 0, wm, wn, lr, lh, af[0], bfr[0]);
    }
  } else if constexpr (RING) {
    // Ring of four 32-k stages (RingDma).  Step kt (stage kt % 4): sub-step
    // 0's MFMAs run on fragments read during the previous step, interleaved
    // with the reads of sub-step 1's fragments and half of this wave's copies
    // of step kt + 3 (into the stage every wave finished reading before the
    // last barrier); then each wave waits for its copies of step kt + 1 (those
    // of steps kt + 2 and kt + 3 may stay in flight) and for its LDS reads,
    // one barrier, and sub-step 1's MFMAs run with the reads of step kt + 1's
    // first fragments and the other half of the copies.  The host sends only
    // splits of a multiple of 128 k here, so the loop runs whole groups of 4
    // steps.
    static_assert(AK && BK_ && !F8, "the ring serves bf16 operands that are both K-contiguous");
    constexpr int NM = 4 * JB;        // MFMAs per sub-step
    constexpr int NR = 4 + JB;        // fragment reads per sub-step
    constexpr int CPO = 16 / NW;      // copies per wave, operand and step
    constexpr int CH = CPO;           // copies per sub-step (A in sub-step 0, B in 1)
    const int nks = (kend - kbeg) / 32;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    RingDma<NW> ra, rb;
    ra.init(p.A, p.lda, p.M, m0, kbeg, w, lane);
    rb.init(p.B, p.ldb, p.N, n0, kbeg, w, lane);
    const unsigned lds0 = (unsigned)(size_t)(lds_ptr_t)&smem[0][0][0];
    const char* Lb = (const char*)&smem[0][0][0];
    // fragment lane offsets (bytes): row wm*128 + lr of A / row wn*32*JB + lr
    // of B (B stages start at 64 KiB), chunk (2kk + lh) ^ ring_swz(lr) = g ^ 2kk
    const int g = lh ^ ring_swz(lr);
    const int ao0 = (wm * 128 + lr) * 64 + 16 * g, ao1 = (wm * 128 + lr) * 64 + 16 * (g ^ 2);
    const int bo0 = 65536 + (wn * 32 * JB + lr) * 64 + 16 * g;
    const int bo1 = 65536 + (wn * 32 * JB + lr) * 64 + 16 * (g ^ 2);
    auto copy = [&](int kt, int stg, int c) {  // c < CPO: A copy c, else B copy c - CPO
      const int i = c % CPO;
      const unsigned blk = (unsigned)(stg * 16384 + (i * NW + wu) * 1024);
      if (c < CPO) ra.load1(kt, nks, lds0 + blk, i);
      else rb.load1(kt, nks, lds0 + 65536u + blk, i);
    };
    auto fa = [&](int stg, int kk, int i) {
      return *(const bf16x8*)(Lb + (kk ? ao1 : ao0) + stg * 16384 + i * 2048);
    };
    auto fb = [&](int stg, int kk, int j) {
      return *(const bf16x8*)(Lb + (kk ? bo1 : bo0) + stg * 16384 + j * 2048);
    };
    // fragment read r of a sub-step, in the MFMAs' order of first use: A0, B0..B(JB-1), A1..A3
    auto rd = [&](bf16x8* a, bf16x8* b, int stg, int kk, int r) {
      if (r == 0) a[0] = fa(stg, kk, 0);
      else if (r <= JB) b[r - 1] = fb(stg, kk, r - 1);
      else a[r - JB] = fa(stg, kk, r - JB);
    };
#pragma unroll
    for (int kt = 0; kt < 3; ++kt)
#pragma unroll
      for (int c = 0; c < 2 * CPO; ++c) copy(kt, kt, c);
    if constexpr (NW == 4) asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(8)\n\ts_barrier" ::: "memory");
    bf16x8 a0[4], b0[JB], a1[4], b1[JB];
#pragma unroll
    for (int r = 0; r < NR; ++r) rd(a0, b0, 0, 0, r);
    for (int kt0 = 0; kt0 < nks; kt0 += 4) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kt = kt0 + u;
        const int sn = (u + 1) & 3, sc = (u + 3) & 3;
#pragma unroll
        for (int q = 0; q < NM; ++q) {
          const int i = q / JB, j = q % JB;
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0[j], a0[i], acc[i][j], 0, 0, 0);
#pragma unroll
          for (int h = 0; h < CH; ++h)
            if (q == h * NM / CH) copy(kt + 3, sc, h);
#pragma unroll
          for (int r = 0; r < NR; ++r)
            if (q == r * NM / NR) rd(a1, b1, u, 1, r);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (NW == 4) asm volatile("s_waitcnt vmcnt(12) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int q = 0; q < NM; ++q) {
          const int i = q / JB, j = q % JB;
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1[j], a1[i], acc[i][j], 0, 0, 0);
#pragma unroll
          for (int h = 0; h < CH; ++h)
            if (q == h * NM / CH) copy(kt + 3, sc, CH + h);
#pragma unroll
          for (int r = 0; r < NR; ++r)
            if (q == r * NM / NR) rd(a0, b0, sn, 0, r);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // the copies past the end still write zeros into the ring, which the
    // epilogue reuses for staging
    WAIT_VM0();
    __syncthreads();
  } else if constexpr (!AK && !BK_ && GEMM_TRD) {
    // both operands M/N-contiguous: copied straight into LDS as [k][m] rows
    // and read as MFMA fragments with the LDS transpose load.  A lane's
    // fragment then holds k = 16kk + 4lh + e%4 + 8(e/4) (e = 0..7) of its row,
    // the same permutation of the contraction in both operands.  The
    // schedule is the one below without the transposed stores.
    TrDma<NW> da, db;
    da.init(p.A, p.lda, p.M, m0, kbeg, kend);
    db.init(p.B, p.ldb, p.N, n0, kbeg, kend);
    constexpr int ND = 32 / NW;
    constexpr int NQ = 2 * ND;
    auto issue1 = [&](int kt, int stg, int q) {
      if (q < ND) da.load1(kt, smem[stg][0], q);
      else db.load1(kt, smem[stg][1], q - ND);
    };
    // transposed-read lane constants: rows 16kk + rl (and + 8), 32-column
    // block c, its physical chunk group (c ^ (rl & 7)), chunk and half within
    const int G = lane >> 4, sl = lane & 15;
    const int rl = 4 * (G >> 1) + (sl >> 2);  // < 8, so rl & 7 = rl
    const int lane_off = rl * 256 + 8 * (2 * (G & 1) + ((sl & 3) >> 1)) + 4 * (sl & 1);
    auto frag = [&](const bf16* S, int c, int kk) {
      const bf16* q0 = S + kk * 16 * 256 + lane_off + 32 * (c ^ rl);
      const bf16x4 lo = tr_read(q0), hi = tr_read(q0 + 8 * 256);
      return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    auto load_tr = [&](const bf16* As, const bf16* Bs, int kk, bf16x8* af, bf16x8* bfr) {
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = frag(As, wm * 4 + i, kk);
#pragma unroll
      for (int j = 0; j < JB; ++j) bfr[j] = frag(Bs, wn * JB + j, kk);
    };
#pragma unroll
    for (int q = 0; q < NQ; ++q) issue1(0, 0, q);
    WAIT_VM0();
    __syncthreads();
    bf16x8 af[2][4], bfr[2][JB];
    load_tr(smem[0][0], smem[0][1], 0, af[0], bfr[0]);
    constexpr int NM = 4 * JB;  // MFMAs per sub-step
    for (int kt = 0; kt < nk; ++kt) {
      const int st = kt & 1;
      const bf16* As = smem[st][0];
      const bf16* Bs = smem[st][1];
      // sub-step 0: its MFMAs interleaved with the next step's copies and
      // the fragment reads of sub-step 1
#pragma unroll
      for (int q = 0; q < NM; ++q) {
        const int i = q / JB, j = q % JB;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[0][j], af[0][i], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int u = q * NQ / NM; u < (q + 1) * NQ / NM; ++u) issue1(kt + 1, st ^ 1, u);
        if (q < 4 + JB) {
          if (q < 4) af[1][q] = frag(As, wm * 4 + q, 1);
          else bfr[1][q - 4] = frag(Bs, wn * JB + q - 4, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int kk = 1; kk < BK / 16 - 1; ++kk) {
        const int cb = kk & 1;
        load_tr(As, Bs, kk + 1, af[cb ^ 1], bfr[cb ^ 1]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < JB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[cb][j], af[cb][i], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int q = 0; q < NM; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2 * (4 + JB) / NM, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < JB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[1][j], af[1][i], acc[i][j], 0, 0, 0);
      WAIT_VM0();
      __syncthreads();
      load_tr(smem[st ^ 1][0], smem[st ^ 1][1], 0, af[0], bfr[0]);
    }
  } else {
    // bf16: a K-contiguous operand is copied straight into LDS (DMA); an
    // M/N-contiguous one is loaded into registers and stored transposed.
    // Per K step: the first 16-wide sub-step's MFMAs are interleaved one to
    // one with the 16 copies (or register loads) of the next step and two to
    // one with the second sub-step's fragment reads; the last sub-step's
    // MFMAs with the transposed LDS stores of the next step.  The order is
    // pinned with scheduling barriers.
    DmaLoader<2, NW> da, db;
    if constexpr (AK) da.init(p.A, p.lda, p.M, m0, kbeg, kend);
    if constexpr (BK_) db.init(p.B, p.ldb, p.N, n0, kbeg, kend);
    // the wave's loads of one K step, in a fixed order: DMA copies of A
    // (32/NW), DMA copies of B (32/NW), register loads of A (8, or 4 with
    // 8 waves), register loads of B (likewise)
    constexpr int ND = 32 / NW;
    constexpr int NRG = HALF ? 4 : 8;  // register loads per operand
    constexpr int NQ = (AK ? ND : NRG) + (BK_ ? ND : NRG);  // at most per wave
    auto issue1 = [&](int kt, int stg, int q) {
      if (q < (AK ? ND : NRG)) {
        if constexpr (AK) da.load1(kt, smem[stg][0], q);
        else la.load1(kt, q);
      } else {
        const int q2 = q - (AK ? ND : NRG);
        if constexpr (BK_) db.load1(kt, smem[stg][1], q2);
        else lb.load1(kt, q2);
      }
    };
    auto store1 = [&](int stg, int q) {  // q < 16: A stores 0-7, B stores 8-15
      if (q < 8) {
        if constexpr (!AK) la.store1(smem[stg][0], q);
      } else {
        if constexpr (!BK_) lb.store1(smem[stg][1], q - 8);
      }
    };
#pragma unroll
    for (int q = 0; q < NQ; ++q) issue1(0, 0, q);
#pragma unroll
    for (int q = 0; q < 16; ++q) store1(0, q);
    WAIT_VM0();
    __syncthreads();
    bf16x8 af[2][4], bfr[2][JB];
    load_frags<JB>(smem[0][0], smem[0][1], 0, wm, wn, lr, lh, af[0], bfr[0]);
    constexpr int NM = 4 * JB;  // MFMAs per sub-step
    for (int kt = 0; kt < nk; ++kt) {
      const int st = kt & 1;
      const bf16* As = smem[st][0];
      const bf16* Bs = smem[st][1];
      // sub-step 0 (fragments in set 0): the NM MFMAs interleaved with the
      // next step's loads and the 4 + JB fragment reads of sub-step 1
#pragma unroll
      for (int q = 0; q < NM; ++q) {
        const int i = q / JB, j = q % JB;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[0][j], af[0][i], acc[i][j], 0, 0, 0);
        // loads: NQ of them over NM MFMAs (one or two per MFMA)
#pragma unroll
        for (int u = q * NQ / NM; u < (q + 1) * NQ / NM; ++u) issue1(kt + 1, st ^ 1, u);
        if (q < 4 + JB) {
          const int r = q, ch = 2 + lh;  // fragment r of sub-step 1: A blocks 0-3, then B blocks
          if (r < 4) {
            const int row = wm * 128 + r * 32 + lr;
            af[1][r] = *(const bf16x8*)(As + row * BK + ((ch ^ swz(row)) * 8));
          } else {
            const int row = wn * 32 * JB + (r - 4) * 32 + lr;
            bfr[1][r - 4] = *(const bf16x8*)(Bs + row * BK + ((ch ^ swz(row)) * 8));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // sub-steps 1 and 2
#pragma unroll
      for (int kk = 1; kk < BK / 16 - 1; ++kk) {
        const int cb = kk & 1;
        load_frags<JB>(As, Bs, kk + 1, wm, wn, lr, lh, af[cb ^ 1], bfr[cb ^ 1]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < JB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[cb][j], af[cb][i], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int q = 0; q < 4 + JB; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, NM / (4 + JB) > 1 ? 2 : 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // sub-step 3 (set 1), with the transposed stores of the next step's
      // register-loaded operands (their stage was last read in step kt-1)
#pragma unroll
      for (int q = 0; q < NM; ++q) {
        const int i = q / JB, j = q % JB;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[1][j], af[1][i], acc[i][j], 0, 0, 0);
#pragma unroll
        for (int u = q * 16 / NM; u < (q + 1) * 16 / NM; ++u) store1(st ^ 1, u);
        __builtin_amdgcn_sched_barrier(0);
      }
      WAIT_VM0();
      __syncthreads();
      load_frags<JB>(smem[st ^ 1][0], smem[st ^ 1][1], 0, wm, wn, lr, lh, af[0], bfr[0]);
    }
  }
  // fp8: both per-tensor scales (amax / 448, the quantiser's float32 values)
  float oscale = 1.0f;
  if constexpr (F8) oscale = (p.amax_a[0] / 448.0f) * (p.amax_b[0] / 448.0f);

  // The output stores are non-temporal: a product's output is written once and
// read by a later kernel, long after it would have left the caches (the
// lm_head logits 3.07 -> 2.89 ms, the ReLU^2-backward product 0.69 -> 0.65 ms).
// Epilogue through LDS, in two passes of 128 rows (the 128 KiB of operand
  // stages hold a [128][256] fp32 half tile).  Pass q: the waves with wm == q
  // write their accumulators (lane: 4 consecutive n of row m, 16-byte chunk
  // XOR-swizzled by the row), then every wave writes whole rows to memory:
  // 64 lanes x 4 columns = one 256-column row per instruction.
  float* stage = (float*)&smem[0][0][0];
  const int ncols = min(BN, p.N - n0);
  float am = 0.f;  // largest |value| this thread stores into the quantiser's input (amax_out)
  if constexpr ((EPI == EPI_STORE || EPI == EPI_SQR) && std::is_same<OT, bf16>::value) {
    // bf16 output with nothing to add: the values are finished in registers
    // and the whole 256x256 tile is staged once as bf16 (128 KiB).  A row is
    // 64 slots of 8 bytes (4 columns); slot s of row r sits at s ^ (r & 31),
    // so the 32 rows of a half-wave's write and the 64 slots of a row read
    // each hit distinct bank pairs.
    bf16* sb = &smem[0][0][0];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 128 + i * 32 + lr;
#pragma unroll
      for (int j = 0; j < JB; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float v = acc[i][j][4 * g + e];
            if constexpr (F8) v *= oscale;
            if constexpr (EPI == EPI_SQR) {
              const float rl = fmaxf(v, 0.f);
              v = rl * rl;
              am = fmaxf(am, v);
            }
            o[e] = (bf16)v;
          }
          const int slot = (wn * 32 * JB + j * 32 + 8 * g + 4 * lh) >> 2;
          *(bf16x4*)(sb + r * 256 + ((slot ^ (r & 31)) << 2)) = o;
        }
    }
    __syncthreads();
    // two rows per instruction, 16 bytes per lane: lane half h takes row
    // 2(k*NW + w) + h, lane l = lane % 32 its slots 2l and 2l + 1, which sit
    // in one aligned 16-byte pair at (2l) ^ x, x = row & 31 (swapped if x is odd)
    const int l32 = lane & 31;
    const bool cok = 8 * l32 < ncols;
#pragma unroll 8
    for (int k = 0; k < BM / NW / 2; ++k) {
      const int r = 2 * (k * NW + w) + (lane >> 5);
      const int m = m0 + r;
      const int x = r & 31;
      bf16x8 v = *(const bf16x8*)(sb + r * 256 + ((((2 * l32) ^ x) & ~1) << 2));
      if (x & 1) v = bf16x8{v[4], v[5], v[6], v[7], v[0], v[1], v[2], v[3]};
      if (cok && m < p.M) __builtin_nontemporal_store(v, (bf16x8*)((bf16*)p.C + (size_t)m * p.ldc + n0 + 8 * l32));
    }
  } else {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int c = lane;            // this lane's 4-column chunk of the row
    const int n = n0 + c * 4;
    const bool cok = c * 4 < ncols;
    constexpr int RPW = 128 / (NW);  // rows per wave per pass
    // residual / saved-u operand for all of this wave's rows of the pass,
    // loaded before the accumulators are staged so the loads overlap it
    OV rv[RPW];
    if (EPI == EPI_RESID || EPI == EPI_DRELU2 || EPI == EPI_DSQR || EPI == EPI_AXPBY) {
#pragma unroll
      for (int k = 0; k < RPW; ++k) {
        const int m = m0 + q * 128 + w + k * (NW);
        rv[k] = (cok && m < p.M) ? *(const OV*)((const OT*)p.R + (size_t)m * p.ldr + n) : OV{};
      }
    }
    if (wm == q) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = i * 32 + lr;
#pragma unroll
        for (int j = 0; j < JB; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int c = (wn * 32 * JB + j * 32 + 8 * g + 4 * lh) >> 2;  // 16-byte chunk (4 floats)
            *(f32x4*)(stage + r * 256 + ((c ^ (r & 15)) << 2)) =
                f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
          }
      }
    }
    __syncthreads();
    if constexpr (EPI == EPI_QKNORM) {
      // Each half-wave takes one row per iteration; 16 lanes per head, lane
      // hl owning columns 4hl..4hl+3 and their RoPE partners 64 + 4hl..: the
      // rotation needs no exchange and the sum of squares is a butterfly
      // over 16 lanes.  The RoPE table entries are fetched 4 rows ahead.
      const int half = lane >> 5, hd = (lane >> 4) & 1, hl = lane & 15;
      const int col = hd * 128 + 4 * hl;                 // tile column of the first value
      const int head = (n0 >> 7) + hd;
      const bool hok = hd * 128 < ncols;
      constexpr int NIT = RPW / 2, RPF = 4;
      f32x4 csr[RPF][2];
#pragma unroll
      for (int k = 0; k < RPF; ++k) {
        const int m = min(m0 + q * 128 + w + (2 * k + half) * (NW), p.M - 1);
        const float* rp = p.rope + ((size_t)(m % p.T) * 64 + 4 * hl) * 2;
        csr[k][0] = *(const f32x4*)rp;
        csr[k][1] = *(const f32x4*)(rp + 4);
      }
#pragma unroll
      for (int k = 0; k < NIT; ++k) {
        const int r = w + (2 * k + half) * (NW);
        const int m = m0 + q * 128 + r;
        const f32x4 cs0 = csr[k % RPF][0], cs1 = csr[k % RPF][1];
        if (k + RPF < NIT) {
          const int mn = min(m0 + q * 128 + w + (2 * (k + RPF) + half) * (NW), p.M - 1);
          const float* rp = p.rope + ((size_t)(mn % p.T) * 64 + 4 * hl) * 2;
          csr[k % RPF][0] = *(const f32x4*)rp;
          csr[k % RPF][1] = *(const f32x4*)(rp + 4);
        }
        const int ca = col >> 2, cb = (col + 64) >> 2;    // 16-byte chunks of the two halves
        const f32x4 a4 = *(const f32x4*)(stage + r * 256 + ((ca ^ (r & 15)) << 2));
        const f32x4 b4 = *(const f32x4*)(stage + r * 256 + ((cb ^ (r & 15)) << 2));
        float va[4] = {a4[0], a4[1], a4[2], a4[3]}, vb[4] = {b4[0], b4[1], b4[2], b4[3]};
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) ss += va[e] * va[e] + vb[e] * vb[e];
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
        if (m < p.M && hok) {
          if (head < p.qk_heads) {
            const float rr = rsqrtf(ss * (1.0f / 128.0f) + p.eps);
            const float cc[4] = {cs0[0], cs0[2], cs1[0], cs1[2]}, sn[4] = {cs0[1], cs0[3], cs1[1], cs1[3]};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float x = va[e], y = vb[e];
              va[e] = rr * (x * cc[e] - y * sn[e]);
              vb[e] = rr * (x * sn[e] + y * cc[e]);
            }
            if (hl == 0) p.rinv[(size_t)m * p.qk_heads + head] = rr;
          }
          bf16x4 oa, ob;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            oa[e] = (bf16)va[e];
            ob[e] = (bf16)vb[e];
          }
          bf16* crow = (bf16*)p.C + (size_t)m * p.ldc + n0 + col;
          *(bf16x4*)crow = oa;
          *(bf16x4*)(crow + 64) = ob;
        }
      }
    } else {
#pragma unroll
    for (int k = 0; k < RPW; ++k) {
      const int r = w + k * (NW);
      const int m = m0 + q * 128 + r;
      if (cok && m < p.M) {
        const f32x4 v4 = *(const f32x4*)(stage + r * 256 + ((c ^ (r & 15)) << 2));
        float v[4] = {v4[0], v4[1], v4[2], v4[3]};
        if constexpr (F8) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] *= oscale;
        }
        if (EPI == EPI_F32) {
          float* C = (float*)p.C;
          size_t off = (size_t)m * p.ldc + n;
          if (p.splits > 1 || p.splits2 > 0) {
            C = p.partial + (size_t)split * p.M * p.N;
            off = (size_t)m * p.N + n;
          } else if (p.accumulate) {
            const f32x4 o = *(const f32x4*)(C + off);
            v[0] += o[0]; v[1] += o[1]; v[2] += o[2]; v[3] += o[3];
          }
          __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, (f32x4*)(C + off));
        } else {
          OT* C = (OT*)p.C;
          const size_t off = (size_t)m * p.ldc + n;
          OV o;
          if (EPI == EPI_RESID) {
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = (OT)(v[e] + (float)rv[k][e]);
          } else if (EPI == EPI_AXPBY) {
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = (OT)(p.alpha * v[e] + p.beta * (float)rv[k][e]);

          } else if (EPI == EPI_DRELU2 || EPI == EPI_DSQR) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float r = fmaxf((float)rv[k][e], 0.f);
              const float dv = v[e] * 2.0f * (EPI == EPI_DSQR ? __builtin_amdgcn_sqrtf(r) : r);  // v_sqrt_f32 (1 ulp)
              o[e] = (OT)dv;
              am = fmaxf(am, fabsf(dv));
            }
          } else if (EPI == EPI_SQR) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float rl = fmaxf(v[e], 0.f);
              o[e] = (OT)(rl * rl);
              am = fmaxf(am, rl * rl);
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = (OT)v[e];
          }
          __builtin_nontemporal_store(o, (OV*)(C + off));
          if (EPI == EPI_RELU2) {
            OV h;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float rl = fmaxf(v[e], 0.f);
              h[e] = (OT)(rl * rl);
              am = fmaxf(am, rl * rl);
            }
            __builtin_nontemporal_store(h, (OV*)((OT*)p.C2 + off));
          }
        }
      }
    }
    }
    if (q == 0) __syncthreads();
  }
  }
  if constexpr (EPI == EPI_RELU2 || EPI == EPI_DRELU2 || EPI == EPI_SQR || EPI == EPI_DSQR) {
    if (p.amax_out) {
      // rounding is monotone: the largest stored value is the rounded largest value
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
      if (lane == 0) atomicMax((unsigned*)p.amax_out, __float_as_uint((float)(OT)am));
    }
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
        else if (EPI == EPI_DSQR) *C = v * 2.0f * sqrtf(fmaxf(((const float*)p.R)[(size_t)m * p.ldr + n], 0.f));
        else if (EPI == EPI_AXPBY) *C = p.alpha * v + p.beta * ((const float*)p.R)[(size_t)m * p.ldr + n];
        else if (EPI == EPI_SQR) *C = fmaxf(v, 0.f) * fmaxf(v, 0.f);
        else *C = v;
        if (EPI == EPI_RELU2) {
          const float r = fmaxf(v, 0.f);
          ((float*)p.C2)[(size_t)m * p.ldc + n] = r * r;
        }
      }
    }
  }
}

template <bool AK, bool BKM, bool F8 = false, typename OT = bf16, int NW = 4, bool RING = false>
hipError_t launch_bf16(const GemmArgs& a, dim3 g, hipStream_t s) {
  g.z = a.batch > 1 ? a.batch : 1;
  switch (a.epi) {
    case EPI_STORE: hipLaunchKernelGGL((gemm_bf16_k<AK, BKM, EPI_STORE, F8, OT, NW, RING>), g, dim3(64 * NW), 0, s, a); break;
    case EPI_RESID: hipLaunchKernelGGL((gemm_bf16_k<AK, BKM, EPI_RESID, F8, OT, NW, RING>), g, dim3(64 * NW), 0, s, a); break;
    case EPI_RELU2: hipLaunchKernelGGL((gemm_bf16_k<AK, BKM, EPI_RELU2, F8, OT, NW, RING>), g, dim3(64 * NW), 0, s, a); break;
    case EPI_DRELU2: hipLaunchKernelGGL((gemm_bf16_k<AK, BKM, EPI_DRELU2, F8, OT, NW, RING>), g, dim3(64 * NW), 0, s, a); break;
    case EPI_SQR:  // the MLP up-projection: both operands K-major
      if constexpr (AK && BKM) {
        hipLaunchKernelGGL((gemm_bf16_k<AK, BKM, EPI_SQR, F8, OT, NW, RING>), g, dim3(64 * NW), 0, s, a);
        break;
      }
      return hipErrorInvalidValue;
    case EPI_DSQR:  // the hidden gradient: dout K-major, the weight either way
      if constexpr (AK) {
        hipLaunchKernelGGL((gemm_bf16_k<AK, BKM, EPI_DSQR, F8, OT, NW, RING>), g, dim3(64 * NW), 0, s, a);
        break;
      }
      return hipErrorInvalidValue;
    case EPI_QKNORM:
      if constexpr (AK && BKM && !F8 && std::is_same<OT, bf16>::value) {
        hipLaunchKernelGGL((gemm_bf16_k<AK, BKM, EPI_QKNORM, F8, OT, NW, RING>), g, dim3(64 * NW), 0, s, a);
        break;
      }
      return hipErrorInvalidValue;
    case EPI_F32:
      if constexpr (std::is_same<OT, bf16>::value) {
        hipLaunchKernelGGL((gemm_bf16_k<AK, BKM, EPI_F32, F8, OT, NW, RING>), g, dim3(64 * NW), 0, s, a);
        break;
      }
      return hipErrorInvalidValue;
    case EPI_AXPBY:
      if constexpr (!F8) {
        hipLaunchKernelGGL((gemm_bf16_k<AK, BKM, EPI_AXPBY, F8, OT, NW, RING>), g, dim3(64 * NW), 0, s, a);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

namespace {
int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    cus[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  }
  return cus[dev];
}
}  // namespace

int gemm_splits(int dt, int M, int N, int K, int epi) {
  if (epi != EPI_F32) return 1;
  const int tile = dt == F32 ? FT : BM;
  const int tiles = ((M + tile - 1) / tile) * ((N + tile - 1) / tile);
  const int kstep = dt == F32 ? FK : (dt == FP8 ? BK8 : BK);
  if (dt == F32) {
    int s = 1;
    // aim for >= 2 workgroups per CU, keep >= 8 K steps per split
    while (tiles * s < 512 && (K / (kstep * (s * 2))) >= 8 && s < 32) s *= 2;
    return s;
  }
  // MFMA path (one workgroup per CU): pick the split count with the least
  // modelled time, in units of one workgroup K step: the rounds of
  // workgroups the CUs run times each one's K steps, plus the split partials'
  // store and reduction (about 0.066 step per 256x256 fp32 tile).  Keeps at
  // least 4 K steps per split.
  const int cus = device_cus();
  const int nsteps = (K + kstep - 1) / kstep;
  int best = 1;
  double bt = 1e300;
  for (int sp = 1; sp <= 32; ++sp) {
    if (sp > 1 && nsteps / sp < 4) break;
    const double rounds = (double)((tiles * sp + cus - 1) / cus);
    const double t = rounds * ((nsteps + sp - 1) / sp) + (sp > 1 ? 0.066 * tiles * sp : 0.0);
    if (t < bt - 1e-9) {
      bt = t;
      best = sp;
    }
  }
  return best;
}

// Two-phase split-K.  With one split count for every tile, the weight
// gradients' tile counts leave the last round of workgroups part-full (144
// tiles of a 6144 x 1536 product: 5 splits, 720 workgroups, 2.8 rounds).  Two
// bands of whole tile rows or columns with two split counts can fill the
// rounds (126 tiles x 2 splits, then 18 x 14 short pieces), at the price of
// more partial slices.  The plan takes the cheapest band and split counts by
// the same cost model (rounds x steps per piece + partial traffic), the longer
// pieces first, and only when the model gains over 3%.
#ifndef GEMM_TWO_PHASE
#define GEMM_TWO_PHASE 1
#endif
SplitPlan gemm_split_plan(int dt, int M, int N, int K) {
  SplitPlan pl{gemm_splits(dt, M, N, K, EPI_F32), 0, 0, 0};
  if (!GEMM_TWO_PHASE || dt == F32 || M <= 0 || N <= 0 || K <= 0) return pl;
  const int nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN;
  const int kstep = dt == FP8 ? BK8 : BK;
  const int nsteps = (K + kstep - 1) / kstep;
  const int cus = device_cus();
  auto cost = [&](int tiles, int sp, bool part) {
    if (tiles == 0) return 0.0;
    return (double)((tiles * sp + cus - 1) / cus) * ((nsteps + sp - 1) / sp) + (part ? 0.066 * tiles * sp : 0.0);
  };
  const double one = cost(nbm * nbn, pl.splits, pl.splits > 1);
  double best = 0.97 * one;
  for (int cols = 0; cols < 2; ++cols) {
    const int bands = cols ? nbn : nbm, other = cols ? nbm : nbn;
    for (int f1 = 1; f1 < bands; ++f1)
      for (int s1 = 1; s1 <= 32; ++s1) {
        if (s1 > 1 && nsteps / s1 < 4) break;
        for (int s2 = s1; s2 <= 32; ++s2) {
          if (s2 > 1 && nsteps / s2 < 4) break;
          const double c = cost(f1 * other, s1, true) + cost((bands - f1) * other, s2, true);
          if (c < best - 1e-9) {
            best = c;
            pl = SplitPlan{s1, cols, f1, s2};
          }
        }
      }
  }
  return pl;
}

// workgroups of a launch: one phase (tiles, splits) or two
static dim3 gemm_grid(const GemmArgs& a) {
  const int nbm = (a.M + BM - 1) / BM, nbn = (a.N + BN - 1) / BN;
  if (a.splits2 > 0) {
    const int r1 = a.split_cols ? nbm : a.first1, c1 = a.split_cols ? a.first1 : nbn;
    const int t2 = nbm * nbn - r1 * c1;
    return dim3(r1 * c1 * a.splits + t2 * a.splits2, 1);
  }
  return dim3(nbm * nbn, a.splits);
}

hipError_t gemm_fp8(int out_dt, const GemmArgs& a, hipStream_t s) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  if (!a.a_kmajor || !a.b_kmajor || !a.amax_a || !a.amax_b) return hipErrorInvalidValue;
  if (a.splits2 > 0 && (a.epi != EPI_F32 || a.batch > 1)) return hipErrorInvalidValue;
  const dim3 g = gemm_grid(a);
  if (out_dt == F32 && a.epi != EPI_F32) return launch_bf16<true, true, true, float, 8>(a, g, s);
  return launch_bf16<true, true, true, bf16, 8>(a, g, s);
}

hipError_t gemm(int dt, const GemmArgs& a, hipStream_t s) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  if (a.batch > 1 && a.splits > 1) return hipErrorInvalidValue;  // a batch runs unsplit
  if (a.splits2 > 0 && (dt != BF16 || a.epi != EPI_F32 || a.batch > 1)) return hipErrorInvalidValue;
  if (dt == BF16) {
    dim3 g = gemm_grid(a);
    // 8 waves (two per SIMD, one wave's MFMAs running while the other waits
    // on its copies or LDS reads): measured 2-10% faster than 4 with both
    // operands copied straight into LDS, 4-6% with an M/N-contiguous operand
    // loaded into registers (each thread loading half of its 8x8 block)
    if (a.a_kmajor && a.b_kmajor) {
#if GEMM_RING
      const int ksplit = ((a.K + a.splits * BK - 1) / (a.splits * BK)) * BK;
      if (a.K % 128 == 0 && ksplit % 128 == 0) return launch_bf16<true, true, false, bf16, RING_NW, true>(a, g, s);
#endif
      return launch_bf16<true, true, false, bf16, GEMM_NW>(a, g, s);
    }
    if (a.a_kmajor) return launch_bf16<true, false, false, bf16, 8>(a, g, s);
    if (!a.b_kmajor) return launch_bf16<false, false, false, bf16, 8>(a, g, s);
    return launch_bf16<false, true, false, bf16, 8>(a, g, s);
  }
  if (a.batch > 1) {  // the fp32 path takes blockIdx.z for split-K: one launch per item
    for (int z = 0; z < a.batch; ++z) {
      GemmArgs b = a;
      b.batch = 1;
      b.A = (const float*)a.A + (size_t)z * a.bsA;
      b.B = (const float*)a.B + (size_t)z * a.bsB;
      b.C = (float*)a.C + (size_t)z * a.bsC;
      if (a.R) b.R = (const float*)a.R + (size_t)z * a.bsR;
      const hipError_t e = gemm(dt, b, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  dim3 g((a.M + FT - 1) / FT, (a.N + FT - 1) / FT, a.splits);
  switch (a.epi) {
    case EPI_STORE: hipLaunchKernelGGL(gemm_f32_k<EPI_STORE>, g, dim3(256), 0, s, a); break;
    case EPI_RESID: hipLaunchKernelGGL(gemm_f32_k<EPI_RESID>, g, dim3(256), 0, s, a); break;
    case EPI_RELU2: hipLaunchKernelGGL(gemm_f32_k<EPI_RELU2>, g, dim3(256), 0, s, a); break;
    case EPI_DRELU2: hipLaunchKernelGGL(gemm_f32_k<EPI_DRELU2>, g, dim3(256), 0, s, a); break;
    case EPI_F32: hipLaunchKernelGGL(gemm_f32_k<EPI_F32>, g, dim3(256), 0, s, a); break;
    case EPI_SQR: hipLaunchKernelGGL(gemm_f32_k<EPI_SQR>, g, dim3(256), 0, s, a); break;
    case EPI_DSQR: hipLaunchKernelGGL(gemm_f32_k<EPI_DSQR>, g, dim3(256), 0, s, a); break;
    case EPI_AXPBY: hipLaunchKernelGGL(gemm_f32_k<EPI_AXPBY>, g, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gdb
