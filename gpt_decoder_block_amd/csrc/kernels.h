// Internal launchers of the gfx950 kernels (not part of the public ABI).
// Every launcher enqueues on `s` and returns the launch status; shapes have
// been validated by the caller (api.cpp).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;

namespace gdb {

// storage dtype of activations/weights; FP8 (OCP e4m3 codes) only names the
// operand type of the fp8 GEMM
enum Dt { F32 = 0, BF16 = 1, FP8 = 2 };

inline int dt_size(int dt) { return dt == BF16 ? 2 : 4; }

// ---------------------------------------------------------------- elementwise
hipError_t fill_f32(float* p, size_t n, float v, hipStream_t s);
// dst = src over `bytes` (a multiple of 16): the bandwidth reference copy
hipError_t stream_copy(const void* src, void* dst, size_t bytes, hipStream_t s);
// Debug scan: *bad = whether any of the n elements (dt: F32 or BF16) is NaN or
// infinite.  Synchronises s; the flag is a static device word.
hipError_t any_nonfinite(int dt, const void* x, size_t n, hipStream_t s, bool* bad);
// out [Cc, R] = in [R, Cc]^T, bf16, R and Cc multiples of 8, out not aliasing in
hipError_t transpose_bf16(const void* in, int R, int Cc, void* out, hipStream_t s);
// xn = x * r, r = 1/sqrt(mean(x^2)+eps) per row of [N, C]
// amax (optional): atomically raised to the largest |xn| stored; zeroed by the caller
hipError_t rmsnorm_fwd(int dt, const void* x, void* xn, float* r, int N, int C, float eps, hipStream_t s,
                       float* amax = nullptr);
// dx = r*(dxn - xn*mean(dxn*xn)) (+ dres if non-null); dx may alias dres
hipError_t rmsnorm_bwd(int dt, const void* dxn, const void* xn, const float* r, const void* dres,
                       void* dx, int N, int C, hipStream_t s);
hipError_t embed_fwd(int dt, const int32_t* ids, const void* wte, void* x, int N, int C, int V, hipStream_t s);
hipError_t embed_bwd(int dt, const int32_t* ids, const void* dx, float* dwte, int N, int C, int V,
                     int accumulate, hipStream_t s);
// QK RMS-norm + RoPE on [N, Q+2KV] rows: q, k heads normalised over D and
// rotated, v copied.  rinv [N, H+Hkv] fp32 (inverse RMS of each q/k head).
hipError_t qk_norm_rope_fwd(int dt, const void* qkv, void* qkvh, float* rinv, const float* rope,
                            int B, int T, int H, int Hkv, int D, float eps, hipStream_t s);
// In place on d (= dqkvh [N, Q+2KV]): dq = r * R^-1 (dqh - qh*mean(dqh*qh)), same for k.
hipError_t qk_norm_rope_bwd(int dt, void* d, const void* qkvh, const float* rinv, const float* rope,
                            int B, int T, int H, int Hkv, int D, hipStream_t s);
// Cross-entropy on logits z [N, V] (in place: z <- (softmax - onehot)/N), per-row loss.
hipError_t ce_fwd_bwd(int dt, void* z, const int32_t* tgt, float* row_loss, int N, int V, hipStream_t s);
// loss = sum(row_loss)/N (one deterministic workgroup)
hipError_t loss_reduce(const float* row_loss, float* loss, int N, hipStream_t s);
// C (+)= sum_z partial[z] over `splits` fp32 [M, N] slices
hipError_t splitk_reduce(const float* partial, float* C, int splits, size_t MN, int accumulate, hipStream_t s);
// the same for a two-phase plan: element (m, n) of C [M, N] sums the first
// `splits` slices if its tile row (split_cols == 0: m / 256) or tile column
// (n / 256) is below first1, else the first `splits2`
hipError_t splitk_reduce2(const float* partial, float* C, int M, int N, int splits, int split_cols, int first1,
                          int splits2, int accumulate, hipStream_t s);

// ----------------------------------------------------------------------- GEMM
// C[m, n] = sum_k A(m, k) * B(n, k)
//   A(m,k) = a_kmajor ? A[m*lda + k] : A[k*lda + m]
//   B(n,k) = b_kmajor ? B[n*ldb + k] : B[k*ldb + n]
enum Epi {
  EPI_STORE = 0,   // C = acc                       (dtype out)
  EPI_RESID = 1,   // C = R + acc                   (dtype out, R may alias C)
  EPI_RELU2 = 2,   // C = acc (u), C2 = relu(acc)^2  (dtype out)
  EPI_DRELU2 = 3,  // C = acc * 2*max(R, 0)          (dtype out, R = saved u)
  EPI_F32 = 4,     // fp32 C (+)= acc (split-K through `partial`)
  EPI_QKNORM = 5,  // bf16, both operands K-major, head_dim 128: the QKV projection
                   // with the QK RMS-norm and RoPE applied to the q and k heads
                   // (columns < qk_heads*128) on the way out; rinv [M, qk_heads]
  EPI_SQR = 6,     // C = relu(acc)^2 only (the block saves h, not u)
  EPI_DSQR = 7,    // C = acc * 2*sqrt(max(R, 0)), R = saved h = relu(u)^2, so
                   // 2*sqrt(h) = 2*relu(u) is the ReLU^2 derivative
  EPI_AXPBY = 8    // C = alpha*acc + beta*R (dtype out, R must not alias C): the
                   // Newton-Schulz lines b*A + c*A@A and a*X + X@B
};
struct GemmArgs {
  const void* A; const void* B;
  int M, N, K, lda, ldb;
  bool a_kmajor, b_kmajor;
  int epi;
  void* C; int ldc;
  const void* R; int ldr;
  void* C2;
  int accumulate;      // EPI_F32
  float alpha, beta;   // EPI_AXPBY
  // batched launch (bf16/fp8 path, splits == 1): item z of `batch` reads and
  // writes at these element offsets times z (0 or 1: one item)
  int batch;
  long long bsA, bsB, bsC, bsR;
  float* partial;      // EPI_F32 split-K scratch [max(splits, splits2), M, N] or null
  int splits;          // >= 1
  // two-phase split-K (EPI_F32, bf16 and fp8 paths): when splits2 > 0, the
  // tiles of the first `first1` tile rows (split_cols == 0) or tile columns
  // (split_cols == 1) take `splits` K ranges and the other tiles `splits2`,
  // in one launch whose first-phase workgroups come first; every tile then
  // writes partials, which splitk_reduce sums with the same phase rule
  int split_cols, first1, splits2;
  const float* amax_a; // fp8: per-tensor amax of A and B (scales amax/448)
  const float* amax_b;
  // EPI_RELU2 / EPI_SQR / EPI_DRELU2 / EPI_DSQR: if set, atomically raised to
  // the largest |value| stored in C2 (ReLU2) or C (the others) -- the next
  // quantiser's amax; the caller zeroes it first
  float* amax_out;
  // EPI_QKNORM: rope table [T][64][2], row m is position m % T
  const float* rope; float* rinv; int T; int qk_heads; float eps;
};
hipError_t gemm(int dt, const GemmArgs& a, hipStream_t s);
// fp8 e4m3 codes, both operands K-major (lda, ldb in codes, multiples of 16);
// K a multiple of 16.  Epilogues as the bf16 GEMM; C, C2 and R of the
// epilogues other than EPI_F32 have dtype out_dt (BF16 or F32).
hipError_t gemm_fp8(int out_dt, const GemmArgs& a, hipStream_t s);
// split-K factor the GEMM will use for this shape (dt FP8 for gemm_fp8)
int gemm_splits(int dt, int M, int N, int K, int epi);
// split-K plan of an EPI_F32 product (dt BF16 or FP8): one phase (splits2 ==
// 0, splits = gemm_splits) or two phases as GemmArgs describes them
struct SplitPlan {
  int splits, split_cols, first1, splits2;
};
SplitPlan gemm_split_plan(int dt, int M, int N, int K);
// fp32 partial slices a plan writes ([slices, M, N])
inline int plan_slices(const SplitPlan& p) { return p.splits2 > p.splits ? p.splits2 : p.splits; }

// ------------------------------------------------------------ fp8 quantiser
// amax[0] = max |x| over n elements (x dtype dt; n a multiple of 8); amax is
// zeroed first (stream-ordered) unless zero = false (the word was zeroed
// already, e.g. with its neighbours in one fp8_amax_zero launch).
hipError_t fp8_amax(int dt, const void* x, size_t n, float* amax, hipStream_t s, bool zero = true);
// zero the `count` amax accumulators at amax (count <= 64; before the
// producers that raise them)
hipError_t fp8_amax_zero(float* amax, hipStream_t s, int count = 1);
// codes e4m3(x / s), s = amax / 448 (float32 division, round to nearest
// even, saturating at 448): x [R, Cc] (dt), Cc a multiple of 16; xq [R, Cc]
// row-major (or null); xqt [Cc, Rp] the transpose with rows R..Rp-1 zero (or
// null), Rp a multiple of 16 and >= R.
hipError_t fp8_quant(int dt, const void* x, int R, int Cc, const float* amax, uint8_t* xq, uint8_t* xqt, int Rp,
                     hipStream_t s);

// ------------------------------------------------------------------ attention
// q, k, v: rows of qkvh [N, ld] at column offsets 0, H*D, (H+Hkv)*D.
struct AttnArgs {
  int B, T, H, Hkv, D, window;
  int qk_normed;                  // q^, k^ rows have RMS <= 1 (QK RMS-norm output)
  const void* qkv; int ld;        // q^, k^, v (row stride ld)
  void* o; int ldo;               // [N, H*D]
  float* lse;                     // [B, H, T]
  // backward
  const void* dout; int lddo;     // dO [N, H*D]
  void* dqkv; int lddq;           // dq^, dk^, dv written at the same offsets
  float* delta;                   // [B, H, T] scratch: rowsum(dO * O)
  float* dq_acc;                  // fp32 scratch [N, H*D] (fp32 path)
  // bf16 backward: if rope is set, dq and dk are taken back through the QK
  // RMS-norm and RoPE on the way out (gradients w.r.t. the raw q, k); rope
  // [T][D/2][2] (cos, sin), rinv [B*T, H + Hkv] of the forward
  const float* rope; const float* rinv;
};
hipError_t attn_fwd(int dt, const AttnArgs& a, hipStream_t s);
hipError_t attn_bwd(int dt, const AttnArgs& a, hipStream_t s);

// decode attention: query row b (q heads at columns h*D of row b, stride ldq)
// against cache rows j of sequence b (k, v at b*bstride + j*ldk + g*D);
// lens [B] device int32, clamped to [0, max_len]
struct DecodeArgs {
  int B, H, Hkv, D, window, max_len;
  int chunk;                      // keys per split (set by attn_decode)
  const void* q; int ldq;
  const void* k; const void* v; int ldk; long long bstride;
  const int32_t* lens;
  void* o; int ldo;               // [B, ldo]
  float* lse;                     // [B, H] or null
  float* part;                    // [B, H, nsplit, D + 4] fp32 (nsplit > 1): o, m, l
};
bool decode_group_supported(int G);
// split plan: keys per split and number of splits for the longest sequence
void decode_plan(int B, int Hkv, int max_len, int window, int* chunk, int* nsplit);
hipError_t attn_decode(int dt, const DecodeArgs& a, hipStream_t s);
// fixed per-device scratch of the allocation-free decode: its size, and its
// device address on the current device (looked up once per device)
size_t decode_scratch_bytes();
hipError_t decode_scratch(void** out);

// --------------------------------------------------------------------- extras
// Kernels that reduce scalar gradients write one fp32 partial row per
// workgroup; *_partials(N) gives the number of rows (at most EXTRA_PBLK for the
// grid-stride ones), then one workgroup adds them in a fixed order.
constexpr int EXTRA_PBLK = 1024;
int mix_partials(int N);        // rows of 2 floats
int ve_gate_partials(int N);    // rows of Hkv*nc floats
int smear_partials(int N);      // rows of ng+1 floats
int backout_partials(int N);    // rows of 1 float
// y = lam[0]*x + lam[1]*x0 (n elements)
hipError_t mix_fwd(int dt, const void* x, const void* x0, const float* lam, void* y, size_t n, hipStream_t s);
// dx = lam[0]*dy (may alias dy); dx0 (+)= lam[1]*dy (fp32); dlam (+)= (sum dy*x, sum dy*x0)
hipError_t mix_bwd(int dt, const void* dy, const void* x, const void* x0, const float* lam, void* dx, float* dx0,
                   int acc_dx0, float* part, float* dlam, int accumulate, int N, int C, hipStream_t s);
// v columns (offset voff) of qkv [N, ldq] += 3*sigmoid(xn[:, :nc] Wg^T) * VE[ids]; s_save [N, Hkv]
hipError_t ve_fwd(int dt, void* qkv, int ldq, int voff, const void* xn, int C, const int32_t* ids, const void* ve,
                  const void* wg, int nc, int Hkv, int D, int V, float* s_save, int N, hipStream_t s);
// ds [N, Hkv] (gradient of the gate logits) and, if dve is non-null, dve (fp32 atomics) from the v
// columns of dqkv
hipError_t ve_bwd(int dt, const void* dqkv, int ldq, int voff, const int32_t* ids, const void* ve,
                  const float* s_save, int Hkv, int D, int V, float* ds, float* dve, int N, hipStream_t s);
// dxn[:, :nc] += ds Wg; dwg (+)= ds^T xn[:, :nc]
hipError_t ve_gate_bwd(int dt, const float* ds, const void* xn, void* dxn, int C, const void* wg, int nc, int Hkv,
                       float* part, float* dwg, int accumulate, int N, hipStream_t s);
// x[t] = e[t] + lam*sigmoid(e[t, :ng] . w)*e[t-1] (t >= 1 within each row of T tokens); s_save [N]
hipError_t smear_fwd(int dt, const void* e, const void* w, int ng, const float* lam, void* x, float* s_save, int N,
                     int T, int C, hipStream_t s);
// de from dx (+ optional fp32 dxa); dlam, dw (+)=
hipError_t smear_bwd(int dt, const void* e, const void* w, int ng, const float* lam, const float* s_save,
                     const void* dx, const float* dxa, void* de, float* part, float* dlam, float* dw, int accumulate,
                     int N, int T, int C, hipStream_t s);
// y = x - lam*xb
hipError_t backout_fwd(int dt, const void* x, const void* xb, const float* lam, void* y, size_t n, hipStream_t s);
// dxb += -lam*dy (in place); dlam (+)= -sum(dy*xb)
hipError_t backout_bwd(int dt, const void* dy, const void* xb, const float* lam, void* dxb, float* part, float* dlam,
                       int accumulate, int N, int C, hipStream_t s);

// ------------------------------------------------------- fixed-order scatter
// bytes of scratch token_order needs for N tokens
size_t token_order_ws_bytes(int N);
// stable sort of the token indices 0..N-1 by id (ids clamped into [0, V)):
// *sorted_ids and *perm point into ws on return (sorted_ids[j] = id of token perm[j])
hipError_t token_order(const int32_t* ids, int N, int V, void* ws, const int32_t** sorted_ids, const int32_t** perm,
                       hipStream_t s);
// out[v, c] (+)= sum over tokens n of id v, in sorted order, of g(n, c) * x[n*ldx + xoff + c] (c < width),
// g = 3*sigmoid(gate_s[n*G + c/D]) if gate_s is non-null, else 1; every row v < V is written
hipError_t rows_segsum(int dt, const int32_t* sorted_ids, const int32_t* perm, int N, const void* x, int ldx, int xoff,
                       int width, const float* gate_s, int G, int D, float* out, int V, int accumulate, hipStream_t s);

// ------------------------------------------------------------------ optimizer
constexpr int OPT_PART = 1024;  // most workgroups (partials) of the reductions below
// Stacks of `count` matrices of n elements each (n a multiple of 4); the
// partials of item i at part[i * OPT_PART ..], *np per item.
// partial sums of x^2
hipError_t sumsq_partials(const float* x, size_t n, int count, float* part, int* np, hipStream_t s);
// buf = mu*buf + g; u = nesterov ? g + mu*buf : buf; partial sums of u^2
hipError_t muon_momentum(const float* g, float* buf, float* u, size_t n, int count, float mu, int nesterov,
                         float* part, int* np, hipStream_t s);
// inv[i] = 1 / (sqrt(sum of item i's partials) * norm_scale + eps)
hipError_t norm_final(const float* part, int np, int count, float norm_scale, float eps, float* inv, hipStream_t s);
// x = g * inv[i] per item (dtype dt)
hipError_t scale_cast(int dt, const float* g, const float* inv, void* x, size_t n, int count, hipStream_t s);
// out = alpha * (sum of `splits` fp32 partials [splits][n]) + beta * R (dtype dt; R may be null)
hipError_t splitk_axpby(int dt, const float* part, int splits, size_t n, float alpha, float beta, const void* R,
                        void* out, hipStream_t s);
// p = p*decay - step*x (x dtype dt); plow (bf16 copy of p) if non-null
hipError_t muon_apply(int dt, float* p, const void* x, bf16* plow, size_t n, float decay, float step, hipStream_t s);
// NorMuon statistics of the NS output x (count items of [m, n], dtype dt): per row r of item i,
// vmean = mean_j x^2, v = beta2*v + (1-beta2)*vmean (state), step = 1/sqrt(max(v, 1e-10)); then per
// item fs[r] = step[r]*sqrt(sum vmean)/max(sqrt(sum vmean*step^2), 1e-10) (fixed-order sums).
// stat: fp32 scratch [2][count*m]; fs [count*m] receives the row factors.
hipError_t normuon_scale(int dt, const void* x, int count, int m, int n, float* v, float beta2, float* stat,
                         float* fs, hipStream_t s);
// p = p*decay - step*fs[row]*x (x dtype dt, rows of n elements); plow (bf16 copy of p) if non-null
hipError_t normuon_apply(int dt, float* p, const void* x, const float* fs, bf16* plow, size_t rows, int n,
                         float decay, float step, hipStream_t s);
// one AdamW step (t counts steps, this one included)
hipError_t adamw(float* p, const float* g, float* m, float* v, bf16* plow, size_t n, float lr, float b1, float b2,
                 float eps, float wd, int t, hipStream_t s);

}  // namespace gdb
