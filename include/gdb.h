/*
 * gdb.h — C ABI of the MI355X (gfx950) decoder-block training hot path.
 *
 * One training step of a nanochat-style GPT as the pages describe it
 * ("Comment Entraîner Votre Propre ChatGPT Pour 50€ ?", section "1. Le modèle
 * GPT": rotary embeddings, QK normalisation, untied token embedding and output
 * projection, ReLU² MLP, grouped-query attention, sliding-window attention;
 * section "3. Gestion de la précision": bias-free Linear layers F.linear(x, W)
 * with W stored [out, in] and explicit compute dtypes):
 *
 *   gdb_embed_fwd -> L x gdb_block_fwd -> gdb_lm_head_ce_fwd_bwd
 *                 -> L x gdb_block_bwd (reverse order) -> gdb_embed_bwd
 *
 * The largest model adds (same section: the value-embedding snippet and the
 * snippets on per-layer residual scaling, smear and backout):
 *
 *   gdb_embed_fwd -> gdb_smear_fwd -> L x gdb_block_fwd(extras) -> gdb_backout_fwd
 *     -> gdb_lm_head_ce_fwd_bwd -> gdb_backout_bwd (when the backward reaches
 *     the block whose output was subtracted) ... L x gdb_block_bwd(extras)
 *     -> gdb_smear_bwd -> gdb_embed_bwd
 *
 * Beside the training step: the optimizer step that follows it
 * (gdb_adamw_step, gdb_muon_step on gdb_newton_schulz) and the generation
 * step of the inference engine (gdb_attention_decode against a KV cache).
 *
 * Conventions shared by every entry point
 *   - Pointers named in a signature are DEVICE pointers unless the comment
 *     says "host".  The caller allocates every buffer (inputs, outputs, saved
 *     activations, workspace); the library never allocates or frees device
 *     memory, never synchronises, and enqueues all work on `stream`
 *     (a hipStream_t passed as void*, NULL = the default stream).
 *   - Activations are row-major [N, C] with N = B*T tokens (row n = b*T + t);
 *     attention views the same memory as [B, T, heads, head_dim].
 *   - dtype GDB_F32: every tensor float32, fp32 arithmetic throughout.
 *     dtype GDB_BF16: weights, activations and activation gradients bfloat16
 *     (round to nearest even); GEMM accumulation, norm statistics, softmax,
 *     log-sum-exp and the loss in float32.  Weight gradients are always
 *     float32 (the masters are fp32).
 *   - Weight gradients are overwritten, or added to when `accumulate` /
 *     cfg->accumulate_wgrad is non-zero (gradient accumulation).
 *   - Every function validates its arguments before enqueuing anything and
 *     returns a gdb_status; on failure gdb_last_error() describes the problem.
 *     No function aborts or throws across the boundary.  Errors from the HIP
 *     runtime (a failed launch) return GDB_EHIP.
 *   - Device pointers must be non-NULL and 16-byte aligned; feature sizes
 *     (C, head_dim, mlp_hidden, V) must be multiples of 8.
 *   - Debug check: with the environment variable GDB_CHECK_FINITE set to a
 *     value other than "0" (read on every call), gdb_block_fwd (x_out),
 *     gdb_block_bwd (dx_in and the four weight gradients) and
 *     gdb_lm_head_ce_fwd_bwd (loss, dx, dw_lm) scan their outputs after the
 *     work and return GDB_ENONFINITE, naming the first tensor that holds a NaN
 *     or an infinity.  The scan synchronises `stream` (the only entry points
 *     that do, and only in this mode); its flag is a static device word, so
 *     nothing is allocated.  Checked calls on one device must not overlap.
 */
#ifndef GDB_H
#define GDB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDB_ABI_VERSION 7

/* Scratch bytes that gdb_smear_bwd and gdb_backout_bwd need in `ws`. */
#define GDB_EXTRAS_WS_BYTES ((size_t)1 << 20)

typedef enum {
  GDB_OK = 0,
  GDB_EINVAL = -1,        /* bad argument (shape, pointer, alignment, dtype) */
  GDB_EUNSUPPORTED = -2,  /* valid but not implemented (e.g. head_dim 96)     */
  GDB_EHIP = -3,          /* the HIP runtime reported an error                */
  GDB_EWORKSPACE = -4,    /* a size query's answer was not respected          */
  GDB_ENONFINITE = -5     /* debug check (GDB_CHECK_FINITE): an output holds NaN or Inf */
} gdb_status;

typedef enum { GDB_F32 = 0, GDB_BF16 = 1 } gdb_dtype;

/* Shape and options of one decoder block.
 *   Q = n_head*head_dim must equal C; KV = n_kv_head*head_dim;
 *   n_head % n_kv_head == 0 (query head h reads K/V head h / (n_head/n_kv_head));
 *   head_dim in {64, 128} (bf16: 128 only); window: < 0 full causal, else key j
 *   is visible from query i iff 0 <= i - j <= window ("window_size" argument of
 *   the attention call, section "5. Unification de Flash Attention").
 *   eps: RMSNorm epsilon (1e-6), used for the block norms and the QK norm.   */
typedef struct {
  int32_t B, T, C;
  int32_t n_head, n_kv_head, head_dim;
  int32_t mlp_hidden;         /* F, the ReLU² MLP width (4*C in every workload) */
  int32_t window;
  int32_t dtype;              /* gdb_dtype */
  int32_t mlp_fp8;            /* the MLP's six products on OCP e4m3 codes (gdb_fp8_quantize) */
  int32_t accumulate_wgrad;   /* 0: dW = ..., 1: dW += ... */
  int32_t deterministic;      /* 1: gdb_block_bwd's results are the same bits on every run (the value
                                 embedding table's gradient sums its tokens in a fixed order instead of
                                 with float atomics); every other reduction of the block is always in a
                                 fixed order */
  float eps;
} gdb_block_cfg;

/* Block weights, all [out, in] row-major in cfg->dtype:
 *   w_qkv  [Q + 2*KV, C]  rows: the Q query rows (head-major), then KV key rows, then KV value rows
 *   w_o    [C, Q]
 *   w_fc   [F, C]
 *   w_proj [C, F]                                                              */
typedef struct {
  const void *w_qkv, *w_o, *w_fc, *w_proj;
} gdb_block_weights;

/* fp32 weight gradients, same shapes as gdb_block_weights. */
typedef struct {
  float *dw_qkv, *dw_o, *dw_fc, *dw_proj;
} gdb_block_wgrads;

/* Per-block extras of the largest model (section "1. Le modèle GPT": the
 * value-embedding snippet and the per-layer residual scaling snippet).
 * Pass NULL to gdb_block_fwd / gdb_block_bwd for a plain block.
 *
 * Residual mixing, active when lambdas != NULL: the block first forms
 *   x = lambdas[0]*x_in + lambdas[1]*x0
 * and runs on x (both residual additions go onto x).
 * Value embedding, active when ve != NULL: right after the QKV projection,
 *   v[n, g, :] += 3*sigmoid(xn1[n, :nc] . ve_gate[g, :]) * ve[ids[n], g*D : (g+1)*D]
 * for every K/V head g (nc = ve_gate_channels, xn1 = the normalised x), before
 * the QK norm and attention. */
typedef struct {
  const float* lambdas;      /* fp32 [2] device: (residual scale, x0 scale); NULL: no mixing        */
  const void* x0;            /* [N, C] dtype: the stream after embedding and smear                   */
  const void* x_in;          /* gdb_block_bwd only: the x_in given to gdb_block_fwd (before mixing)  */
  const int32_t* ids;        /* int32 [N] input token ids (clamped into [0, ve_vocab))               */
  const void* ve;            /* [ve_vocab, n_kv_head*head_dim] dtype; NULL: no value embedding       */
  const void* ve_gate;       /* [n_kv_head, ve_gate_channels] dtype                                  */
  int32_t ve_vocab;
  int32_t ve_gate_channels;  /* 1 .. min(64, C); 32 in the pages' model                              */
} gdb_block_extras;

/* fp32 gradients of the extras.  dlambdas [2], dve and dve_gate are
 * overwritten, or added to when cfg->accumulate_wgrad != 0 (dve's rows are
 * summed with float atomics in no fixed order, or, with cfg->deterministic,
 * in token order after a stable sort of the ids).
 * dx0 [N, C] receives lambdas[1]*dx (the x0 share of the mixed stream's
 * gradient): overwritten, or added to when accumulate_dx0 != 0, so the
 * blocks of one backward pass can sum their shares in place. */
typedef struct {
  float* dlambdas;           /* [2] */
  float* dx0;                /* [N, C] */
  float* dve;                /* [ve_vocab, n_kv_head*head_dim] */
  float* dve_gate;           /* [n_kv_head, ve_gate_channels] */
  int32_t accumulate_dx0;
} gdb_block_extras_grads;

/* ABI version (GDB_ABI_VERSION of the built library). */
int32_t gdb_abi_version(void);

/* Text of the last error on the calling thread ("" if none). Valid until the
 * next gdb_* call on this thread. */
const char* gdb_last_error(void);

/* Sizes in bytes of the opaque `saved` buffer that gdb_block_fwd fills and
 * gdb_block_bwd reads, and of the scratch workspaces of each direction.
 * Any argument pointer may be NULL to skip that answer. */
gdb_status gdb_block_sizes(const gdb_block_cfg* cfg, size_t* saved_bytes,
                           size_t* ws_fwd_bytes, size_t* ws_bwd_bytes);

/* HOST function: fill out_host[T][head_dim/2][2] with (cos, sin) of the rotary
 * angle t * base^(-2j/head_dim), j < head_dim/2, computed in double precision
 * and rounded to float.  Dimension j is paired with j + head_dim/2; positions
 * restart at 0 on every sequence ("Embeddings rotatifs (RoPE)", section
 * "1. Le modèle GPT").  The table is copied to the device by the caller. */
gdb_status gdb_rope_table_host(int32_t T, int32_t head_dim, double base, float* out_host);

/* Token embedding lookup (untied embedding, section "1. Le modèle GPT"):
 * x0[n, :] = wte[ids[n], :].  ids int32 [N] with values in [0, V) (out-of-range
 * ids are a caller error; they are clamped, never read out of bounds);
 * wte [V, C] and x0 [N, C] in `dtype`. */
gdb_status gdb_embed_fwd(int32_t N, int32_t C, int32_t V, int32_t dtype,
                         const int32_t* ids, const void* wte, void* x0, void* stream);

/* Embedding gradient: dwte[v, :] (+)= sum of dx0[n, :] over n with ids[n] == v.
 * dx0 [N, C] in `dtype`; dwte [V, C] float32, overwritten unless `accumulate`.
 * deterministic == 0: float32 atomics, summation order not fixed (ws may be
 * NULL).  deterministic != 0: the tokens are sorted by id (stable), then each
 * row adds its tokens in token order: the same bits on every run; ws must
 * hold gdb_embed_bwd_ws_bytes bytes. */
gdb_status gdb_embed_bwd_ws_bytes(int32_t N, int32_t deterministic, size_t* ws_bytes);
gdb_status gdb_embed_bwd(int32_t N, int32_t C, int32_t V, int32_t dtype,
                         const int32_t* ids, const void* dx0, float* dwte,
                         int32_t accumulate, int32_t deterministic, void* ws, void* stream);

/* Forward of one pre-norm decoder block on x_in [N, C]:
 *   xn1 = rms(x_in); [q k v] = xn1 W_qkv^T;  q^ = rope(rms_D(q)), k^ = rope(rms_D(k));
 *   o = softmax(q^ k^T / sqrt(head_dim), causal/window mask) v  (GQA head sharing);
 *   x_mid = x_in + o W_o^T;  xn2 = rms(x_mid);  h = relu(xn2 W_fc^T)^2;
 *   x_out = x_mid + h W_proj^T.
 * ex: NULL, or the extras above (x_in is then the stream before mixing).
 * rope_tab: device copy of gdb_rope_table_host(T, head_dim, base).
 * saved: gdb_block_sizes' saved_bytes, kept intact until gdb_block_bwd.
 * ws: ws_fwd_bytes of scratch.  x_out must not alias x_in. */
gdb_status gdb_block_fwd(const gdb_block_cfg* cfg, const gdb_block_weights* w,
                         const gdb_block_extras* ex, const float* rope_tab,
                         const void* x_in, void* x_out, void* saved, void* ws, void* stream);

/* Backward of gdb_block_fwd: given dx_out [N, C] (gradient w.r.t. x_out) and
 * the `saved` buffer of the matching forward, writes dx_in [N, C] (may alias
 * dx_out) and the fp32 weight gradients.  ex: the forward's extras (with x_in
 * set when mixing) or NULL; dex: their gradients (required when ex uses any
 * extra).  ws: ws_bwd_bytes of scratch. */
gdb_status gdb_block_bwd(const gdb_block_cfg* cfg, const gdb_block_weights* w,
                         const gdb_block_extras* ex, const float* rope_tab,
                         const void* saved, const void* dx_out, void* dx_in,
                         const gdb_block_wgrads* dw, const gdb_block_extras_grads* dex,
                         void* ws, void* stream);

/* Workspace of gdb_lm_head_ce_fwd_bwd (holds the normalised stream, its
 * inverse RMS, the [N, V] logits/gradients, per-row losses). */
gdb_status gdb_lm_head_ce_sizes(int32_t N, int32_t C, int32_t V, int32_t dtype,
                                size_t* ws_bytes);

/* Final RMSNorm, lm_head and mean next-token cross-entropy, forward and
 * backward in one call:
 *   xf = rms(x); z = xf W_lm^T; loss = (1/N) sum_n (logsumexp(z_n) - z_n[targets[n]]);
 *   dz = (softmax(z) - onehot(targets)) / N;  dxf = dz W_lm;  dW_lm (+)= dz^T xf;
 *   dx = rms backward of dxf.
 * x [N, C], w_lm [V, C], dx [N, C] in `dtype`; targets int32 [N] in [0, V);
 * loss: device float32 scalar (written); row_loss: NULL, or device float32
 * [N] that receives each token's loss logsumexp(z_n) - z_n[targets[n]];
 * dw_lm [V, C] float32. */
gdb_status gdb_lm_head_ce_fwd_bwd(int32_t N, int32_t C, int32_t V, int32_t dtype, float eps,
                                  const void* x, const void* w_lm, const int32_t* targets,
                                  float* loss, float* row_loss, void* dx, float* dw_lm, int32_t accumulate,
                                  void* ws, void* stream);

/* Smear, once after the embedding (section "1. Le modèle GPT", the smear
 * snippet): with s[n] = e[n, :ng] . w,
 *   x[b, t] = e[b, t] + lam[0]*sigmoid(s[b, t])*e[b, t-1]  for t >= 1,  x[b, 0] = e[b, 0].
 * The gate reads the current token; the mixed-in vector is the previous
 * token's embedding.  e, x [B*T, C] and w [ng] in dtype, 1 <= ng <= min(63, C);
 * lam: fp32 [1] device; s_save fp32 [B*T] is written for the backward.
 * x must not alias e. */
gdb_status gdb_smear_fwd(int32_t B, int32_t T, int32_t C, int32_t ng, int32_t dtype,
                         const void* e, const void* w, const float* lam, void* x,
                         float* s_save, void* stream);
/* Backward of gdb_smear_fwd.  The gradient w.r.t. x is dx [B*T, C] (dtype)
 * plus, if dxa != NULL, the fp32 addend dxa [B*T, C] (the summed dx0 shares
 * of the blocks).  Writes de [B*T, C] (dtype; must not alias dx or dxa) and
 * the fp32 gradients dlam [1] and dw [ng], overwritten or added to
 * (`accumulate`).  ws: GDB_EXTRAS_WS_BYTES of scratch. */
gdb_status gdb_smear_bwd(int32_t B, int32_t T, int32_t C, int32_t ng, int32_t dtype,
                         const void* e, const void* w, const float* lam, const float* s_save,
                         const void* dx, const float* dxa, void* de, float* dlam, float* dw,
                         int32_t accumulate, void* ws, void* stream);

/* Backout, once before the final norm (section "1. Le modèle GPT", the backout
 * snippet): y = x - lam[0]*x_bo, where x_bo is the output of block L/2 - 1.
 * [N, C] in dtype; y may alias x but not x_bo; lam fp32 [1] device. */
gdb_status gdb_backout_fwd(int32_t N, int32_t C, int32_t dtype, const void* x, const void* x_bo,
                           const float* lam, void* y, void* stream);
/* Backward: dy is the gradient w.r.t. y.  dx_bo += -lam[0]*dy in place (call
 * it once dx_bo holds the gradient w.r.t. the output of block L/2 - 1 from the
 * blocks above); dlam (fp32 [1]) = or += -sum(dy * x_bo).  dy's gradient
 * w.r.t. x is dy itself.  ws: GDB_EXTRAS_WS_BYTES of scratch. */
gdb_status gdb_backout_bwd(int32_t N, int32_t C, int32_t dtype, const void* dy, const void* x_bo,
                           const float* lam, void* dx_bo, float* dlam, int32_t accumulate,
                           void* ws, void* stream);

/* Residual mixing of one block of the largest model (section "1. Le modèle
 * GPT", the per-layer residual scaling snippet), as gdb_block_fwd applies it
 * when gdb_block_extras.lambdas is set: y = lam[0]*x + lam[1]*x0 over
 * [N, C] rows (dtype); lam fp32 [2] device.  y may alias x. */
gdb_status gdb_mix_fwd(int32_t N, int32_t C, int32_t dtype, const void* x, const void* x0, const float* lam,
                       void* y, void* stream);
/* Its backward, given dy = the gradient w.r.t. y: dx = lam[0]*dy (dtype, may
 * alias dy); dx0 (fp32 [N, C]) = lam[1]*dy, or += when accumulate_dx0;
 * dlam (fp32 [2]) = or += (sum dy*x, sum dy*x0), summed in a fixed order.
 * ws: GDB_EXTRAS_WS_BYTES of scratch. */
gdb_status gdb_mix_bwd(int32_t N, int32_t C, int32_t dtype, const void* dy, const void* x, const void* x0,
                       const float* lam, void* dx, float* dx0, int32_t accumulate_dx0, float* dlam,
                       int32_t accumulate, void* ws, void* stream);

/* Value embedding of one block (section "1. Le modèle GPT", the
 * value-embedding snippet), as gdb_block_fwd applies it when
 * gdb_block_extras.ve is set.  For each token n and K/V head g:
 *   s[n, g] = xn[n, :nc] . wg[g, :]   (fp32, saved in s_save [N, Hkv]),
 *   v[n, g, :] += 3*sigmoid(s[n, g]) * ve[ids[n], g*D : (g+1)*D],
 * where v[n] is the row qkv + n*ldq + voff (dtype, updated in place), xn
 * [N, ldx] the block's normalised input, ve [V, Hkv*D], wg [Hkv, nc] (dtype);
 * ids int32 [N] (clamped into [0, V)).  1 <= nc <= min(64, ldx), Hkv <= 64,
 * D in {64, 128}; ldq, voff, ldx multiples of 8. */
gdb_status gdb_ve_fwd(int32_t N, int32_t Hkv, int32_t D, int32_t dtype, void* qkv, int32_t ldq, int32_t voff,
                      const void* xn, int32_t ldx, const int32_t* ids, const void* ve, int32_t V, const void* wg,
                      int32_t nc, float* s_save, void* stream);
/* Its backward, with dv the rows dqkv + n*ldq + voff (the gradient w.r.t.
 * the v that came out of the addition, which passes to the projection's v
 * unchanged):
 *   ds[n, g] = (dv[n, g, :] . ve[ids[n], g, :]) * 3*sig(s)*(1 - sig(s));
 *   dve[ids[n], g, :] (+)= 3*sigmoid(s[n, g]) * dv[n, g, :];
 *   dwg[g, c] (+)= sum_n ds[n, g] * xn[n, c];   dxn[n, :nc] += ds[n, :] @ wg
 * (dxn [N, ldx] dtype, in place; dve, dwg fp32, overwritten unless
 * `accumulate`; deterministic as in gdb_embed_bwd).  ws:
 * gdb_ve_bwd_ws_bytes of scratch. */
gdb_status gdb_ve_bwd_ws_bytes(int32_t N, int32_t Hkv, int32_t nc, int32_t deterministic, size_t* ws_bytes);
gdb_status gdb_ve_bwd(int32_t N, int32_t Hkv, int32_t D, int32_t dtype, const void* dqkv, int32_t ldq, int32_t voff,
                      const int32_t* ids, const void* ve, int32_t V, const float* s_save, const void* xn, void* dxn,
                      int32_t ldx, const void* wg, int32_t nc, float* dve, float* dwg, int32_t accumulate,
                      int32_t deterministic, void* ws, void* stream);

/* ------------------------------------------------------------------------
 * Building blocks.  The calls above are compositions of these; they are
 * exported so each stage can be run and checked on its own.  Same
 * conventions (device pointers, caller-owned memory, async on `stream`).
 * ---------------------------------------------------------------------- */

/* Bandwidth reference: dst = src over `bytes` (a multiple of 16; the
 * buffers must not overlap), 16-byte non-temporal loads and stores.  The
 * memory-bound kernels (norms, cross-entropy, embedding, optimizer) are
 * compared against its rate as well as against the HBM's nominal peak. */
gdb_status gdb_stream_copy(size_t bytes, const void* src, void* dst, void* stream);

/* RMSNorm without affine over rows of x [N, C]: xn = x * r, r[n] = 1/sqrt(mean(x[n]^2) + eps)
 * (r float32 [N]).  RMSNorm with eps = 1e-6 is the norm before attention, before
 * the MLP, on q and k per head, and before the lm_head. */
gdb_status gdb_rmsnorm_fwd(int32_t N, int32_t C, int32_t dtype, float eps, const void* x, void* xn,
                           float* r, void* stream);
/* dx = r * (dxn - xn * mean(dxn * xn)) + dres   (dres may be NULL or alias dx). */
gdb_status gdb_rmsnorm_bwd(int32_t N, int32_t C, int32_t dtype, const void* dxn, const void* xn,
                           const float* r, const void* dres, void* dx, void* stream);

/* GEMM C[m, n] = sum_k A(m, k) B(n, k) with fp32 accumulation (bf16 dtype: MFMA).
 *   A(m, k) = a_kmajor ? A[m*lda + k] : A[k*lda + m];  B(n, k) likewise with ldb.
 *   epi 0: C = acc;  1: C = R + acc;  2: C = acc and C2 = relu(acc)^2;
 *   3: C = acc * 2*max(R, 0);  6: C = relu(acc)^2;  7: C = acc * 2*sqrt(max(R, 0))
 *   (R = relu(u)^2 saved by epi 6, so 2*sqrt(R) = 2*relu(u), the ReLU^2
 *   derivative; the block keeps h only and uses 6 and 7);
 *   (C, C2, R in dtype, leading dims ldc, ldr; bf16 epi 6 needs both operands
 *   K-major and epi 7 A K-major, else GDB_EUNSUPPORTED; 5 is not accepted)
 *   4: C float32 [M, N] with ldc == N, C = acc or C += acc (accumulate); needs
 *      gdb_gemm_ws_bytes of workspace for the split-K partial sums.
 * The bias-free Linear y = x W^T of section "3. Gestion de la précision" is
 * A = x (K-major), B = W [out, in] (K-major). M, N, K, lda, ldb, ldc, ldr must be
 * multiples of 8 except M (tokens) when A is K-major and K when A is M-major. */
gdb_status gdb_gemm_ws_bytes(int32_t dtype, int32_t M, int32_t N, int32_t K, int32_t epi, size_t* ws_bytes);
gdb_status gdb_gemm(int32_t dtype, int32_t M, int32_t N, int32_t K, const void* A, int32_t a_kmajor,
                    int32_t lda, const void* B, int32_t b_kmajor, int32_t ldb, int32_t epi, void* C,
                    int32_t ldc, const void* R, int32_t ldr, void* C2, int32_t accumulate, void* ws,
                    void* stream);

/* fp8 operands ("Comment Entraîner Votre Propre ChatGPT Pour 50€ ?",
 * section "1. Le modèle GPT": the largest model runs most matrix products in
 * fp8).  Per-tensor dynamic scaling of x [R, Cc] (dtype):
 *   amax = max |x| (float32, written to the device scalar *amax),
 *   s = amax / 448 and code = e4m3(x / s), both float32 operations, round to
 *   nearest even, saturating at 448 (OCP e4m3fn; amax = 0 gives all-zero codes).
 * xq [R, Cc] receives the codes row-major, xqt [Cc, Rp] their transpose with
 * columns R..Rp-1 zero (Rp a multiple of 16, >= R); either may be NULL.
 * Cc must be a multiple of 16.  With mlp_fp8 the block quantises xn2, h,
 * w_fc, w_proj and the gradients dx_out and du this way. */
gdb_status gdb_fp8_quantize(int32_t R, int32_t Cc, int32_t dtype, const void* x, float* amax,
                            uint8_t* xq, uint8_t* xqt, int32_t Rp, void* stream);

/* GEMM on e4m3 codes, both operands K-contiguous:
 *   C[m, n] = s_a s_b sum_k A[m*lda + k] B[n*ldb + k],  s = amax / 448 of each operand,
 * with fp32 accumulation (v_mfma_f32_32x32x64_f8f6f4) and the epilogues of
 * gdb_gemm: epi 0-3, 6 and 7 with C, C2 and R in `dtype`; epi 4 fp32 C (needs
 * gdb_gemm_fp8_ws_bytes of workspace).  K, lda, ldb multiples of 16. */
gdb_status gdb_gemm_fp8_ws_bytes(int32_t M, int32_t N, int32_t K, int32_t epi, size_t* ws_bytes);
gdb_status gdb_gemm_fp8(int32_t dtype, int32_t M, int32_t N, int32_t K, const uint8_t* A, int32_t lda,
                        const float* amax_a, const uint8_t* B, int32_t ldb, const float* amax_b, int32_t epi,
                        void* C, int32_t ldc, const void* R, int32_t ldr, void* C2, int32_t accumulate,
                        void* ws, void* stream);

/* QK RMS-norm + RoPE on rows of qkv [B*T, (H + 2*Hkv)*D] (q heads, k heads, v heads):
 * out rows hold rope(rms_D(q_h)), rope(rms_D(k_g)) and v copied; rinv float32
 * [B*T, H + Hkv] receives the inverse RMS of each q and k head.  out != qkv. */
gdb_status gdb_qk_norm_rope_fwd(int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t D, int32_t dtype,
                                float eps, const void* qkv, void* out, float* rinv, const float* rope_tab,
                                void* stream);
/* Backward, in place on d [B*T, (H + 2*Hkv)*D]: the q/k parts of d (gradients
 * w.r.t. the rotated, normalised heads) become gradients w.r.t. the raw q/k;
 * the v part is left as is.  qkvh: the forward's output, rinv its factors. */
gdb_status gdb_qk_norm_rope_bwd(int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t D, int32_t dtype,
                                void* d, const void* qkvh, const float* rinv, const float* rope_tab,
                                void* stream);

/* Attention forward on rows of qkv [B*T, ld] holding q heads at column h*D,
 * k heads at (H + g)*D and v heads at (H + Hkv + g)*D:
 *   o[n, h*D + d] = sum_j P_ij v_j[d],  P = softmax over visible j of q.k / sqrt(D);
 *   lse float32 [B, H, T] = log-sum-exp of each row of scaled scores.
 * window as in gdb_block_cfg.  bf16: D = 128 only.
 * qk_normed != 0 promises that every q and k head vector has RMS <= 1 (the
 * output of the QK RMS-norm, as in gdb_block_fwd); then |score| <= sqrt(D)
 * and the kernel uses that fixed softmax offset instead of a running max.
 * With larger vectors and qk_normed != 0 the result is undefined.
 * bf16: one sequence's qkv rows must span under 2 GiB (T * ld * 2 bytes),
 * else GDB_EUNSUPPORTED. */
gdb_status gdb_attention_fwd(int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t D, int32_t window,
                             int32_t qk_normed, int32_t dtype, const void* qkv, int32_t ld, void* o,
                             int32_t ldo, float* lse, void* stream);
/* Attention backward: from dO [B*T, lddo] writes dq, dk, dv into dqkv [B*T, lddq]
 * at the same column offsets as qkv (dk, dv summed over the query heads that
 * share a K/V head). delta: float32 scratch [B, H, T].  bf16: one sequence's
 * qkv rows and dO rows must each span under 2 GiB (T * ld * 2 and
 * T * lddo * 2 bytes), else GDB_EUNSUPPORTED. */
gdb_status gdb_attention_bwd(int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t D, int32_t window,
                             int32_t dtype, const void* qkv, int32_t ld, const void* o, int32_t ldo,
                             const float* lse, const void* dout, int32_t lddo, void* dqkv, int32_t lddq,
                             float* delta, void* stream);

/* Decode attention against a key/value cache ("Comment Entraîner Votre
 * Propre ChatGPT Pour 50€ ?", section "6. Moteur d'inférence": generation
 * after the prompt is prefilled into a KV cache; the masking rule is the
 * training attention's, section "5. Unification de Flash Attention").
 * One new query per sequence b, at position i = lens[b] - 1:
 *   o[b, h*D + d] = sum_j P_j v_j[d],  P = softmax over visible j of q.k_j / sqrt(D),
 *   key j visible iff j <= i and (window < 0 or i - j <= window),
 *   query head h reads K/V head g = h / (H / Hkv);
 *   lse float32 [B, H] (optional, may be NULL) = log-sum-exp of the scores.
 * q: row b at q + b*ldq holds the H query heads (column h*D); the query's own
 *   key and value must already be in the cache at position i.
 * k, v: key / value of position j of sequence b at (k|v) + b*bstride + j*ldk,
 *   head g at column g*D (elements of `dtype`); a dedicated cache
 *   [B][Tmax][Hkv][D] has ldk = Hkv*D, bstride = Tmax*Hkv*D, and the packed
 *   QKV rows of a prefill serve as well (ldk = (H + 2*Hkv)*D, bstride = T*ldk,
 *   k and v offset by H*D and (H + Hkv)*D).
 * lens: DEVICE int32 [B], each in [1, max_len]; values outside are clamped
 *   to [0, max_len] and a length of 0 gives o = 0, lse = -inf.
 * max_len (host): bound on every length; it sizes the split-KV grid.
 * ws: fp32 scratch of gdb_attention_decode_ws_bytes bytes (NULL if that is 0).
 * D = 64 or 128 (bf16 and fp32); H / Hkv in {1, 2, 3, 4, 6, 8}. */
gdb_status gdb_attention_decode_ws_bytes(int32_t B, int32_t H, int32_t Hkv, int32_t D, int32_t max_len,
                                         int32_t window, size_t* ws_bytes);
gdb_status gdb_attention_decode(int32_t B, int32_t H, int32_t Hkv, int32_t D, int32_t window, int32_t dtype,
                                const void* q, int32_t ldq, const void* k, const void* v, int32_t ldk,
                                int64_t bstride, const int32_t* lens, int32_t max_len, void* o, int32_t ldo,
                                float* lse, void* ws, size_t ws_bytes, void* stream);

/* gdb_attention_decode without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, result and validation as
 * gdb_attention_decode; the split-KV partials go to a fixed device array
 * inside the library (16 MiB per GPU, held until the process ends; every
 * split plan fits in it, and a larger need returns GDB_EWORKSPACE).  The
 * call allocates nothing.  All calls on one GPU share that array: calls that
 * overlap on one GPU (concurrent streams or threads) race and must not be
 * issued. */
gdb_status gdb_attention_decode_noalloc(int32_t B, int32_t H, int32_t Hkv, int32_t D, int32_t window, int32_t dtype,
                                        const void* q, int32_t ldq, const void* k, const void* v, int32_t ldk,
                                        int64_t bstride, const int32_t* lens, int32_t max_len, void* o,
                                        int32_t ldo, float* lse, void* stream);

/* Optimizer step after the backward (the Japanese and French articles,
 * section 2 on the Muon optimizer): AdamW for embeddings, lm_head and scalar
 * parameters; Muon for matrices, i.e. momentum orthogonalised by the Polar
 * Express Newton-Schulz loop, one (a, b, c) triple per iteration:
 *   A = X^T X;  B = b*A + c*A@A;  X = a*X + X@B,
 * starting from X0 = G / (||G||_F * norm_scale + eps).  The coefficient table
 * is the caller's (the pages print two of its five triples).  The products
 * run on the MFMA GEMM in `dtype` (bf16: bf16 operands and results, fp32
 * accumulation; fp32: all fp32); a wide matrix (m < n) takes the Gram on the
 * other side, X X^T (the same map).
 *
 * Both calls take a stack of `count` matrices of the same shape, stored one
 * after the other ([count][m][n]); each item is normalised and iterated on
 * its own, and the stack's products run as one batched launch (at d24 the
 * 24 layers' matrices of one shape fill the GPU where one 1536 x 1536
 * product does not).
 *
 * gdb_newton_schulz: G float32 [count][m][n] -> X [count][m][n] in `dtype`
 *   (X != G).  coeffs: HOST float [steps][3]; m, n multiples of 8; steps in
 *   [0, 64]; count in [1, 65535].  ws: gdb_newton_schulz_ws_bytes bytes. */
gdb_status gdb_newton_schulz_ws_bytes(int32_t count, int32_t m, int32_t n, int32_t dtype, size_t* ws_bytes);
gdb_status gdb_newton_schulz(int32_t count, int32_t m, int32_t n, int32_t dtype, const float* G, void* X,
                             const float* coeffs, int32_t steps, float norm_scale, float eps, void* ws,
                             size_t ws_bytes, void* stream);
/* gdb_muon_step on matrix parameters p float32 [count][m][n] with gradients g
 * and momentum buffers buf (float32, updated in place), per item:
 *   buf = momentum*buf + g;  U = nesterov ? g + momentum*buf : buf;
 *   p = p*(1 - lr*wd) - lr*scale*NS(U)
 * (the momentum form, decay and the shape scale are inputs: the pages name
 * Muon only as momentum orthogonalised by Newton-Schulz).  p_bf16 (optional,
 * NULL to skip) receives the bf16 rounding of the new p.
 * ws: gdb_muon_ws_bytes bytes. */
gdb_status gdb_muon_ws_bytes(int32_t count, int32_t m, int32_t n, int32_t dtype, size_t* ws_bytes);
gdb_status gdb_muon_step(int32_t count, int32_t m, int32_t n, int32_t dtype, float* p, void* p_bf16, const float* g,
                         float* buf, float lr, float momentum, int32_t nesterov, float wd, float scale,
                         const float* coeffs, int32_t steps, float norm_scale, float eps, void* ws, size_t ws_bytes,
                         void* stream);
/* gdb_normuon_step: Muon with the NorMuon variance normalisation the
 * pages print in part (section "2. L'optimiseur Muon", "Réduction de la
 * variance NorMuon": the orthogonalised update is normalised per neuron to
 * avoid a collapse of its scale).  Per item, with O = NS(U) from Muon's
 * momentum step above and r the rows of O (one output neuron each):
 *   v_mean[r] = mean_j O[r, j]^2;          v_norm = sqrt(sum_r v_mean[r]);
 *   v[r] = beta2*v[r] + (1 - beta2)*v_mean[r]   (v: fp32 state [count][m]);
 *   step[r] = 1/sqrt(max(v[r], 1e-10));
 *   v_norm_new = sqrt(sum_r v_mean[r]*step[r]^2);
 *   final[r] = step[r] * v_norm / max(v_norm_new, 1e-10);
 *   p = p*(1 - lr*wd) - lr*scale*final[r]*O[r, :]
 * (the update keeps O's Frobenius norm and equalises its rows' RMS as far
 * as v tracks them).  Sums over rows are in a fixed order.  ws:
 * gdb_normuon_ws_bytes bytes. */
gdb_status gdb_normuon_ws_bytes(int32_t count, int32_t m, int32_t n, int32_t dtype, size_t* ws_bytes);
gdb_status gdb_normuon_step(int32_t count, int32_t m, int32_t n, int32_t dtype, float* p, void* p_bf16,
                            const float* g, float* buf, float* v, float lr, float momentum, int32_t nesterov,
                            float wd, float scale, float beta2, const float* coeffs, int32_t steps,
                            float norm_scale, float eps, void* ws, size_t ws_bytes, void* stream);
/* gdb_adamw_step on n float32 parameters (n a multiple of 8), step t >= 1:
 *   p *= 1 - lr*wd;  m = b1*m + (1-b1)*g;  v = b2*v + (1-b2)*g^2;
 *   p -= lr * (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)
 * (decoupled weight decay with bias correction).  p_bf16 optional as above. */
gdb_status gdb_adamw_step(int64_t n, float* p, void* p_bf16, const float* g, float* m, float* v, int32_t t, float lr,
                          float beta1, float beta2, float eps, float wd, void* stream);

/* Fused softmax cross-entropy on logits z [N, V] (overwritten by
 * dz = (softmax(z) - onehot(targets)) / N), row_loss float32 [N] =
 * logsumexp(z_n) - z_n[targets[n]], loss = mean(row_loss) (device scalar). */
gdb_status gdb_cross_entropy(int32_t N, int32_t V, int32_t dtype, void* z, const int32_t* targets,
                             float* row_loss, float* loss, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* GDB_H */
