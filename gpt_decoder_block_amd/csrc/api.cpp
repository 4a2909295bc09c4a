// C ABI of the decoder-block hot path: argument validation, layout of the
// caller-provided saved/workspace buffers, and the composition of the kernels
// into block forward, block backward and the fused lm_head + cross-entropy.
// Validation happens before any HIP call, so every argument error is
// reported without touching a device.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <initializer_list>
#include <stdlib.h>
#include <cmath>
#include <string>

#include "../../include/gdb.h"
#include "kernels.h"

using namespace gdb;

namespace {

thread_local std::string g_err;

gdb_status fail(gdb_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

#define HIPCHK(expr)                                                                    \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess) return fail(GDB_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

#define CHECK_PTR(p)                                                                       \
  do {                                                                                     \
    if ((p) == nullptr) return fail(GDB_EINVAL, "%s is NULL", #p);                         \
    if (((uintptr_t)(p)) & 15) return fail(GDB_EINVAL, "%s is not 16-byte aligned", #p);  \
  } while (0)

// Debug check of the outputs (GDB_CHECK_FINITE in the environment, read on
// every call): the first output holding a NaN or an infinity is named in the
// error.  Off, it only clears the error text, as every successful call does.
struct Output {
  int dt;
  const void* p;
  size_t n;
  const char* name;
};
bool check_finite_on() {
  const char* e = getenv("GDB_CHECK_FINITE");
  return e && *e && strcmp(e, "0") != 0;
}
gdb_status finished(std::initializer_list<Output> outs, hipStream_t s) {
  if (check_finite_on()) {
    for (const Output& o : outs) {
      bool bad = false;
      HIPCHK(any_nonfinite(o.dt, o.p, o.n, s, &bad));
      if (bad) return fail(GDB_ENONFINITE, "%s holds NaN or Inf (GDB_CHECK_FINITE)", o.name);
    }
  }
  g_err.clear();
  return GDB_OK;
}

// Sequential carving of a caller buffer into 256-byte aligned pieces; with a
// NULL base it only measures.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <typename T>
  T* take(size_t bytes) {
    off = (off + 255) & ~(size_t)255;
    T* p = base ? (T*)(base + off) : nullptr;
    off += bytes;
    return p;
  }
};

struct BlockDims {
  int B, T, N, C, H, Hkv, D, Q, KV, W3, F, window, dt, s;
  float eps;
  bool fp8;   // MLP GEMMs on e4m3 codes
  bool det;   // deterministic backward (fixed-order value-embedding table gradient)
  int Np;     // N rounded up to 16: K of the fp8 weight-gradient GEMMs
};

// Largest value-embedding gate width (one lane per channel).
constexpr int MAX_VE_GATE = 64;

gdb_status check_cfg(const gdb_block_cfg* c, BlockDims* d) {
  if (!c) return fail(GDB_EINVAL, "cfg is NULL");
  if (c->B <= 0 || c->T <= 0 || c->C <= 0) return fail(GDB_EINVAL, "B, T, C must be positive (got %d, %d, %d)", c->B, c->T, c->C);
  if (c->dtype != GDB_F32 && c->dtype != GDB_BF16) return fail(GDB_EINVAL, "unknown dtype %d", c->dtype);
  if (c->n_head <= 0 || c->n_kv_head <= 0) return fail(GDB_EINVAL, "n_head and n_kv_head must be positive");
  if (c->n_head % c->n_kv_head != 0) return fail(GDB_EINVAL, "n_head (%d) must be a multiple of n_kv_head (%d)", c->n_head, c->n_kv_head);
  if (c->head_dim != 64 && c->head_dim != 128) return fail(GDB_EUNSUPPORTED, "head_dim %d not supported (64 or 128)", c->head_dim);
  if (c->dtype == GDB_BF16 && c->head_dim != 128) return fail(GDB_EUNSUPPORTED, "bf16 attention needs head_dim 128 (got %d)", c->head_dim);
  if (c->n_head * c->head_dim != c->C) return fail(GDB_EUNSUPPORTED, "n_head*head_dim (%d) must equal C (%d)", c->n_head * c->head_dim, c->C);
  if (c->C % 8 || c->mlp_hidden <= 0 || c->mlp_hidden % 8) return fail(GDB_EINVAL, "C and mlp_hidden must be positive multiples of 8");
  if (c->window < -1) return fail(GDB_EINVAL, "window must be >= -1 (got %d)", c->window);
  if (c->mlp_fp8 && (c->C % 16 || c->mlp_hidden % 16)) return fail(GDB_EINVAL, "mlp_fp8 needs C and mlp_hidden multiples of 16");
  if (!(c->eps > 0.f) || !std::isfinite(c->eps)) return fail(GDB_EINVAL, "eps must be positive and finite");
  if (c->deterministic != 0 && c->deterministic != 1) return fail(GDB_EINVAL, "deterministic must be 0 or 1");
  if ((long long)c->B * c->T > (1LL << 30)) return fail(GDB_EINVAL, "B*T too large");
  d->B = c->B; d->T = c->T; d->N = c->B * c->T; d->C = c->C;
  d->H = c->n_head; d->Hkv = c->n_kv_head; d->D = c->head_dim;
  d->Q = d->H * d->D; d->KV = d->Hkv * d->D; d->W3 = d->Q + 2 * d->KV;
  d->F = c->mlp_hidden; d->window = c->window >= c->T - 1 ? -1 : c->window;
  d->dt = c->dtype; d->s = dt_size(c->dtype); d->eps = c->eps;
  d->fp8 = c->mlp_fp8 != 0;
  d->det = c->deterministic != 0;
  d->Np = (d->N + 15) / 16 * 16;
  return GDB_OK;
}

struct Saved {
  void *xn1, *qkvh, *o, *xn2, *h;
  float *r1, *rqk, *lse, *r2;
  float* ve_s;          // value-embedding gate logits [N, Hkv]
  // fp8 MLP: transposed codes for the backward and the four amax values
  uint8_t *xn2T, *hT, *wfcT, *wprojT;   // [C, Np], [F, Np], [C, F], [F, C]
  float* amax;                          // xn2, w_fc, h, w_proj
};
struct WsFwd {
  void *qkv, *x_mid;
  void* x_mix;          // residual-mixed block input [N, C]
  uint8_t *xn2q, *wfcq, *hq, *wprojq;  // fp8 MLP codes, row-major
};
struct WsBwd {
  void *du, *dxn, *dx_mid, *dout, *dqkv;
  float *delta, *partial;
  float* ds;            // value-embedding gate logit gradients [N, Hkv]
  float* xpart;         // partial sums of the extras' parameter gradients
  uint8_t *doutq, *doutT, *duq, *duT;  // fp8 MLP backward codes: [N, C], [C, Np], [N, F], [F, Np]
  float* amax8;                        // dout, du
  void* wt;             // bf16: K-major copy of the weight of the current data-gradient product
  void* order;          // deterministic: token sort scratch (token_order)
};

void carve_saved(const BlockDims& d, Carver& c, Saved& s) {
  const size_t N = d.N;
  s.xn1 = c.take<char>(N * d.C * d.s);
  s.r1 = c.take<float>(N * 4);
  s.qkvh = c.take<char>(N * d.W3 * d.s);
  s.rqk = c.take<float>(N * (d.H + d.Hkv) * 4);
  s.o = c.take<char>(N * d.Q * d.s);
  s.lse = c.take<float>(N * d.H * 4);
  s.xn2 = c.take<char>(N * d.C * d.s);
  s.r2 = c.take<float>(N * 4);
  s.h = c.take<char>(N * d.F * d.s);
  s.ve_s = c.take<float>(N * d.Hkv * 4);
  const size_t f8 = d.fp8 ? 1 : 0, Np = d.Np;
  s.xn2T = c.take<uint8_t>(f8 * d.C * Np);
  s.hT = c.take<uint8_t>(f8 * d.F * Np);
  s.wfcT = c.take<uint8_t>(f8 * d.C * d.F);
  s.wprojT = c.take<uint8_t>(f8 * d.F * d.C);
  s.amax = c.take<float>(f8 * 4 * 4);
}
void carve_fwd(const BlockDims& d, Carver& c, WsFwd& w) {
  // raw q, k, v: only the fp32 path (bf16 normalises them in the GEMM epilogue)
  w.qkv = c.take<char>(d.dt == F32 ? (size_t)d.N * d.W3 * d.s : 0);
  w.x_mid = c.take<char>((size_t)d.N * d.C * d.s);
  w.x_mix = c.take<char>((size_t)d.N * d.C * d.s);
  const size_t f8 = d.fp8 ? 1 : 0, N = d.N;
  w.xn2q = c.take<uint8_t>(f8 * N * d.C);
  w.wfcq = c.take<uint8_t>(f8 * d.F * d.C);
  w.hq = c.take<uint8_t>(f8 * N * d.F);
  w.wprojq = c.take<uint8_t>(f8 * d.C * d.F);
}
size_t wgrad_partial_floats(const BlockDims& d) {
  size_t m = 0;
  const int shapes[4][2] = {{d.C, d.F}, {d.F, d.C}, {d.C, d.Q}, {d.W3, d.C}};
  for (auto& sh : shapes) {
    const SplitPlan pl = gemm_split_plan(d.dt, sh[0], sh[1], d.N);
    if (pl.splits > 1 || pl.splits2 > 0) m = std::max(m, (size_t)plan_slices(pl) * sh[0] * sh[1]);
    if (d.fp8) {
      const SplitPlan p8 = gemm_split_plan(FP8, sh[0], sh[1], d.Np);
      if (p8.splits > 1 || p8.splits2 > 0) m = std::max(m, (size_t)plan_slices(p8) * sh[0] * sh[1]);
    }
  }
  return m;
}
void carve_bwd(const BlockDims& d, Carver& c, WsBwd& w) {
  const size_t N = d.N;
  w.du = c.take<char>(N * d.F * d.s);
  w.dxn = c.take<char>(N * d.C * d.s);
  w.dx_mid = c.take<char>(N * d.C * d.s);
  w.dout = c.take<char>(N * d.Q * d.s);
  w.dqkv = c.take<char>(N * d.W3 * d.s);
  w.delta = c.take<float>(N * d.H * 4);
  w.partial = c.take<float>(wgrad_partial_floats(d) * 4);
  w.ds = c.take<float>(N * d.Hkv * 4);
  const size_t xp = std::max((size_t)mix_partials(d.N) * 2, (size_t)ve_gate_partials(d.N) * d.Hkv * MAX_VE_GATE);
  w.xpart = c.take<float>(xp * 4);
  const size_t f8 = d.fp8 ? 1 : 0, Np = d.Np;
  w.wt = c.take<char>(d.dt == BF16 ? (size_t)std::max(std::max(d.W3, d.F), d.Q) * d.C * 2 : 0);
  w.doutq = c.take<uint8_t>(f8 * N * d.C);
  w.doutT = c.take<uint8_t>(f8 * d.C * Np);
  w.duq = c.take<uint8_t>(f8 * N * d.F);
  w.duT = c.take<uint8_t>(f8 * d.F * Np);
  w.amax8 = c.take<float>(f8 * 2 * 4);
  w.order = c.take<char>(d.det ? token_order_ws_bytes(d.N) : 0);
}

// Which extras a call uses; validates their pointers and sizes.
struct Extras {
  bool mix = false, ve = false;
};
gdb_status check_extras(const BlockDims& d, const gdb_block_extras* ex, bool bwd, Extras* e) {
  *e = Extras{};
  if (!ex) return GDB_OK;
  if (ex->lambdas) {
    e->mix = true;
    if (((uintptr_t)ex->lambdas) & 3) return fail(GDB_EINVAL, "ex->lambdas is not 4-byte aligned");
    CHECK_PTR(ex->x0);
    if (bwd) CHECK_PTR(ex->x_in);
  }
  if (ex->ve) {
    e->ve = true;
    CHECK_PTR(ex->ve);
    CHECK_PTR(ex->ve_gate);
    if (!ex->ids || (((uintptr_t)ex->ids) & 3)) return fail(GDB_EINVAL, "ex->ids is NULL or not 4-byte aligned");
    if (ex->ve_vocab <= 0) return fail(GDB_EINVAL, "ex->ve_vocab must be positive (got %d)", ex->ve_vocab);
    if (ex->ve_gate_channels < 1 || ex->ve_gate_channels > MAX_VE_GATE || ex->ve_gate_channels > d.C)
      return fail(GDB_EINVAL, "ex->ve_gate_channels must be in [1, min(%d, C)] (got %d)", MAX_VE_GATE,
                  ex->ve_gate_channels);
    if (d.Hkv > 64) return fail(GDB_EUNSUPPORTED, "value embeddings need n_kv_head <= 64 (got %d)", d.Hkv);
  }
  return GDB_OK;
}

GemmArgs gemm_args(const void* A, bool ak, int lda, const void* B, bool bk, int ldb, int M, int N, int K,
                   int epi, void* C, int ldc) {
  GemmArgs g{};
  g.A = A; g.B = B; g.M = M; g.N = N; g.K = K; g.lda = lda; g.ldb = ldb;
  g.a_kmajor = ak; g.b_kmajor = bk; g.epi = epi; g.C = C; g.ldc = ldc;
  g.splits = 1;
  return g;
}

// fp32 weight gradient C[M, N] (+)= sum_k A[k, m] B[k, n] (A, B token-major)
hipError_t wgrad(int dt, const void* A, int lda, const void* B, int ldb, int M, int N, int K, float* C,
                 int accumulate, float* partial, hipStream_t s) {
  GemmArgs g = gemm_args(A, false, lda, B, false, ldb, M, N, K, EPI_F32, C, N);
  g.accumulate = accumulate;
  const SplitPlan pl = gemm_split_plan(dt, M, N, K);
  g.splits = pl.splits;
  g.split_cols = pl.split_cols; g.first1 = pl.first1; g.splits2 = pl.splits2;
  g.partial = partial;
  hipError_t e = gemm(dt, g, s);
  if (e != hipSuccess || (g.splits == 1 && g.splits2 == 0)) return e;
  if (g.splits2 > 0)
    return splitk_reduce2(partial, C, M, N, g.splits, g.split_cols, g.first1, g.splits2, accumulate, s);
  return splitk_reduce(partial, C, g.splits, (size_t)M * N, accumulate, s);
}

// fp32 weight gradient from fp8 codes: C[M, N] (+)= s_a s_b sum_k A[m, k] B[n, k]
// (A [M, K], B [N, K] row-major codes, K the padded token count)
hipError_t wgrad_fp8(const uint8_t* A, const float* amax_a, const uint8_t* B, const float* amax_b, int M, int N,
                     int K, float* C, int accumulate, float* partial, hipStream_t s) {
  GemmArgs g = gemm_args(A, true, K, B, true, K, M, N, K, EPI_F32, C, N);
  g.accumulate = accumulate;
  const SplitPlan pl = gemm_split_plan(FP8, M, N, K);
  g.splits = pl.splits;
  g.split_cols = pl.split_cols; g.first1 = pl.first1; g.splits2 = pl.splits2;
  g.partial = partial;
  g.amax_a = amax_a; g.amax_b = amax_b;
  hipError_t e = gemm_fp8(BF16, g, s);  // fp32 output: the element type of C is fixed
  if (e != hipSuccess || (g.splits == 1 && g.splits2 == 0)) return e;
  if (g.splits2 > 0)
    return splitk_reduce2(partial, C, M, N, g.splits, g.split_cols, g.first1, g.splits2, accumulate, s);
  return splitk_reduce(partial, C, g.splits, (size_t)M * N, accumulate, s);
}

}  // namespace

extern "C" {

int32_t gdb_abi_version(void) { return GDB_ABI_VERSION; }

const char* gdb_last_error(void) { return g_err.c_str(); }

gdb_status gdb_block_sizes(const gdb_block_cfg* cfg, size_t* saved_bytes, size_t* ws_fwd_bytes,
                           size_t* ws_bwd_bytes) {
  BlockDims d;
  gdb_status st = check_cfg(cfg, &d);
  if (st != GDB_OK) return st;
  Saved sv;
  WsFwd wf;
  WsBwd wb;
  Carver c1(nullptr), c2(nullptr), c3(nullptr);
  carve_saved(d, c1, sv);
  carve_fwd(d, c2, wf);
  carve_bwd(d, c3, wb);
  if (saved_bytes) *saved_bytes = c1.off;
  if (ws_fwd_bytes) *ws_fwd_bytes = c2.off;
  if (ws_bwd_bytes) *ws_bwd_bytes = c3.off;
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_rope_table_host(int32_t T, int32_t head_dim, double base, float* out_host) {
  if (T <= 0 || head_dim <= 0 || head_dim % 2) return fail(GDB_EINVAL, "T and head_dim must be positive, head_dim even");
  if (!(base > 1.0)) return fail(GDB_EINVAL, "rope base must be > 1");
  if (!out_host) return fail(GDB_EINVAL, "out_host is NULL");
  const int hd = head_dim / 2;
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < hd; ++j) {
      const double th = (double)t * std::pow(base, -2.0 * j / head_dim);
      out_host[((size_t)t * hd + j) * 2] = (float)std::cos(th);
      out_host[((size_t)t * hd + j) * 2 + 1] = (float)std::sin(th);
    }
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_embed_fwd(int32_t N, int32_t C, int32_t V, int32_t dtype, const int32_t* ids, const void* wte,
                         void* x0, void* stream) {
  if (N < 0 || C <= 0 || V <= 0 || C % 8) return fail(GDB_EINVAL, "bad sizes N=%d C=%d V=%d (C multiple of 8)", N, C, V);
  if (dtype != GDB_F32 && dtype != GDB_BF16) return fail(GDB_EINVAL, "unknown dtype %d", dtype);
  if (N == 0) { g_err.clear(); return GDB_OK; }
  CHECK_PTR(ids); CHECK_PTR(wte); CHECK_PTR(x0);
  HIPCHK(embed_fwd(dtype, ids, wte, x0, N, C, V, (hipStream_t)stream));
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_embed_bwd_ws_bytes(int32_t N, int32_t deterministic, size_t* ws_bytes) {
  if (N < 0) return fail(GDB_EINVAL, "N must be >= 0");
  if (!ws_bytes) return fail(GDB_EINVAL, "ws_bytes is NULL");
  *ws_bytes = deterministic ? token_order_ws_bytes(N) : 0;
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_embed_bwd(int32_t N, int32_t C, int32_t V, int32_t dtype, const int32_t* ids, const void* dx0,
                         float* dwte, int32_t accumulate, int32_t deterministic, void* ws, void* stream) {
  if (N < 0 || C <= 0 || V <= 0 || C % 8) return fail(GDB_EINVAL, "bad sizes N=%d C=%d V=%d (C multiple of 8)", N, C, V);
  if (dtype != GDB_F32 && dtype != GDB_BF16) return fail(GDB_EINVAL, "unknown dtype %d", dtype);
  CHECK_PTR(dwte);
  if (N > 0) { CHECK_PTR(ids); CHECK_PTR(dx0); }
  hipStream_t s = (hipStream_t)stream;
  if (deterministic && N > 0) {
    CHECK_PTR(ws);
    const int32_t *sk, *perm;
    HIPCHK(token_order(ids, N, V, ws, &sk, &perm, s));
    HIPCHK(rows_segsum(dtype, sk, perm, N, dx0, C, 0, C, nullptr, 1, C, dwte, V, accumulate ? 1 : 0, s));
  } else {
    HIPCHK(embed_bwd(dtype, ids, dx0, dwte, N, C, V, accumulate, s));
  }
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_block_fwd(const gdb_block_cfg* cfg, const gdb_block_weights* w, const gdb_block_extras* ex,
                         const float* rope_tab, const void* x_in, void* x_out, void* saved, void* ws, void* stream) {
  BlockDims d;
  gdb_status st = check_cfg(cfg, &d);
  if (st != GDB_OK) return st;
  if (!w) return fail(GDB_EINVAL, "weights is NULL");
  CHECK_PTR(w->w_qkv); CHECK_PTR(w->w_o); CHECK_PTR(w->w_fc); CHECK_PTR(w->w_proj);
  CHECK_PTR(rope_tab); CHECK_PTR(x_in); CHECK_PTR(x_out); CHECK_PTR(saved); CHECK_PTR(ws);
  if (x_in == x_out) return fail(GDB_EINVAL, "x_out must not alias x_in");
  Extras xe;
  if ((st = check_extras(d, ex, false, &xe)) != GDB_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  Saved sv;
  WsFwd wf;
  Carver c1(saved), c2(ws);
  carve_saved(d, c1, sv);
  carve_fwd(d, c2, wf);
  const int dt = d.dt, N = d.N;

  const void* x = x_in;
  if (xe.mix) {
    HIPCHK(mix_fwd(dt, x_in, ex->x0, ex->lambdas, wf.x_mix, (size_t)N * d.C, s));
    x = wf.x_mix;
  }
  HIPCHK(rmsnorm_fwd(dt, x, sv.xn1, sv.r1, N, d.C, d.eps, s));
  if (dt == BF16) {
    // QKV projection with the QK RMS-norm and RoPE fused into its epilogue
    GemmArgs gq = gemm_args(sv.xn1, true, d.C, w->w_qkv, true, d.C, N, d.W3, d.C, EPI_QKNORM, sv.qkvh, d.W3);
    gq.rope = rope_tab; gq.rinv = sv.rqk; gq.T = d.T; gq.qk_heads = d.H + d.Hkv; gq.eps = d.eps;
    HIPCHK(gemm(dt, gq, s));
    if (xe.ve)
      HIPCHK(ve_fwd(dt, sv.qkvh, d.W3, d.Q + d.KV, sv.xn1, d.C, ex->ids, ex->ve, ex->ve_gate,
                    ex->ve_gate_channels, d.Hkv, d.D, ex->ve_vocab, sv.ve_s, N, s));
  } else {
    HIPCHK(gemm(dt, gemm_args(sv.xn1, true, d.C, w->w_qkv, true, d.C, N, d.W3, d.C, EPI_STORE, wf.qkv, d.W3), s));
    if (xe.ve)
      HIPCHK(ve_fwd(dt, wf.qkv, d.W3, d.Q + d.KV, sv.xn1, d.C, ex->ids, ex->ve, ex->ve_gate, ex->ve_gate_channels,
                    d.Hkv, d.D, ex->ve_vocab, sv.ve_s, N, s));
    HIPCHK(qk_norm_rope_fwd(dt, wf.qkv, sv.qkvh, sv.rqk, rope_tab, d.B, d.T, d.H, d.Hkv, d.D, d.eps, s));
  }
  AttnArgs at{};
  at.B = d.B; at.T = d.T; at.H = d.H; at.Hkv = d.Hkv; at.D = d.D; at.window = d.window;
  at.qk_normed = 1;  // q^, k^ come out of the QK RMS-norm
  at.qkv = sv.qkvh; at.ld = d.W3; at.o = sv.o; at.ldo = d.Q; at.lse = sv.lse;
  HIPCHK(attn_fwd(dt, at, s));
  GemmArgs g = gemm_args(sv.o, true, d.Q, w->w_o, true, d.Q, N, d.C, d.Q, EPI_RESID, wf.x_mid, d.C);
  g.R = x; g.ldr = d.C;
  HIPCHK(gemm(dt, g, s));
  if (d.fp8) {
    // e4m3 codes of both operands of each MLP product (row-major for the
    // forward, transposed copies kept for the backward), per-tensor scales;
    // the amax of xn2 and h comes from the kernels that write them; the four
    // accumulators are zeroed together
    HIPCHK(fp8_amax_zero(sv.amax, s, 4));
    HIPCHK(rmsnorm_fwd(dt, wf.x_mid, sv.xn2, sv.r2, N, d.C, d.eps, s, sv.amax + 0));
    HIPCHK(fp8_quant(dt, sv.xn2, N, d.C, sv.amax + 0, wf.xn2q, sv.xn2T, d.Np, s));
    HIPCHK(fp8_amax(dt, w->w_fc, (size_t)d.F * d.C, sv.amax + 1, s, false));
    HIPCHK(fp8_quant(dt, w->w_fc, d.F, d.C, sv.amax + 1, wf.wfcq, sv.wfcT, d.F, s));
    g = gemm_args(wf.xn2q, true, d.C, wf.wfcq, true, d.C, N, d.F, d.C, EPI_SQR, sv.h, d.F);
    g.amax_a = sv.amax + 0; g.amax_b = sv.amax + 1;
    g.amax_out = sv.amax + 2;
    HIPCHK(gemm_fp8(dt, g, s));
    HIPCHK(fp8_quant(dt, sv.h, N, d.F, sv.amax + 2, wf.hq, sv.hT, d.Np, s));
    HIPCHK(fp8_amax(dt, w->w_proj, (size_t)d.C * d.F, sv.amax + 3, s, false));
    HIPCHK(fp8_quant(dt, w->w_proj, d.C, d.F, sv.amax + 3, wf.wprojq, sv.wprojT, d.C, s));
    g = gemm_args(wf.hq, true, d.F, wf.wprojq, true, d.F, N, d.C, d.F, EPI_RESID, x_out, d.C);
    g.R = wf.x_mid; g.ldr = d.C; g.amax_a = sv.amax + 2; g.amax_b = sv.amax + 3;
    HIPCHK(gemm_fp8(dt, g, s));
    return finished({{dt, x_out, (size_t)N * d.C, "x_out"}}, s);
  }
  HIPCHK(rmsnorm_fwd(dt, wf.x_mid, sv.xn2, sv.r2, N, d.C, d.eps, s));
  // only h = relu(u)^2 is kept: the backward's ReLU^2 derivative 2*relu(u) is 2*sqrt(h)
  g = gemm_args(sv.xn2, true, d.C, w->w_fc, true, d.C, N, d.F, d.C, EPI_SQR, sv.h, d.F);
  HIPCHK(gemm(dt, g, s));
  g = gemm_args(sv.h, true, d.F, w->w_proj, true, d.F, N, d.C, d.F, EPI_RESID, x_out, d.C);
  g.R = wf.x_mid; g.ldr = d.C;
  HIPCHK(gemm(dt, g, s));
  return finished({{dt, x_out, (size_t)N * d.C, "x_out"}}, s);
}

// Data gradient dX [N, Nn] = dY [N, K] . W [K, Nn] (W row-major, the layout of
// the forward's K-major weight).  In bf16 W is first copied transposed into
// wt, so the product runs with both operands K-major, the GEMM's fastest
// layout (the copy costs a few percent of the product); fp32 reads W as is.
static GemmArgs dgrad_args(int dt, const void* dY, int K, const void* W, int Nn, int N, int epi, void* dX, void* wt,
                           hipStream_t s, hipError_t* err) {
  *err = hipSuccess;
  if (dt == BF16) {
    *err = transpose_bf16(W, K, Nn, wt, s);
    return gemm_args(dY, true, K, wt, true, K, N, Nn, K, epi, dX, Nn);
  }
  return gemm_args(dY, true, K, W, false, Nn, N, Nn, K, epi, dX, Nn);
}

gdb_status gdb_block_bwd(const gdb_block_cfg* cfg, const gdb_block_weights* w, const gdb_block_extras* ex,
                         const float* rope_tab, const void* saved, const void* dx_out, void* dx_in,
                         const gdb_block_wgrads* dw, const gdb_block_extras_grads* dex, void* ws, void* stream) {
  BlockDims d;
  gdb_status st = check_cfg(cfg, &d);
  if (st != GDB_OK) return st;
  if (!w || !dw) return fail(GDB_EINVAL, "weights or wgrads is NULL");
  CHECK_PTR(w->w_qkv); CHECK_PTR(w->w_o); CHECK_PTR(w->w_fc); CHECK_PTR(w->w_proj);
  CHECK_PTR(dw->dw_qkv); CHECK_PTR(dw->dw_o); CHECK_PTR(dw->dw_fc); CHECK_PTR(dw->dw_proj);
  CHECK_PTR(rope_tab); CHECK_PTR(saved); CHECK_PTR(dx_out); CHECK_PTR(dx_in); CHECK_PTR(ws);
  Extras xe;
  if ((st = check_extras(d, ex, true, &xe)) != GDB_OK) return st;
  if (xe.mix || xe.ve) {
    if (!dex) return fail(GDB_EINVAL, "extras given without extras gradients");
    if (xe.mix) {
      if (!dex->dlambdas || (((uintptr_t)dex->dlambdas) & 3)) return fail(GDB_EINVAL, "dex->dlambdas is NULL or misaligned");
      CHECK_PTR(dex->dx0);
    }
    if (xe.ve) { CHECK_PTR(dex->dve); CHECK_PTR(dex->dve_gate); }
  }
  hipStream_t s = (hipStream_t)stream;
  Saved sv;
  WsBwd wb;
  Carver c1((void*)saved), c2(ws);
  carve_saved(d, c1, sv);
  carve_bwd(d, c2, wb);
  const int dt = d.dt, N = d.N, acc = cfg->accumulate_wgrad ? 1 : 0;

  // MLP
  if (d.fp8) {
    // straight-through fp8: the same codes and scales as the forward for the
    // weights and saved activations, fresh ones for dout and du
    HIPCHK(fp8_amax_zero(wb.amax8, s, 2));
    HIPCHK(fp8_amax(dt, dx_out, (size_t)N * d.C, wb.amax8 + 0, s, false));
    HIPCHK(fp8_quant(dt, dx_out, N, d.C, wb.amax8 + 0, wb.doutq, wb.doutT, d.Np, s));
    // du's amax comes from the GEMM that writes it
    GemmArgs g = gemm_args(wb.doutq, true, d.C, sv.wprojT, true, d.C, N, d.F, d.C, EPI_DSQR, wb.du, d.F);
    g.R = sv.h; g.ldr = d.F; g.amax_a = wb.amax8 + 0; g.amax_b = sv.amax + 3;
    g.amax_out = wb.amax8 + 1;
    HIPCHK(gemm_fp8(dt, g, s));
    HIPCHK(wgrad_fp8(wb.doutT, wb.amax8 + 0, sv.hT, sv.amax + 2, d.C, d.F, d.Np, dw->dw_proj, acc, wb.partial, s));
    HIPCHK(fp8_quant(dt, wb.du, N, d.F, wb.amax8 + 1, wb.duq, wb.duT, d.Np, s));
    g = gemm_args(wb.duq, true, d.F, sv.wfcT, true, d.F, N, d.C, d.F, EPI_STORE, wb.dxn, d.C);
    g.amax_a = wb.amax8 + 1; g.amax_b = sv.amax + 1;
    HIPCHK(gemm_fp8(dt, g, s));
    HIPCHK(wgrad_fp8(wb.duT, wb.amax8 + 1, sv.xn2T, sv.amax + 0, d.F, d.C, d.Np, dw->dw_fc, acc, wb.partial, s));
  } else {
    hipError_t te;
    GemmArgs g = dgrad_args(dt, dx_out, d.C, w->w_proj, d.F, N, EPI_DSQR, wb.du, wb.wt, s, &te);
    HIPCHK(te);
    g.R = sv.h; g.ldr = d.F;
    HIPCHK(gemm(dt, g, s));
    HIPCHK(wgrad(dt, dx_out, d.C, sv.h, d.F, d.C, d.F, N, dw->dw_proj, acc, wb.partial, s));
    g = dgrad_args(dt, wb.du, d.F, w->w_fc, d.C, N, EPI_STORE, wb.dxn, wb.wt, s, &te);
    HIPCHK(te);
    HIPCHK(gemm(dt, g, s));
    HIPCHK(wgrad(dt, wb.du, d.F, sv.xn2, d.C, d.F, d.C, N, dw->dw_fc, acc, wb.partial, s));
  }
  HIPCHK(rmsnorm_bwd(dt, wb.dxn, sv.xn2, sv.r2, dx_out, wb.dx_mid, N, d.C, s));
  // attention output projection
  {
    hipError_t te;
    GemmArgs g = dgrad_args(dt, wb.dx_mid, d.C, w->w_o, d.Q, N, EPI_STORE, wb.dout, wb.wt, s, &te);
    HIPCHK(te);
    HIPCHK(gemm(dt, g, s));
  }
  HIPCHK(wgrad(dt, wb.dx_mid, d.C, sv.o, d.Q, d.C, d.Q, N, dw->dw_o, acc, wb.partial, s));
  // attention
  AttnArgs at{};
  at.B = d.B; at.T = d.T; at.H = d.H; at.Hkv = d.Hkv; at.D = d.D; at.window = d.window;
  at.qkv = sv.qkvh; at.ld = d.W3; at.o = sv.o; at.ldo = d.Q; at.lse = sv.lse;
  at.dout = wb.dout; at.lddo = d.Q; at.dqkv = wb.dqkv; at.lddq = d.W3; at.delta = wb.delta;
  if (dt == BF16) {
    // the QK RMS-norm and RoPE backward happen in the dQ and dK epilogues
    at.rope = rope_tab; at.rinv = sv.rqk;
    HIPCHK(attn_bwd(dt, at, s));
  } else {
    HIPCHK(attn_bwd(dt, at, s));
    HIPCHK(qk_norm_rope_bwd(dt, wb.dqkv, sv.qkvh, sv.rqk, rope_tab, d.B, d.T, d.H, d.Hkv, d.D, s));
  }
  // value embeddings: gate-logit gradients and the table's rows (dv passes through unchanged)
  if (xe.ve) {
    if (d.det) {
      // the table's rows add their tokens in token order (stable sort by id)
      const int32_t *sk, *perm;
      HIPCHK(ve_bwd(dt, wb.dqkv, d.W3, d.Q + d.KV, ex->ids, ex->ve, sv.ve_s, d.Hkv, d.D, ex->ve_vocab, wb.ds,
                    nullptr, N, s));
      HIPCHK(token_order(ex->ids, N, ex->ve_vocab, wb.order, &sk, &perm, s));
      HIPCHK(rows_segsum(dt, sk, perm, N, wb.dqkv, d.W3, d.Q + d.KV, d.KV, sv.ve_s, d.Hkv, d.D, dex->dve, ex->ve_vocab,
                         acc, s));
    } else {
      if (!acc) HIPCHK(fill_f32(dex->dve, (size_t)ex->ve_vocab * d.KV, 0.f, s));
      HIPCHK(ve_bwd(dt, wb.dqkv, d.W3, d.Q + d.KV, ex->ids, ex->ve, sv.ve_s, d.Hkv, d.D, ex->ve_vocab, wb.ds,
                    dex->dve, N, s));
    }
  }
  // QKV projection
  {
    hipError_t te;
    GemmArgs g = dgrad_args(dt, wb.dqkv, d.W3, w->w_qkv, d.C, N, EPI_STORE, wb.dxn, wb.wt, s, &te);
    HIPCHK(te);
    HIPCHK(gemm(dt, g, s));
  }
  HIPCHK(wgrad(dt, wb.dqkv, d.W3, sv.xn1, d.C, d.W3, d.C, N, dw->dw_qkv, acc, wb.partial, s));
  if (xe.ve)
    HIPCHK(ve_gate_bwd(dt, wb.ds, sv.xn1, wb.dxn, d.C, ex->ve_gate, ex->ve_gate_channels, d.Hkv, wb.xpart,
                       dex->dve_gate, acc, N, s));
  if (xe.mix) {
    HIPCHK(rmsnorm_bwd(dt, wb.dxn, sv.xn1, sv.r1, wb.dx_mid, wb.dx_mid, N, d.C, s));
    HIPCHK(mix_bwd(dt, wb.dx_mid, ex->x_in, ex->x0, ex->lambdas, dx_in, dex->dx0, dex->accumulate_dx0 ? 1 : 0,
                   wb.xpart, dex->dlambdas, acc, N, d.C, s));
  } else {
    HIPCHK(rmsnorm_bwd(dt, wb.dxn, sv.xn1, sv.r1, wb.dx_mid, dx_in, N, d.C, s));
  }
  return finished({{dt, dx_in, (size_t)N * d.C, "dx_in"},
                   {F32, dw->dw_qkv, (size_t)d.W3 * d.C, "dw_qkv"},
                   {F32, dw->dw_o, (size_t)d.C * d.Q, "dw_o"},
                   {F32, dw->dw_fc, (size_t)d.F * d.C, "dw_fc"},
                   {F32, dw->dw_proj, (size_t)d.C * d.F, "dw_proj"}},
                  s);
}

namespace {
struct HeadWs {
  void *xf, *z, *dxf;
  float *rf, *row_loss, *partial;
};
gdb_status check_head(int N, int C, int V, int dtype) {
  if (N <= 0 || C <= 0 || V <= 0) return fail(GDB_EINVAL, "N, C, V must be positive (got %d, %d, %d)", N, C, V);
  if (C % 8 || V % 8) return fail(GDB_EINVAL, "C and V must be multiples of 8");
  if (dtype != GDB_F32 && dtype != GDB_BF16) return fail(GDB_EINVAL, "unknown dtype %d", dtype);
  return GDB_OK;
}
void carve_head(int N, int C, int V, int dt, Carver& c, HeadWs& h) {
  const int s = dt_size(dt);
  h.xf = c.take<char>((size_t)N * C * s);
  h.rf = c.take<float>((size_t)N * 4);
  h.z = c.take<char>((size_t)N * V * s);
  h.row_loss = c.take<float>((size_t)N * 4);
  h.dxf = c.take<char>((size_t)N * C * s);
  const SplitPlan pl = gemm_split_plan(dt, V, C, N);
  h.partial = c.take<float>(pl.splits > 1 || pl.splits2 > 0 ? (size_t)plan_slices(pl) * V * C * 4 : 0);
}
}  // namespace

gdb_status gdb_lm_head_ce_sizes(int32_t N, int32_t C, int32_t V, int32_t dtype, size_t* ws_bytes) {
  gdb_status st = check_head(N, C, V, dtype);
  if (st != GDB_OK) return st;
  HeadWs h;
  Carver c(nullptr);
  carve_head(N, C, V, dtype, c, h);
  if (ws_bytes) *ws_bytes = c.off;
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_lm_head_ce_fwd_bwd(int32_t N, int32_t C, int32_t V, int32_t dtype, float eps, const void* x,
                                  const void* w_lm, const int32_t* targets, float* loss, float* row_loss, void* dx,
                                  float* dw_lm, int32_t accumulate, void* ws, void* stream) {
  gdb_status st = check_head(N, C, V, dtype);
  if (st != GDB_OK) return st;
  if (!(eps > 0.f) || !std::isfinite(eps)) return fail(GDB_EINVAL, "eps must be positive and finite");
  CHECK_PTR(x); CHECK_PTR(w_lm); CHECK_PTR(targets); CHECK_PTR(loss); CHECK_PTR(dx); CHECK_PTR(dw_lm); CHECK_PTR(ws);
  if (row_loss && (((uintptr_t)row_loss) & 3)) return fail(GDB_EINVAL, "row_loss is not 4-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  HeadWs h;
  Carver c(ws);
  carve_head(N, C, V, dtype, c, h);
  if (row_loss) h.row_loss = row_loss;
  HIPCHK(rmsnorm_fwd(dtype, x, h.xf, h.rf, N, C, eps, s));
  HIPCHK(gemm(dtype, gemm_args(h.xf, true, C, w_lm, true, C, N, V, C, EPI_STORE, h.z, V), s));
  HIPCHK(ce_fwd_bwd(dtype, h.z, targets, h.row_loss, N, V, s));
  HIPCHK(loss_reduce(h.row_loss, loss, N, s));
  HIPCHK(gemm(dtype, gemm_args(h.z, true, V, w_lm, false, C, N, C, V, EPI_STORE, h.dxf, C), s));
  HIPCHK(wgrad(dtype, h.z, V, h.xf, C, V, C, N, dw_lm, accumulate ? 1 : 0, h.partial, s));
  HIPCHK(rmsnorm_bwd(dtype, h.dxf, h.xf, h.rf, nullptr, dx, N, C, s));
  return finished({{F32, loss, 1, "loss"}, {dtype, dx, (size_t)N * C, "dx"}, {F32, dw_lm, (size_t)V * C, "dw_lm"}},
                  s);
}

// ----------------------------------------------------------- building blocks
gdb_status gdb_stream_copy(size_t bytes, const void* src, void* dst, void* stream) {
  if (bytes % 16) return fail(GDB_EINVAL, "bytes must be a multiple of 16");
  if (bytes == 0) { g_err.clear(); return GDB_OK; }
  CHECK_PTR(src); CHECK_PTR(dst);
  if ((const char*)src < (const char*)dst + bytes && (const char*)dst < (const char*)src + bytes)
    return fail(GDB_EINVAL, "src and dst overlap");
  HIPCHK(stream_copy(src, dst, bytes, (hipStream_t)stream));
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_rmsnorm_fwd(int32_t N, int32_t C, int32_t dtype, float eps, const void* x, void* xn, float* r,
                           void* stream) {
  if (N < 0 || C <= 0 || C % 8) return fail(GDB_EINVAL, "bad sizes N=%d C=%d (C multiple of 8)", N, C);
  if (dtype != GDB_F32 && dtype != GDB_BF16) return fail(GDB_EINVAL, "unknown dtype %d", dtype);
  if (!(eps > 0.f) || !std::isfinite(eps)) return fail(GDB_EINVAL, "eps must be positive and finite");
  CHECK_PTR(x); CHECK_PTR(xn); CHECK_PTR(r);
  HIPCHK(rmsnorm_fwd(dtype, x, xn, r, N, C, eps, (hipStream_t)stream));
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_rmsnorm_bwd(int32_t N, int32_t C, int32_t dtype, const void* dxn, const void* xn, const float* r,
                           const void* dres, void* dx, void* stream) {
  if (N < 0 || C <= 0 || C % 8) return fail(GDB_EINVAL, "bad sizes N=%d C=%d (C multiple of 8)", N, C);
  if (dtype != GDB_F32 && dtype != GDB_BF16) return fail(GDB_EINVAL, "unknown dtype %d", dtype);
  CHECK_PTR(dxn); CHECK_PTR(xn); CHECK_PTR(r); CHECK_PTR(dx);
  if (dres && (((uintptr_t)dres) & 15)) return fail(GDB_EINVAL, "dres is not 16-byte aligned");
  HIPCHK(rmsnorm_bwd(dtype, dxn, xn, r, dres, dx, N, C, (hipStream_t)stream));
  g_err.clear();
  return GDB_OK;
}

// epilogues of the GEMM entry points: 0-4, 6 (SQR) and 7 (DSQR); 5 is internal
static bool public_epi(int epi) { return (epi >= EPI_STORE && epi <= EPI_F32) || epi == EPI_SQR || epi == EPI_DSQR; }

gdb_status gdb_gemm_ws_bytes(int32_t dtype, int32_t M, int32_t N, int32_t K, int32_t epi, size_t* ws_bytes) {
  if (dtype != GDB_F32 && dtype != GDB_BF16) return fail(GDB_EINVAL, "unknown dtype %d", dtype);
  if (M < 0 || N < 0 || K < 0) return fail(GDB_EINVAL, "negative size");
  if (!public_epi(epi)) return fail(GDB_EINVAL, "unknown epilogue %d", epi);
  size_t b = 0;
  if (epi == EPI_F32) {
    const SplitPlan pl = gemm_split_plan(dtype, M, N, K);
    if (pl.splits > 1 || pl.splits2 > 0) b = (size_t)plan_slices(pl) * M * N * 4;
  }
  if (ws_bytes) *ws_bytes = b;
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_gemm(int32_t dtype, int32_t M, int32_t N, int32_t K, const void* A, int32_t a_kmajor, int32_t lda,
                    const void* B, int32_t b_kmajor, int32_t ldb, int32_t epi, void* C, int32_t ldc, const void* R,
                    int32_t ldr, void* C2, int32_t accumulate, void* ws, void* stream) {
  if (dtype != GDB_F32 && dtype != GDB_BF16) return fail(GDB_EINVAL, "unknown dtype %d", dtype);
  if (M < 0 || N < 0 || K < 0) return fail(GDB_EINVAL, "negative size");
  if (!public_epi(epi)) return fail(GDB_EINVAL, "unknown epilogue %d", epi);
  if (N % 8 || ldc % 8 || lda % 8 || ldb % 8) return fail(GDB_EINVAL, "N, lda, ldb, ldc must be multiples of 8");
  if (a_kmajor ? (K % 8 != 0) : (M % 8 != 0)) return fail(GDB_EINVAL, "the contiguous dimension of A must be a multiple of 8");
  if (b_kmajor && K % 8) return fail(GDB_EINVAL, "K must be a multiple of 8 when B is K-major");
  if (lda < (a_kmajor ? K : M) || ldb < (b_kmajor ? K : N) || ldc < N) return fail(GDB_EINVAL, "leading dimension too small");
  if (M == 0 || N == 0) { g_err.clear(); return GDB_OK; }
  CHECK_PTR(A); CHECK_PTR(B); CHECK_PTR(C);
  if (epi == EPI_RESID || epi == EPI_DRELU2 || epi == EPI_DSQR) {
    CHECK_PTR(R);
    if (ldr % 8 || ldr < N) return fail(GDB_EINVAL, "ldr must be a multiple of 8 and >= N");
  }
  if (epi == EPI_RELU2) CHECK_PTR(C2);
  if (epi == EPI_F32 && ldc != N) return fail(GDB_EINVAL, "fp32 output needs ldc == N");
  if (dtype == GDB_BF16 && epi == EPI_SQR && !(a_kmajor && b_kmajor))
    return fail(GDB_EUNSUPPORTED, "epilogue 6 needs both operands K-major in bf16");
  if (dtype == GDB_BF16 && epi == EPI_DSQR && !a_kmajor)
    return fail(GDB_EUNSUPPORTED, "epilogue 7 needs A K-major in bf16");
  GemmArgs g = gemm_args(A, a_kmajor != 0, lda, B, b_kmajor != 0, ldb, M, N, K, epi, C, ldc);
  g.R = R; g.ldr = ldr; g.C2 = C2; g.accumulate = accumulate ? 1 : 0;
  if (epi == EPI_F32) {
    const SplitPlan pl = gemm_split_plan(dtype, M, N, K);
    g.splits = pl.splits;
    g.split_cols = pl.split_cols; g.first1 = pl.first1; g.splits2 = pl.splits2;
    const bool split = g.splits > 1 || g.splits2 > 0;
    if (split) CHECK_PTR(ws);
    g.partial = (float*)ws;
    HIPCHK(gemm(dtype, g, (hipStream_t)stream));
    if (g.splits2 > 0)
      HIPCHK(splitk_reduce2(g.partial, (float*)C, M, N, g.splits, g.split_cols, g.first1, g.splits2, g.accumulate,
                            (hipStream_t)stream));
    else if (split)
      HIPCHK(splitk_reduce(g.partial, (float*)C, g.splits, (size_t)M * N, g.accumulate, (hipStream_t)stream));
  } else {
    HIPCHK(gemm(dtype, g, (hipStream_t)stream));
  }
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_fp8_quantize(int32_t R, int32_t Cc, int32_t dtype, const void* x, float* amax, uint8_t* xq,
                            uint8_t* xqt, int32_t Rp, void* stream) {
  if (dtype != GDB_F32 && dtype != GDB_BF16) return fail(GDB_EINVAL, "unknown dtype %d", dtype);
  if (R < 0 || Cc < 0 || Cc % 16) return fail(GDB_EINVAL, "R must be >= 0 and Cc a multiple of 16 (got %d, %d)", R, Cc);
  if ((long long)R * Cc > (1LL << 40)) return fail(GDB_EINVAL, "tensor too large");
  if (xqt && (Rp < R || Rp % 16)) return fail(GDB_EINVAL, "Rp must be a multiple of 16 and >= R (got %d)", Rp);
  if (!amax || (((uintptr_t)amax) & 3)) return fail(GDB_EINVAL, "amax is NULL or not 4-byte aligned");
  if (!xq && !xqt) return fail(GDB_EINVAL, "xq and xqt are both NULL");
  if (R > 0 && Cc > 0) CHECK_PTR(x);
  if (xq) CHECK_PTR(xq);
  if (xqt) CHECK_PTR(xqt);
  hipStream_t s = (hipStream_t)stream;
  HIPCHK(fp8_amax(dtype, x, (size_t)R * Cc, amax, s));
  HIPCHK(fp8_quant(dtype, x, R, Cc, amax, xq, xqt, xqt ? Rp : R, s));
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_gemm_fp8_ws_bytes(int32_t M, int32_t N, int32_t K, int32_t epi, size_t* ws_bytes) {
  if (M < 0 || N < 0 || K < 0) return fail(GDB_EINVAL, "negative size");
  if (!public_epi(epi)) return fail(GDB_EINVAL, "unknown epilogue %d", epi);
  const int sp = gemm_splits(FP8, M, N, K, epi);
  if (ws_bytes) *ws_bytes = sp > 1 ? (size_t)sp * M * N * 4 : 0;
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_gemm_fp8(int32_t dtype, int32_t M, int32_t N, int32_t K, const uint8_t* A, int32_t lda,
                        const float* amax_a, const uint8_t* B, int32_t ldb, const float* amax_b, int32_t epi, void* C,
                        int32_t ldc, const void* R, int32_t ldr, void* C2, int32_t accumulate, void* ws,
                        void* stream) {
  if (dtype != GDB_F32 && dtype != GDB_BF16) return fail(GDB_EINVAL, "unknown dtype %d", dtype);
  if (M < 0 || N < 0 || K < 0) return fail(GDB_EINVAL, "negative size");
  if (!public_epi(epi)) return fail(GDB_EINVAL, "unknown epilogue %d", epi);
  if (K % 16 || lda % 16 || ldb % 16) return fail(GDB_EINVAL, "K, lda, ldb must be multiples of 16");
  if (N % 8 || ldc % 8) return fail(GDB_EINVAL, "N and ldc must be multiples of 8");
  if (lda < K || ldb < K || ldc < N) return fail(GDB_EINVAL, "leading dimension too small");
  if (M == 0 || N == 0) { g_err.clear(); return GDB_OK; }
  CHECK_PTR(A); CHECK_PTR(B); CHECK_PTR(C);
  if (!amax_a || !amax_b || (((uintptr_t)amax_a) & 3) || (((uintptr_t)amax_b) & 3))
    return fail(GDB_EINVAL, "amax_a or amax_b is NULL or not 4-byte aligned");
  if (epi == EPI_RESID || epi == EPI_DRELU2 || epi == EPI_DSQR) {
    CHECK_PTR(R);
    if (ldr % 8 || ldr < N) return fail(GDB_EINVAL, "ldr must be a multiple of 8 and >= N");
  }
  if (epi == EPI_RELU2) CHECK_PTR(C2);
  if (epi == EPI_F32 && ldc != N) return fail(GDB_EINVAL, "fp32 output needs ldc == N");
  hipStream_t s = (hipStream_t)stream;
  GemmArgs g = gemm_args(A, true, lda, B, true, ldb, M, N, K, epi, C, ldc);
  g.R = R; g.ldr = ldr; g.C2 = C2; g.accumulate = accumulate ? 1 : 0;
  g.amax_a = amax_a; g.amax_b = amax_b;
  if (epi == EPI_F32) {
    g.splits = gemm_splits(FP8, M, N, K, epi);
    if (g.splits > 1) CHECK_PTR(ws);
    g.partial = (float*)ws;
  }
  HIPCHK(gemm_fp8(dtype, g, s));
  if (epi == EPI_F32 && g.splits > 1) HIPCHK(splitk_reduce(g.partial, (float*)C, g.splits, (size_t)M * N, g.accumulate, s));
  g_err.clear();
  return GDB_OK;
}

namespace {
gdb_status check_attn(int B, int T, int H, int Hkv, int D, int window, int dtype) {
  if (B <= 0 || T <= 0 || H <= 0 || Hkv <= 0) return fail(GDB_EINVAL, "B, T, H, Hkv must be positive");
  if (H % Hkv) return fail(GDB_EINVAL, "H (%d) must be a multiple of Hkv (%d)", H, Hkv);
  if (dtype != GDB_F32 && dtype != GDB_BF16) return fail(GDB_EINVAL, "unknown dtype %d", dtype);
  if (D != 64 && D != 128) return fail(GDB_EUNSUPPORTED, "head_dim %d not supported", D);
  if (dtype == GDB_BF16 && D != 128) return fail(GDB_EUNSUPPORTED, "bf16 attention needs head_dim 128");
  if (window < -1) return fail(GDB_EINVAL, "window must be >= -1");
  return GDB_OK;
}
}  // namespace

gdb_status gdb_qk_norm_rope_fwd(int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t D, int32_t dtype, float eps,
                                const void* qkv, void* out, float* rinv, const float* rope_tab, void* stream) {
  gdb_status st = check_attn(B, T, H, Hkv, D, -1, dtype);
  if (st != GDB_OK) return st;
  if (!(eps > 0.f) || !std::isfinite(eps)) return fail(GDB_EINVAL, "eps must be positive and finite");
  CHECK_PTR(qkv); CHECK_PTR(out); CHECK_PTR(rinv); CHECK_PTR(rope_tab);
  if (qkv == out) return fail(GDB_EINVAL, "out must not alias qkv");
  HIPCHK(qk_norm_rope_fwd(dtype, qkv, out, rinv, rope_tab, B, T, H, Hkv, D, eps, (hipStream_t)stream));
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_qk_norm_rope_bwd(int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t D, int32_t dtype, void* d,
                                const void* qkvh, const float* rinv, const float* rope_tab, void* stream) {
  gdb_status st = check_attn(B, T, H, Hkv, D, -1, dtype);
  if (st != GDB_OK) return st;
  CHECK_PTR(d); CHECK_PTR(qkvh); CHECK_PTR(rinv); CHECK_PTR(rope_tab);
  HIPCHK(qk_norm_rope_bwd(dtype, d, qkvh, rinv, rope_tab, B, T, H, Hkv, D, (hipStream_t)stream));
  g_err.clear();
  return GDB_OK;
}

// The bf16 attention kernels address one sequence's rows by 32-bit byte
// offsets from the sequence's first row.
static bool seq_fits_32bit(int T, int ld) { return (size_t)T * (size_t)ld * 2 <= 0x7FFFFF00ull; }

gdb_status gdb_attention_fwd(int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t D, int32_t window,
                             int32_t qk_normed, int32_t dtype, const void* qkv, int32_t ld, void* o, int32_t ldo,
                             float* lse, void* stream) {
  gdb_status st = check_attn(B, T, H, Hkv, D, window, dtype);
  if (st != GDB_OK) return st;
  if (ld < (H + 2 * Hkv) * D || ld % 8 || ldo < H * D || ldo % 8) return fail(GDB_EINVAL, "bad leading dimension");
  if (dtype == GDB_BF16 && !seq_fits_32bit(T, ld))
    return fail(GDB_EUNSUPPORTED, "bf16 attention: a sequence's qkv rows (T * ld * 2 bytes) must span under 2 GiB");
  CHECK_PTR(qkv); CHECK_PTR(o); CHECK_PTR(lse);
  AttnArgs at{};
  at.B = B; at.T = T; at.H = H; at.Hkv = Hkv; at.D = D; at.window = window >= T - 1 ? -1 : window;
  at.qk_normed = qk_normed ? 1 : 0;
  at.qkv = qkv; at.ld = ld; at.o = o; at.ldo = ldo; at.lse = lse;
  HIPCHK(attn_fwd(dtype, at, (hipStream_t)stream));
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_attention_bwd(int32_t B, int32_t T, int32_t H, int32_t Hkv, int32_t D, int32_t window, int32_t dtype,
                             const void* qkv, int32_t ld, const void* o, int32_t ldo, const float* lse,
                             const void* dout, int32_t lddo, void* dqkv, int32_t lddq, float* delta, void* stream) {
  gdb_status st = check_attn(B, T, H, Hkv, D, window, dtype);
  if (st != GDB_OK) return st;
  if (ld < (H + 2 * Hkv) * D || ld % 8 || ldo < H * D || ldo % 8 || lddo < H * D || lddo % 8 ||
      lddq < (H + 2 * Hkv) * D || lddq % 8)
    return fail(GDB_EINVAL, "bad leading dimension");
  if (dtype == GDB_BF16 && (!seq_fits_32bit(T, ld) || !seq_fits_32bit(T, lddo)))
    return fail(GDB_EUNSUPPORTED,
                "bf16 attention: a sequence's qkv and dO rows (T * ld * 2, T * lddo * 2 bytes) must span under 2 GiB");
  CHECK_PTR(qkv); CHECK_PTR(o); CHECK_PTR(lse); CHECK_PTR(dout); CHECK_PTR(dqkv); CHECK_PTR(delta);
  AttnArgs at{};
  at.B = B; at.T = T; at.H = H; at.Hkv = Hkv; at.D = D; at.window = window >= T - 1 ? -1 : window;
  at.qkv = qkv; at.ld = ld; at.o = (void*)o; at.ldo = ldo; at.lse = (float*)lse;
  at.dout = dout; at.lddo = lddo; at.dqkv = dqkv; at.lddq = lddq; at.delta = delta;
  HIPCHK(attn_bwd(dtype, at, (hipStream_t)stream));
  g_err.clear();
  return GDB_OK;
}

namespace {
gdb_status check_decode(int B, int H, int Hkv, int D, int max_len, int window) {
  if (B <= 0 || H <= 0 || Hkv <= 0) return fail(GDB_EINVAL, "B, H, Hkv must be positive");
  if (H % Hkv) return fail(GDB_EINVAL, "H (%d) must be a multiple of Hkv (%d)", H, Hkv);
  if (!decode_group_supported(H / Hkv)) return fail(GDB_EUNSUPPORTED, "H / Hkv = %d not supported", H / Hkv);
  if (D != 64 && D != 128) return fail(GDB_EUNSUPPORTED, "head_dim %d not supported", D);
  if (max_len <= 0) return fail(GDB_EINVAL, "max_len must be positive");
  if (window < -1) return fail(GDB_EINVAL, "window must be >= -1");
  return GDB_OK;
}
size_t decode_ws(int B, int H, int Hkv, int D, int max_len, int window) {
  int chunk = 0, nsplit = 1;
  decode_plan(B, Hkv, max_len, window, &chunk, &nsplit);
  return nsplit > 1 ? (size_t)B * H * nsplit * (D + 4) * sizeof(float) : 0;
}
}  // namespace

gdb_status gdb_attention_decode_ws_bytes(int32_t B, int32_t H, int32_t Hkv, int32_t D, int32_t max_len,
                                         int32_t window, size_t* ws_bytes) {
  gdb_status st = check_decode(B, H, Hkv, D, max_len, window);
  if (st != GDB_OK) return st;
  if (!ws_bytes) return fail(GDB_EINVAL, "ws_bytes is NULL");
  *ws_bytes = decode_ws(B, H, Hkv, D, max_len, window);
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_attention_decode(int32_t B, int32_t H, int32_t Hkv, int32_t D, int32_t window, int32_t dtype,
                                const void* q, int32_t ldq, const void* k, const void* v, int32_t ldk,
                                int64_t bstride, const int32_t* lens, int32_t max_len, void* o, int32_t ldo,
                                float* lse, void* ws, size_t ws_bytes, void* stream) {
  gdb_status st = check_decode(B, H, Hkv, D, max_len, window);
  if (st != GDB_OK) return st;
  if (dtype != GDB_F32 && dtype != GDB_BF16) return fail(GDB_EINVAL, "unknown dtype %d", dtype);
  if (ldq < H * D || ldq % 8 || ldo < H * D || ldo % 8 || ldk < Hkv * D || ldk % 8)
    return fail(GDB_EINVAL, "bad leading dimension");
  if (B > 1 && (bstride < (int64_t)(max_len - 1) * ldk + Hkv * D || bstride % 8))
    return fail(GDB_EINVAL, "bstride must be a multiple of 8 covering max_len rows");
  CHECK_PTR(q); CHECK_PTR(k); CHECK_PTR(v); CHECK_PTR(lens); CHECK_PTR(o);
  if (lse && (((uintptr_t)lse) & 15)) return fail(GDB_EINVAL, "lse is not 16-byte aligned");
  const size_t need = decode_ws(B, H, Hkv, D, max_len, window);
  if (need) {
    CHECK_PTR(ws);
    if (ws_bytes < need) return fail(GDB_EWORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
  }
  DecodeArgs a{};
  a.B = B; a.H = H; a.Hkv = Hkv; a.D = D; a.window = window; a.max_len = max_len;
  a.q = q; a.ldq = ldq; a.k = k; a.v = v; a.ldk = ldk; a.bstride = bstride; a.lens = lens;
  a.o = o; a.ldo = ldo; a.lse = lse; a.part = (float*)ws;
  HIPCHK(attn_decode(dtype, a, (hipStream_t)stream));
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_attention_decode_noalloc(int32_t B, int32_t H, int32_t Hkv, int32_t D, int32_t window, int32_t dtype,
                                        const void* q, int32_t ldq, const void* k, const void* v, int32_t ldk,
                                        int64_t bstride, const int32_t* lens, int32_t max_len, void* o, int32_t ldo,
                                        float* lse, void* stream) {
  gdb_status st = check_decode(B, H, Hkv, D, max_len, window);
  if (st != GDB_OK) return st;
  if (dtype != GDB_F32 && dtype != GDB_BF16) return fail(GDB_EINVAL, "unknown dtype %d", dtype);
  if (ldq < H * D || ldq % 8 || ldo < H * D || ldo % 8 || ldk < Hkv * D || ldk % 8)
    return fail(GDB_EINVAL, "bad leading dimension");
  if (B > 1 && (bstride < (int64_t)(max_len - 1) * ldk + Hkv * D || bstride % 8))
    return fail(GDB_EINVAL, "bstride must be a multiple of 8 covering max_len rows");
  CHECK_PTR(q); CHECK_PTR(k); CHECK_PTR(v); CHECK_PTR(lens); CHECK_PTR(o);
  if (lse && (((uintptr_t)lse) & 15)) return fail(GDB_EINVAL, "lse is not 16-byte aligned");
  const size_t need = decode_ws(B, H, Hkv, D, max_len, window);
  if (need > decode_scratch_bytes())
    return fail(GDB_EWORKSPACE, "this decode needs %zu bytes of split scratch, above the fixed %zu", need,
                decode_scratch_bytes());
  void* part = nullptr;
  if (need) HIPCHK(decode_scratch(&part));
  DecodeArgs a{};
  a.B = B; a.H = H; a.Hkv = Hkv; a.D = D; a.window = window; a.max_len = max_len;
  a.q = q; a.ldq = ldq; a.k = k; a.v = v; a.ldk = ldk; a.bstride = bstride; a.lens = lens;
  a.o = o; a.ldo = ldo; a.lse = lse; a.part = (float*)part;
  HIPCHK(attn_decode(dtype, a, (hipStream_t)stream));
  g_err.clear();
  return GDB_OK;
}

// ----------------------------------------------------------------- optimizer
namespace {
size_t al256(size_t b) { return (b + 255) / 256 * 256; }

// workspace of the Newton-Schulz iteration on a stack of `count` [m, n]
// matrices; with `muon` also the fp32 momentum-blended stack and the
// iteration's output
struct NsWs {
  size_t x, xa, a, bm, part, npart, inv, u, total;
};
// split count of the Gram product of a single matrix (a stack runs its
// products unsplit, batched over the items)
int ns_gram_splits(int count, int m, int n, int dt) {
  const int s_ = std::min(m, n), L = std::max(m, n);
  return count > 1 ? 1 : gemm_splits(dt, s_, s_, L, EPI_F32);
}

NsWs ns_layout(int count, int m, int n, int dt, bool muon) {
  const int s_ = std::min(m, n);
  const size_t es = dt_size(dt), mn = (size_t)count * m * n, ss = (size_t)count * s_ * s_;
  NsWs w{};
  size_t o = 0;
  if (muon) { w.u = o; o += al256(mn * 4); w.x = o; o += al256(mn * es); }
  w.xa = o; o += al256(mn * es);
  w.a = o; o += al256(ss * es);
  w.bm = o; o += al256(ss * es);
  w.part = o; o += count > 1 ? 0 : al256((size_t)ns_gram_splits(count, m, n, dt) * s_ * s_ * 4);
  w.npart = o; o += al256((size_t)count * OPT_PART * 4);
  w.inv = o; o += al256((size_t)count * 4);
  w.total = o;
  return w;
}

gdb_status check_ns(int count, int m, int n, int dtype, const float* coeffs, int steps) {
  if (count <= 0 || count > 65535) return fail(GDB_EINVAL, "count must be in [1, 65535]");
  if (m <= 0 || n <= 0 || m % 8 || n % 8) return fail(GDB_EINVAL, "m, n must be positive multiples of 8");
  if (dtype != GDB_F32 && dtype != GDB_BF16) return fail(GDB_EINVAL, "unknown dtype %d", dtype);
  if (steps < 0 || steps > 64) return fail(GDB_EINVAL, "steps must be in [0, 64]");
  if (steps > 0 && !coeffs) return fail(GDB_EINVAL, "coeffs is NULL");
  for (int i = 0; i < 3 * steps; ++i)
    if (!std::isfinite(coeffs[i])) return fail(GDB_EINVAL, "coefficient %d is not finite", i);
  return GDB_OK;
}

// the iteration from x0 (already in `start`), ending in `out`; `other` is the
// ping-pong partner.  Tall matrices take the Gram X^T X, wide ones X X^T
// (the same map: X p(X^T X) = p(X X^T) X).  A single matrix runs its Gram
// split over K into fp32 partials, added and cast in one pass; a stack runs
// every product as one batched launch over its items.  The two other lines
// apply their axpy in the GEMM epilogue.
hipError_t ns_iterate(int dt, int count, int m, int n, const float* coeffs, int steps, void* out, void* other,
                      void* A, void* Bm, float* part, hipStream_t s) {
  const bool tall = m >= n;
  const int s_ = tall ? n : m, L = tall ? m : n;
  const int spg = ns_gram_splits(count, m, n, dt);
  const long long smn = (long long)m * n, sss = (long long)s_ * s_;
  auto batched = [&](GemmArgs g, long long sa, long long sb, long long sc, long long sr) {
    g.batch = count;
    g.bsA = sa; g.bsB = sb; g.bsC = sc; g.bsR = sr;
    return g;
  };
  void* cur = steps % 2 == 0 ? out : other;
  for (int it = 0; it < steps; ++it) {
    const float a = coeffs[3 * it], b = coeffs[3 * it + 1], c = coeffs[3 * it + 2];
    void* nxt = cur == out ? other : out;
    // A = X^T X (tall: both operands M/N-contiguous) or X X^T (wide: both K-contiguous)
    hipError_t e;
    if (count == 1) {
      GemmArgs g = gemm_args(cur, !tall, n, cur, !tall, n, s_, s_, L, EPI_F32, part, s_);
      g.splits = spg;
      g.partial = part;
      e = gemm(dt, g, s);
      if (e == hipSuccess) e = splitk_axpby(dt, part, spg, (size_t)sss, 1.0f, 0.0f, nullptr, A, s);
    } else {
      e = gemm(dt, batched(gemm_args(cur, !tall, n, cur, !tall, n, s_, s_, L, EPI_STORE, A, s_), smn, smn, sss, 0), s);
    }
    // B = b A + c A A (A symmetric: its rows serve as the second operand's K-contiguous rows)
    GemmArgs g2 = batched(gemm_args(A, true, s_, A, true, s_, s_, s_, s_, EPI_AXPBY, Bm, s_), sss, sss, sss, sss);
    g2.R = A; g2.ldr = s_; g2.alpha = c; g2.beta = b;
    if (e == hipSuccess) e = gemm(dt, g2, s);
    // X' = a X + X B (tall) or a X + B X (wide); B symmetric
    GemmArgs g3 = tall ? batched(gemm_args(cur, true, n, Bm, true, s_, m, n, s_, EPI_AXPBY, nxt, n), smn, sss, smn, smn)
                       : batched(gemm_args(Bm, true, s_, cur, false, n, m, n, s_, EPI_AXPBY, nxt, n), sss, smn, smn, smn);
    g3.R = cur; g3.ldr = n; g3.alpha = 1.0f; g3.beta = a;
    if (e == hipSuccess) e = gemm(dt, g3, s);
    if (e != hipSuccess) return e;
    cur = nxt;
  }
  return hipSuccess;
}
}  // namespace

gdb_status gdb_newton_schulz_ws_bytes(int32_t count, int32_t m, int32_t n, int32_t dtype, size_t* ws_bytes) {
  gdb_status st = check_ns(count, m, n, dtype, nullptr, 0);
  if (st != GDB_OK) return st;
  if (!ws_bytes) return fail(GDB_EINVAL, "ws_bytes is NULL");
  *ws_bytes = ns_layout(count, m, n, dtype, false).total;
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_newton_schulz(int32_t count, int32_t m, int32_t n, int32_t dtype, const float* G, void* X,
                             const float* coeffs, int32_t steps, float norm_scale, float eps, void* ws,
                             size_t ws_bytes, void* stream) {
  gdb_status st = check_ns(count, m, n, dtype, coeffs, steps);
  if (st != GDB_OK) return st;
  if (!(norm_scale > 0.f) || !std::isfinite(norm_scale) || !(eps >= 0.f) || !std::isfinite(eps))
    return fail(GDB_EINVAL, "norm_scale must be positive and eps non-negative");
  CHECK_PTR(G); CHECK_PTR(X); CHECK_PTR(ws);
  const NsWs w = ns_layout(count, m, n, dtype, false);
  if (ws_bytes < w.total) return fail(GDB_EWORKSPACE, "workspace %zu bytes < %zu", ws_bytes, w.total);
  if ((const void*)G == X) return fail(GDB_EINVAL, "X must not alias G");
  char* b = (char*)ws;
  hipStream_t s = (hipStream_t)stream;
  const size_t mn = (size_t)m * n;
  int np = 0;
  void* start = steps % 2 == 0 ? X : (void*)(b + w.xa);
  HIPCHK(sumsq_partials(G, mn, count, (float*)(b + w.npart), &np, s));
  HIPCHK(norm_final((float*)(b + w.npart), np, count, norm_scale, eps, (float*)(b + w.inv), s));
  HIPCHK(scale_cast(dtype, G, (float*)(b + w.inv), start, mn, count, s));
  HIPCHK(ns_iterate(dtype, count, m, n, coeffs, steps, X, b + w.xa, b + w.a, b + w.bm, (float*)(b + w.part), s));
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_muon_ws_bytes(int32_t count, int32_t m, int32_t n, int32_t dtype, size_t* ws_bytes) {
  gdb_status st = check_ns(count, m, n, dtype, nullptr, 0);
  if (st != GDB_OK) return st;
  if (!ws_bytes) return fail(GDB_EINVAL, "ws_bytes is NULL");
  *ws_bytes = ns_layout(count, m, n, dtype, true).total;
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_muon_step(int32_t count, int32_t m, int32_t n, int32_t dtype, float* p, void* p_bf16, const float* g,
                         float* buf, float lr, float momentum, int32_t nesterov, float wd, float scale,
                         const float* coeffs, int32_t steps, float norm_scale, float eps, void* ws, size_t ws_bytes,
                         void* stream) {
  gdb_status st = check_ns(count, m, n, dtype, coeffs, steps);
  if (st != GDB_OK) return st;
  for (float f : {lr, momentum, wd, scale, norm_scale, eps})
    if (!std::isfinite(f)) return fail(GDB_EINVAL, "non-finite hyperparameter");
  if (!(norm_scale > 0.f) || eps < 0.f) return fail(GDB_EINVAL, "norm_scale must be positive and eps non-negative");
  CHECK_PTR(p); CHECK_PTR(g); CHECK_PTR(buf); CHECK_PTR(ws);
  if (p_bf16 && (((uintptr_t)p_bf16) & 15)) return fail(GDB_EINVAL, "p_bf16 is not 16-byte aligned");
  const NsWs w = ns_layout(count, m, n, dtype, true);
  if (ws_bytes < w.total) return fail(GDB_EWORKSPACE, "workspace %zu bytes < %zu", ws_bytes, w.total);
  char* b = (char*)ws;
  hipStream_t s = (hipStream_t)stream;
  const size_t mn = (size_t)m * n;
  int np = 0;
  void* X = b + w.x;
  void* start = steps % 2 == 0 ? X : (void*)(b + w.xa);
  HIPCHK(muon_momentum(g, buf, (float*)(b + w.u), mn, count, momentum, nesterov ? 1 : 0, (float*)(b + w.npart), &np,
                       s));
  HIPCHK(norm_final((float*)(b + w.npart), np, count, norm_scale, eps, (float*)(b + w.inv), s));
  HIPCHK(scale_cast(dtype, (float*)(b + w.u), (float*)(b + w.inv), start, mn, count, s));
  HIPCHK(ns_iterate(dtype, count, m, n, coeffs, steps, X, b + w.xa, b + w.a, b + w.bm, (float*)(b + w.part), s));
  HIPCHK(muon_apply(dtype, p, X, (bf16*)p_bf16, mn * count, 1.0f - lr * wd, lr * scale, s));
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_adamw_step(int64_t n, float* p, void* p_bf16, const float* g, float* m, float* v, int32_t t, float lr,
                          float beta1, float beta2, float eps, float wd, void* stream) {
  if (n <= 0 || n % 8) return fail(GDB_EINVAL, "n must be a positive multiple of 8");
  if (t < 1) return fail(GDB_EINVAL, "t counts steps from 1");
  for (float f : {lr, beta1, beta2, eps, wd})
    if (!std::isfinite(f)) return fail(GDB_EINVAL, "non-finite hyperparameter");
  if (!(beta1 >= 0.f && beta1 < 1.f && beta2 >= 0.f && beta2 < 1.f)) return fail(GDB_EINVAL, "betas must be in [0, 1)");
  if (!(eps > 0.f)) return fail(GDB_EINVAL, "eps must be positive");
  CHECK_PTR(p); CHECK_PTR(g); CHECK_PTR(m); CHECK_PTR(v);
  if (p_bf16 && (((uintptr_t)p_bf16) & 15)) return fail(GDB_EINVAL, "p_bf16 is not 16-byte aligned");
  HIPCHK(adamw(p, g, m, v, (bf16*)p_bf16, (size_t)n, lr, beta1, beta2, eps, wd, t, (hipStream_t)stream));
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_cross_entropy(int32_t N, int32_t V, int32_t dtype, void* z, const int32_t* targets, float* row_loss,
                             float* loss, void* stream) {
  if (N <= 0 || V <= 0 || V % 8) return fail(GDB_EINVAL, "N must be positive, V a positive multiple of 8");
  if (dtype != GDB_F32 && dtype != GDB_BF16) return fail(GDB_EINVAL, "unknown dtype %d", dtype);
  CHECK_PTR(z); CHECK_PTR(targets); CHECK_PTR(row_loss); CHECK_PTR(loss);
  HIPCHK(ce_fwd_bwd(dtype, z, targets, row_loss, N, V, (hipStream_t)stream));
  HIPCHK(loss_reduce(row_loss, loss, N, (hipStream_t)stream));
  g_err.clear();
  return GDB_OK;
}

// ---------------------------------------------------------- smear, backout
namespace {
gdb_status check_rows(int32_t N, int32_t C, int32_t dtype) {
  if (N < 0 || C <= 0 || C % 8) return fail(GDB_EINVAL, "bad sizes N=%d C=%d (C a positive multiple of 8)", N, C);
  if (dtype != GDB_F32 && dtype != GDB_BF16) return fail(GDB_EINVAL, "unknown dtype %d", dtype);
  return GDB_OK;
}
gdb_status check_scalar(const float* p, const char* name) {
  if (!p || (((uintptr_t)p) & 3)) return fail(GDB_EINVAL, "%s is NULL or not 4-byte aligned", name);
  return GDB_OK;
}
constexpr int MAX_SMEAR = 63;
}  // namespace

gdb_status gdb_smear_fwd(int32_t B, int32_t T, int32_t C, int32_t ng, int32_t dtype, const void* e, const void* w,
                         const float* lam, void* x, float* s_save, void* stream) {
  gdb_status st;
  if (B < 0 || T <= 0) return fail(GDB_EINVAL, "B must be >= 0 and T positive (got %d, %d)", B, T);
  if ((long long)B * T > (1LL << 30)) return fail(GDB_EINVAL, "B*T too large");
  if ((st = check_rows(B * T, C, dtype)) != GDB_OK) return st;
  if (ng < 1 || ng > MAX_SMEAR || ng > C) return fail(GDB_EINVAL, "ng must be in [1, min(%d, C)] (got %d)", MAX_SMEAR, ng);
  if (B == 0) { g_err.clear(); return GDB_OK; }
  CHECK_PTR(e); CHECK_PTR(w); CHECK_PTR(x); CHECK_PTR(s_save);
  if ((st = check_scalar(lam, "lam")) != GDB_OK) return st;
  if (x == e) return fail(GDB_EINVAL, "x must not alias e");
  HIPCHK(smear_fwd(dtype, e, w, ng, lam, x, s_save, B * T, T, C, (hipStream_t)stream));
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_smear_bwd(int32_t B, int32_t T, int32_t C, int32_t ng, int32_t dtype, const void* e, const void* w,
                         const float* lam, const float* s_save, const void* dx, const float* dxa, void* de,
                         float* dlam, float* dw, int32_t accumulate, void* ws, void* stream) {
  gdb_status st;
  if (B <= 0 || T <= 0) return fail(GDB_EINVAL, "B and T must be positive (got %d, %d)", B, T);
  if ((long long)B * T > (1LL << 30)) return fail(GDB_EINVAL, "B*T too large");
  if ((st = check_rows(B * T, C, dtype)) != GDB_OK) return st;
  if (ng < 1 || ng > MAX_SMEAR || ng > C) return fail(GDB_EINVAL, "ng must be in [1, min(%d, C)] (got %d)", MAX_SMEAR, ng);
  CHECK_PTR(e); CHECK_PTR(w); CHECK_PTR(s_save); CHECK_PTR(dx); CHECK_PTR(de); CHECK_PTR(ws);
  if (dxa) CHECK_PTR(dxa);
  if ((st = check_scalar(lam, "lam")) != GDB_OK) return st;
  if ((st = check_scalar(dlam, "dlam")) != GDB_OK) return st;
  if ((st = check_scalar(dw, "dw")) != GDB_OK) return st;
  if (de == dx || de == (const void*)dxa) return fail(GDB_EINVAL, "de must not alias dx or dxa");
  const int nb = smear_partials(B * T);
  if ((size_t)nb * (ng + 1) * 4 > GDB_EXTRAS_WS_BYTES) return fail(GDB_EWORKSPACE, "extras workspace too small");
  HIPCHK(smear_bwd(dtype, e, w, ng, lam, s_save, dx, dxa, de, (float*)ws, dlam, dw, accumulate ? 1 : 0, B * T, T, C,
                   (hipStream_t)stream));
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_backout_fwd(int32_t N, int32_t C, int32_t dtype, const void* x, const void* x_bo, const float* lam,
                           void* y, void* stream) {
  gdb_status st;
  if ((st = check_rows(N, C, dtype)) != GDB_OK) return st;
  if (N == 0) { g_err.clear(); return GDB_OK; }
  CHECK_PTR(x); CHECK_PTR(x_bo); CHECK_PTR(y);
  if ((st = check_scalar(lam, "lam")) != GDB_OK) return st;
  if (y == x_bo && x != x_bo) return fail(GDB_EINVAL, "y must not alias x_bo");
  HIPCHK(backout_fwd(dtype, x, x_bo, lam, y, (size_t)N * C, (hipStream_t)stream));
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_backout_bwd(int32_t N, int32_t C, int32_t dtype, const void* dy, const void* x_bo, const float* lam,
                           void* dx_bo, float* dlam, int32_t accumulate, void* ws, void* stream) {
  gdb_status st;
  if ((st = check_rows(N, C, dtype)) != GDB_OK) return st;
  if (N == 0) return fail(GDB_EINVAL, "N must be positive");
  CHECK_PTR(dy); CHECK_PTR(x_bo); CHECK_PTR(dx_bo); CHECK_PTR(ws);
  if ((st = check_scalar(lam, "lam")) != GDB_OK) return st;
  if ((st = check_scalar(dlam, "dlam")) != GDB_OK) return st;
  if (dx_bo == dy || dx_bo == x_bo) return fail(GDB_EINVAL, "dx_bo must not alias dy or x_bo");
  HIPCHK(backout_bwd(dtype, dy, x_bo, lam, dx_bo, (float*)ws, dlam, accumulate ? 1 : 0, N, C, (hipStream_t)stream));
  g_err.clear();
  return GDB_OK;
}

// ------------------------------------------------- mixing, value embedding
gdb_status gdb_mix_fwd(int32_t N, int32_t C, int32_t dtype, const void* x, const void* x0, const float* lam, void* y,
                       void* stream) {
  gdb_status st;
  if ((st = check_rows(N, C, dtype)) != GDB_OK) return st;
  if (N == 0) { g_err.clear(); return GDB_OK; }
  CHECK_PTR(x); CHECK_PTR(x0); CHECK_PTR(y);
  if ((st = check_scalar(lam, "lam")) != GDB_OK) return st;
  HIPCHK(mix_fwd(dtype, x, x0, lam, y, (size_t)N * C, (hipStream_t)stream));
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_mix_bwd(int32_t N, int32_t C, int32_t dtype, const void* dy, const void* x, const void* x0,
                       const float* lam, void* dx, float* dx0, int32_t accumulate_dx0, float* dlam, int32_t accumulate,
                       void* ws, void* stream) {
  gdb_status st;
  if ((st = check_rows(N, C, dtype)) != GDB_OK) return st;
  if (N == 0) return fail(GDB_EINVAL, "N must be positive");
  CHECK_PTR(dy); CHECK_PTR(x); CHECK_PTR(x0); CHECK_PTR(dx); CHECK_PTR(dx0); CHECK_PTR(ws);
  if ((st = check_scalar(lam, "lam")) != GDB_OK) return st;
  if ((st = check_scalar(dlam, "dlam")) != GDB_OK) return st;
  if ((size_t)mix_partials(N) * 2 * 4 > GDB_EXTRAS_WS_BYTES) return fail(GDB_EWORKSPACE, "extras workspace too small");
  HIPCHK(mix_bwd(dtype, dy, x, x0, lam, dx, dx0, accumulate_dx0 ? 1 : 0, (float*)ws, dlam, accumulate ? 1 : 0, N, C,
                 (hipStream_t)stream));
  g_err.clear();
  return GDB_OK;
}

namespace {
gdb_status check_ve(int32_t N, int32_t Hkv, int32_t D, int32_t dtype, int32_t ldq, int32_t voff, int32_t ldx, int32_t V,
                    int32_t nc) {
  if (N < 0) return fail(GDB_EINVAL, "N must be >= 0");
  if (dtype != GDB_F32 && dtype != GDB_BF16) return fail(GDB_EINVAL, "unknown dtype %d", dtype);
  if (Hkv < 1 || Hkv > 64) return fail(GDB_EUNSUPPORTED, "Hkv must be in [1, 64] (got %d)", Hkv);
  if (D != 64 && D != 128) return fail(GDB_EUNSUPPORTED, "D must be 64 or 128 (got %d)", D);
  if (V <= 0) return fail(GDB_EINVAL, "V must be positive");
  if (ldx <= 0 || ldx % 8 || ldq % 8 || voff % 8 || voff < 0 || voff + Hkv * D > ldq)
    return fail(GDB_EINVAL, "ldx, ldq, voff must be multiples of 8 with voff + Hkv*D <= ldq");
  if (nc < 1 || nc > MAX_VE_GATE || nc > ldx) return fail(GDB_EINVAL, "nc must be in [1, min(%d, ldx)]", MAX_VE_GATE);
  return GDB_OK;
}
size_t ve_bwd_ws(int N, int Hkv, int nc, int det) {
  return al256((size_t)ve_gate_partials(N) * Hkv * nc * 4) + al256((size_t)std::max(N, 1) * Hkv * 4) +
         (det ? token_order_ws_bytes(N) : 0);
}
}  // namespace

gdb_status gdb_ve_fwd(int32_t N, int32_t Hkv, int32_t D, int32_t dtype, void* qkv, int32_t ldq, int32_t voff,
                      const void* xn, int32_t ldx, const int32_t* ids, const void* ve, int32_t V, const void* wg,
                      int32_t nc, float* s_save, void* stream) {
  gdb_status st;
  if ((st = check_ve(N, Hkv, D, dtype, ldq, voff, ldx, V, nc)) != GDB_OK) return st;
  if (N == 0) { g_err.clear(); return GDB_OK; }
  CHECK_PTR(qkv); CHECK_PTR(xn); CHECK_PTR(ve); CHECK_PTR(wg); CHECK_PTR(s_save);
  if (!ids || (((uintptr_t)ids) & 3)) return fail(GDB_EINVAL, "ids is NULL or not 4-byte aligned");
  HIPCHK(ve_fwd(dtype, qkv, ldq, voff, xn, ldx, ids, ve, wg, nc, Hkv, D, V, s_save, N, (hipStream_t)stream));
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_ve_bwd_ws_bytes(int32_t N, int32_t Hkv, int32_t nc, int32_t deterministic, size_t* ws_bytes) {
  if (N < 0 || Hkv < 1 || Hkv > 64 || nc < 1 || nc > MAX_VE_GATE) return fail(GDB_EINVAL, "bad sizes");
  if (!ws_bytes) return fail(GDB_EINVAL, "ws_bytes is NULL");
  *ws_bytes = ve_bwd_ws(N, Hkv, nc, deterministic ? 1 : 0);
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_ve_bwd(int32_t N, int32_t Hkv, int32_t D, int32_t dtype, const void* dqkv, int32_t ldq, int32_t voff,
                      const int32_t* ids, const void* ve, int32_t V, const float* s_save, const void* xn, void* dxn,
                      int32_t ldx, const void* wg, int32_t nc, float* dve, float* dwg, int32_t accumulate,
                      int32_t deterministic, void* ws, void* stream) {
  gdb_status st;
  if ((st = check_ve(N, Hkv, D, dtype, ldq, voff, ldx, V, nc)) != GDB_OK) return st;
  if (N == 0) return fail(GDB_EINVAL, "N must be positive");
  CHECK_PTR(dqkv); CHECK_PTR(ve); CHECK_PTR(s_save); CHECK_PTR(xn); CHECK_PTR(dxn); CHECK_PTR(wg); CHECK_PTR(dve);
  CHECK_PTR(ws);
  if (!ids || (((uintptr_t)ids) & 3)) return fail(GDB_EINVAL, "ids is NULL or not 4-byte aligned");
  if ((st = check_scalar(dwg, "dwg")) != GDB_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  char* b = (char*)ws;
  float* part = (float*)b;
  float* ds = (float*)(b + al256((size_t)ve_gate_partials(N) * Hkv * nc * 4));
  void* ord = b + al256((size_t)ve_gate_partials(N) * Hkv * nc * 4) + al256((size_t)N * Hkv * 4);
  const int acc = accumulate ? 1 : 0;
  if (deterministic) {
    const int32_t *sk, *perm;
    HIPCHK(ve_bwd(dtype, dqkv, ldq, voff, ids, ve, s_save, Hkv, D, V, ds, nullptr, N, s));
    HIPCHK(token_order(ids, N, V, ord, &sk, &perm, s));
    HIPCHK(rows_segsum(dtype, sk, perm, N, dqkv, ldq, voff, Hkv * D, s_save, Hkv, D, dve, V, acc, s));
  } else {
    if (!acc) HIPCHK(fill_f32(dve, (size_t)V * Hkv * D, 0.f, s));
    HIPCHK(ve_bwd(dtype, dqkv, ldq, voff, ids, ve, s_save, Hkv, D, V, ds, dve, N, s));
  }
  HIPCHK(ve_gate_bwd(dtype, ds, xn, dxn, ldx, wg, nc, Hkv, part, dwg, acc, N, s));
  g_err.clear();
  return GDB_OK;
}

// ---------------------------------------------------------------- NorMuon
gdb_status gdb_normuon_ws_bytes(int32_t count, int32_t m, int32_t n, int32_t dtype, size_t* ws_bytes) {
  gdb_status st = check_ns(count, m, n, dtype, nullptr, 0);
  if (st != GDB_OK) return st;
  if (!ws_bytes) return fail(GDB_EINVAL, "ws_bytes is NULL");
  *ws_bytes = ns_layout(count, m, n, dtype, true).total + al256((size_t)count * m * 3 * 4);
  g_err.clear();
  return GDB_OK;
}

gdb_status gdb_normuon_step(int32_t count, int32_t m, int32_t n, int32_t dtype, float* p, void* p_bf16,
                            const float* g, float* buf, float* v, float lr, float momentum, int32_t nesterov,
                            float wd, float scale, float beta2, const float* coeffs, int32_t steps, float norm_scale,
                            float eps, void* ws, size_t ws_bytes, void* stream) {
  gdb_status st = check_ns(count, m, n, dtype, coeffs, steps);
  if (st != GDB_OK) return st;
  for (float f : {lr, momentum, wd, scale, norm_scale, eps, beta2})
    if (!std::isfinite(f)) return fail(GDB_EINVAL, "non-finite hyperparameter");
  if (!(norm_scale > 0.f) || eps < 0.f) return fail(GDB_EINVAL, "norm_scale must be positive and eps non-negative");
  if (!(beta2 >= 0.f && beta2 < 1.f)) return fail(GDB_EINVAL, "beta2 must be in [0, 1)");
  CHECK_PTR(p); CHECK_PTR(g); CHECK_PTR(buf); CHECK_PTR(v); CHECK_PTR(ws);
  if (p_bf16 && (((uintptr_t)p_bf16) & 15)) return fail(GDB_EINVAL, "p_bf16 is not 16-byte aligned");
  const NsWs w = ns_layout(count, m, n, dtype, true);
  const size_t need = w.total + al256((size_t)count * m * 3 * 4);
  if (ws_bytes < need) return fail(GDB_EWORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
  char* b = (char*)ws;
  hipStream_t s = (hipStream_t)stream;
  const size_t mn = (size_t)m * n;
  int np = 0;
  void* X = b + w.x;
  void* start = steps % 2 == 0 ? X : (void*)(b + w.xa);
  float* stat = (float*)(b + w.total);
  float* fs = stat + 2 * (size_t)count * m;
  HIPCHK(muon_momentum(g, buf, (float*)(b + w.u), mn, count, momentum, nesterov ? 1 : 0, (float*)(b + w.npart), &np,
                       s));
  HIPCHK(norm_final((float*)(b + w.npart), np, count, norm_scale, eps, (float*)(b + w.inv), s));
  HIPCHK(scale_cast(dtype, (float*)(b + w.u), (float*)(b + w.inv), start, mn, count, s));
  HIPCHK(ns_iterate(dtype, count, m, n, coeffs, steps, X, b + w.xa, b + w.a, b + w.bm, (float*)(b + w.part), s));
  HIPCHK(normuon_scale(dtype, X, count, m, n, v, beta2, stat, fs, s));
  HIPCHK(normuon_apply(dtype, p, X, fs, (bf16*)p_bf16, (size_t)count * m, n, 1.0f - lr * wd, lr * scale, s));
  g_err.clear();
  return GDB_OK;
}

}  // extern "C"
