"""Stage-wise parity: each stage of the block that a discrete decision or a
cancelling reduction makes hard to judge at block level, run alone through
the C ABI on seeded inputs that the GPU and the oracle share exactly.

* fp8 MLP: the six products of the largest model's MLP (section "1. Le
  modèle GPT" of "Comment Entraîner Votre Propre ChatGPT Pour 50€ ?": most
  matrix products in fp8) in the layouts the block uses, each operand a
  seeded tensor of the block's dtype: the e4m3 codes must be bit-exact, each
  product within the dtype's bar.
* the e4m3 quantiser on every finite bfloat16 bit pattern.
* reductions of the extras (residual mixing scalars, value-embedding gate,
  smear, backout): plain relative bars on seeded inputs.
* the deterministic backward: the same bits on every run, and parity.
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpt_decoder_block_amd import ops
from gpu_util import DEV, TDT, TOL, assert_close, dev, empty, host, rounded
from seeded_inputs import draw_ids_zipf, draw_upstream, workload

pytestmark = pytest.mark.gpu
RNG = np.random.default_rng(20260)


def _e4m3_values(codes: torch.Tensor) -> np.ndarray:
    """uint8 e4m3fn codes -> float64 values (torch's e4m3fn decode, on the host)."""
    return codes.cpu().view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _quant(x_np, dt, Rp=None):
    """GPU codes of x (row-major and, with Rp, transposed) and its amax; checks
    them bit-exact against the oracle's quantiser on the same values."""
    R, Cc = x_np.shape
    xq = torch.empty((R, Cc), dtype=torch.uint8, device=DEV)
    xqt = torch.full((Cc, Rp), 0x5A, dtype=torch.uint8, device=DEV) if Rp else None
    amax = empty((1,), torch.float32, fill=-1.0)
    ops.fp8_quantize(dev(x_np, dt), amax, xq, xqt, Rp or 0)
    torch.cuda.synchronize()
    q_ref, s_ref = O.fp8_quantize(x_np.astype(np.float64), dt)
    np.testing.assert_array_equal(_e4m3_values(xq), q_ref)
    if Rp:
        qt = _e4m3_values(xqt)
        np.testing.assert_array_equal(qt[:, :R], q_ref.T)
        assert not np.any(qt[:, R:])
    assert float(host(amax)[0]) == float(np.max(np.abs(x_np)))
    return xq, xqt, amax


@pytest.mark.parametrize("name,N", [("d26", 130), ("tiny", 37)])
def test_fp8_mlp_stages(name, N):
    """The block's six fp8 products, stage by stage, from seeded tensors:
    forward  h = relu2(q(xn2) q(w_fc)^T),  x_out = x_mid + q(h) q(w_proj)^T;
    backward du = (q(dout) q(w_proj^T)^T) * 2 sqrt(h),  dw_proj = q(dout)^T q(h),
             dxn2 = q(du) q(w_fc^T)^T,  dw_fc = q(du)^T q(xn2).
    Codes bit-exact; bf16 outputs within 2e-2.  Both sides multiply the same
    codes, so only the accumulation and the output rounding differ; fp32
    outputs (the weight gradients, and everything in an fp32 model) are held
    to 1e-3: the fp8 MFMA's own accumulation differs from exact summation by
    about 1e-4 of the sum of the terms' magnitudes (an in-bounds probe of
    v_mfma_f32_32x32x64_f8f6f4), above the fp32 bar of 1e-4."""
    w = workload(name)
    dt = "bf16" if name == "d26" else "f32"
    C, F = w.C, w.mlp_hidden
    Np = (N + 15) // 16 * 16
    print(f"fp8 mlp stages {name} dt={dt} N={N} C={C} F={F}", flush=True)
    g = np.random.default_rng(11)
    x_mid = rounded(g.standard_normal((N, C)), dt)
    xn2 = g.standard_normal((N, C))
    xn2 = rounded(xn2 / np.sqrt(np.mean(xn2 ** 2, axis=1, keepdims=True)), dt)      # unit-RMS rows
    w_fc = rounded(g.standard_normal((F, C)) * 0.02, dt)
    w_proj = rounded(g.standard_normal((C, F)) * 0.02, dt)
    u = g.standard_normal((N, F)) * 0.6
    h = rounded(O.relu2(u), dt)                                                      # relu(u)^2: zeros and a tail
    dout = rounded(g.standard_normal((N, C)) * 1e-3, dt)
    du = rounded(g.standard_normal((N, F)) * 1e-4 * (u > 0), dt)                    # zero where relu is off
    f64 = lambda a: np.asarray(a, dtype=np.float64)
    out_tol = TOL[dt] if dt == "bf16" else 1e-3

    # forward: up-projection with the squared ReLU
    xq, xqt, am_x = _quant(xn2, dt, Np)
    wq, wqt, am_w = _quant(w_fc, dt, F)
    hg = empty((N, F), dt)
    ops.gemm_fp8(N, F, C, xq, C, am_x, wq, C, am_w, ops.EPI_SQR, hg, F)
    torch.cuda.synchronize()
    assert_close(hg, O.relu2(O.mm_nt(f64(xn2), f64(w_fc), True, dt)), dt, "h", tol=out_tol)
    # forward: down-projection onto the residual
    hq, hqt, am_h = _quant(h, dt, Np)
    pq, pqt, am_p = _quant(w_proj, dt, C)
    xo = empty((N, C), dt)
    ops.gemm_fp8(N, C, F, hq, F, am_h, pq, F, am_p, ops.EPI_RESID, xo, C, R=dev(x_mid, dt), ldr=C)
    torch.cuda.synchronize()
    assert_close(xo, f64(x_mid) + O.mm_nt(f64(h), f64(w_proj), True, dt), dt, "x_out", tol=out_tol)
    # backward: dh = dout . w_proj with the ReLU^2 derivative from h (2 sqrt(h) = 2 relu(u))
    dq, dqt, am_d = _quant(dout, dt, Np)
    dug = empty((N, F), dt)
    ops.gemm_fp8(N, F, C, dq, C, am_d, pqt, C, am_p, ops.EPI_DSQR, dug, F, R=dev(h, dt), ldr=F)
    torch.cuda.synchronize()
    dh_ref = O.mm_nt(f64(dout), f64(w_proj).T, True, dt)
    assert_close(dug, dh_ref * O.relu2_grad(np.sqrt(f64(h))), dt, "du", tol=out_tol)
    # weight gradient of the down-projection: K = tokens (padded to Np with zero codes)
    dwp = empty((C, F), torch.float32, fill=float("nan"))
    ws = torch.empty(max(ops.gemm_fp8_ws_bytes(C, F, Np, ops.EPI_F32), 16), dtype=torch.uint8, device=DEV)
    ops.gemm_fp8(C, F, Np, dqt, Np, am_d, hqt, Np, am_h, ops.EPI_F32, dwp, F, ws=ws)
    torch.cuda.synchronize()
    assert_close(dwp, O.mm_nt(f64(dout).T, f64(h).T, True, dt), "f32", "dw_proj", tol=1e-3)
    # backward through the up-projection, from a seeded du
    uq, uqt, am_u = _quant(du, dt, Np)
    dxn = empty((N, C), dt)
    ops.gemm_fp8(N, C, F, uq, F, am_u, wqt, F, am_w, ops.EPI_STORE, dxn, C)
    torch.cuda.synchronize()
    assert_close(dxn, O.mm_nt(f64(du), f64(w_fc).T, True, dt), dt, "dxn2", tol=out_tol)
    dwf = empty((F, C), torch.float32, fill=float("nan"))
    ws = torch.empty(max(ops.gemm_fp8_ws_bytes(F, C, Np, ops.EPI_F32), 16), dtype=torch.uint8, device=DEV)
    ops.gemm_fp8(F, C, Np, uqt, Np, am_u, xqt, Np, am_x, ops.EPI_F32, dwf, C, ws=ws)
    torch.cuda.synchronize()
    assert_close(dwf, O.mm_nt(f64(du).T, f64(xn2).T, True, dt), "f32", "dw_fc", tol=1e-3)


def _finite_bf16_patterns() -> np.ndarray:
    """Every bfloat16 bit pattern that is finite, as float32 values."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    return f[np.isfinite(f)]


@pytest.mark.parametrize("amax", [448.0, 1.0, 24576.0, float.fromhex("0x1.0p-100"), None])
def test_fp8_quantize_every_bf16_pattern(amax):
    # all finite bf16 values whose magnitude is at most amax, plus amax itself
    # (a bf16 value, so the per-tensor scale is amax / 448: scale 1 at
    # amax = 448); None takes every finite pattern (amax = the largest bf16)
    v = _finite_bf16_patterns()
    if amax is not None:
        v = np.concatenate([v[np.abs(v) <= amax], [amax]]).astype(np.float32)
    pad = (-v.size) % 64
    x = np.concatenate([v, np.zeros(pad, dtype=np.float32)]).reshape(-1, 64)
    print(f"fp8 quantize exhaustive amax={amax} values={v.size}", flush=True)
    _quant(x, "bf16", (x.shape[0] + 15) // 16 * 16)


# ------------------------------------------------------------- reductions
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("N,C", [(130, 1664), (4099, 128)])
def test_mix_stage(dt, N, C):
    # residual mixing forward and backward on seeded rows: the two scalar
    # gradients are fixed-order fp32 sums of N*C products, held to the plain bar
    g = np.random.default_rng(N + C)
    x, x0, dy = (rounded(g.standard_normal((N, C)), dt) for _ in range(3))
    a, b = 1.3, 0.7
    lam = torch.tensor([a, b], dtype=torch.float32, device=DEV)
    y = empty((N, C), dt)
    ops.mix_fwd(dev(x, dt), dev(x0, dt), lam, y)
    dx, dx0, dlam = empty((N, C), dt), torch.full((N, C), 0.25, device=DEV), empty((2,), torch.float32, fill=1.0)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    ops.mix_bwd(dev(dy, dt), dev(x, dt), dev(x0, dt), lam, dx, dx0, dlam, ws, accumulate_dx0=True,
                accumulate=True)
    torch.cuda.synchronize()
    f = lambda t: np.asarray(t, dtype=np.float64)
    assert_close(y, O.mix_forward(f(x), f(x0), a, b), dt, "y")
    r = O.mix_backward(f(dy), f(x), f(x0), a, b)
    assert_close(dx, r["dx"], dt, "dx")
    assert_close(dx0, 0.25 + r["dx0"], "f32", "dx0", tol=1e-6)
    e = assert_close(dlam, [1.0 + r["da"], 1.0 + r["db"]], dt, "dlam")
    # the sums themselves, against fp64: fp32 accumulation only
    d = host(dlam) - 1.0
    for k, i in (("da", 0), ("db", 1)):
        assert abs(d[i] - r[k]) <= 1e-6 * r["sum_abs"][k], (k, d[i], r[k])
    print(f"mix stage dt={dt} N={N} C={C} dlam err {e:.2e}", flush=True)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("deterministic", [False, True])
@pytest.mark.parametrize("Hkv,nc", [(13, 32), (40, 64), (3, 5), (20, 12)])
def test_value_embedding_stage(dt, deterministic, Hkv, nc):
    # d26-like heads (13 K/V heads of 128), 32 gate channels, repeated ids; the
    # other head/channel counts take every lanes-per-head split of the gate
    # logits (8, 1, 2 lanes per head) and several passes over the heads
    N, D, V = 300, 128, 97
    C, KV = 1664, Hkv * 128
    ld = C + 2 * KV
    voff = C + KV
    g = np.random.default_rng(7 + int(deterministic))
    qkv = rounded(g.standard_normal((N, ld)), dt)
    xn = rounded(g.standard_normal((N, C)), dt)
    ve = rounded(g.standard_normal((V, KV)) * 0.5, dt)
    wg = rounded(g.standard_normal((Hkv, nc)) * 0.2, dt)
    ids = g.integers(0, V, size=N).astype(np.int32)
    ids[:40] = 5                                         # one id repeated many times
    dqkv = rounded(g.standard_normal((N, ld)) * 0.1, dt)
    dxn0 = rounded(g.standard_normal((N, C)) * 0.1, dt)
    qg, idg = dev(qkv, dt), torch.from_numpy(ids).to(DEV)
    s_save = empty((N, Hkv), torch.float32)
    ops.ve_fwd(Hkv, D, qg, voff, dev(xn, dt), idg, dev(ve, dt), dev(wg, dt), s_save)
    dve = empty((V, KV), torch.float32, fill=3.0)
    dwg = empty((Hkv, nc), torch.float32, fill=3.0)
    dxn = dev(dxn0, dt)
    ws = torch.empty(ops.ve_bwd_ws_bytes(N, Hkv, nc, deterministic), dtype=torch.uint8, device=DEV)
    ops.ve_bwd(Hkv, D, dev(dqkv, dt), voff, idg, dev(ve, dt), s_save, dev(xn, dt), dxn, dev(wg, dt), dve, dwg, ws,
               accumulate=False, deterministic=deterministic)
    torch.cuda.synchronize()
    f = lambda a: np.asarray(a, dtype=np.float64)
    v = f(qkv[:, voff:]).reshape(1, N, Hkv, D)
    v2, c = O.ve_forward(f(xn).reshape(1, N, C), v, ids.reshape(1, N), f(ve), f(wg))
    ref_q = f(qkv).copy()
    ref_q[:, voff:] = v2.reshape(N, KV)
    assert_close(qg, ref_q, dt, "qkv (v updated)")
    assert_close(s_save, c["ve_s"].reshape(N, Hkv), "f32", "gate logits", tol=1e-5)
    r = O.ve_backward(f(dqkv[:, voff:]).reshape(1, N, Hkv, D), f(xn).reshape(1, N, C), ids.reshape(1, N), f(wg),
                      V, c)
    e1 = assert_close(dve, r["dve"], dt, "dve")
    e2 = assert_close(dwg, r["dwg"], dt, "dve_gate")
    e3 = assert_close(dxn, f(dxn0) + r["dxn"].reshape(N, C), dt, "dxn")
    print(f"ve stage dt={dt} det={deterministic} Hkv={Hkv} nc={nc} errs dve {e1:.2e} dwg {e2:.2e} dxn {e3:.2e}",
          flush=True)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_smear_and_backout_stages(dt):
    w = workload("d26")
    B, T, C, ng = 3, 77, w.C, w.smear_channels
    N = B * T
    g = np.random.default_rng(17)
    e = rounded(g.standard_normal((N, C)), dt)
    ws_ = rounded(g.standard_normal(ng) * 0.3, dt)
    dx = rounded(g.standard_normal((N, C)) * 0.1, dt)
    dxa = (g.standard_normal((N, C)) * 0.05).astype(np.float32)
    lam = 0.8
    lg = torch.tensor([lam], dtype=torch.float32, device=DEV)
    x, s_save = empty((N, C), dt), empty((N,), torch.float32)
    ops.smear_fwd(B, T, dev(e, dt), dev(ws_, dt), lg, x, s_save)
    de = empty((N, C), dt)
    dlam, dw = empty((1,), torch.float32), empty((ng,), torch.float32)
    wsx = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    ops.smear_bwd(B, T, dev(e, dt), dev(ws_, dt), lg, s_save, dev(dx, dt), torch.from_numpy(dxa).to(DEV), de, dlam,
                  dw, wsx)
    torch.cuda.synchronize()
    f = lambda a: np.asarray(a, dtype=np.float64)
    xr, c = O.smear_forward(f(e).reshape(B, T, C), f(ws_), lam)
    assert_close(x, xr.reshape(N, C), dt, "smear x")
    der, dwr, dlr = O.smear_backward((f(dx) + f(dxa)).reshape(B, T, C), f(e).reshape(B, T, C), f(ws_), lam, c)
    assert_close(de, der.reshape(N, C), dt, "smear de")
    assert_close(dw, dwr, dt, "smear dw")
    assert_close(dlam, [dlr], dt, "smear dlam")
    # backout
    xb = rounded(g.standard_normal((N, C)), dt)
    dy = rounded(g.standard_normal((N, C)) * 0.1, dt)
    dxb0 = rounded(g.standard_normal((N, C)) * 0.1, dt)
    y = empty((N, C), dt)
    ops.backout_fwd(dev(e, dt), dev(xb, dt), lg, y)
    dxb, dl = dev(dxb0, dt), empty((1,), torch.float32)
    ops.backout_bwd(dev(dy, dt), dev(xb, dt), lg, dxb, dl, wsx)
    torch.cuda.synchronize()
    assert_close(y, O.backout_forward(f(e), f(xb), lam), dt, "backout y")
    rb = O.backout_backward(f(dy), f(xb), lam)
    assert_close(dxb, f(dxb0) + rb["dx_bo"], dt, "backout dx_bo")
    assert_close(dl, [rb["dlam"]], dt, "backout dlam")


# ------------------------------------------------------ deterministic mode
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("N,V,C", [(4096, 32768, 1536), (1000, 700, 128), (70000, 300, 64)])
def test_embed_bwd_deterministic(dt, N, V, C):
    # Zipf-distributed ids (a few ids take a large share of the tokens): the
    # fixed-order path gives the same bits on every call and matches the oracle
    w = workload("d24").with_(B=1, T=N - 1, vocab=V)
    ids = draw_ids_zipf(w).reshape(-1)[:N].astype(np.int32)
    g = np.random.default_rng(N)
    dx = rounded(g.standard_normal((N, C)), dt)
    idg, dxg = torch.from_numpy(ids).to(DEV), dev(dx, dt)
    ws = torch.empty(max(ops.embed_bwd_ws_bytes(N, True), 16), dtype=torch.uint8, device=DEV)
    outs = []
    for rep in range(3):
        dw = empty((V, C), torch.float32, fill=float(rep))
        ops.embed_bwd(idg, dxg, dw, ws=ws)
        outs.append(dw)
    acc = empty((V, C), torch.float32, fill=0.5)
    ops.embed_bwd(idg, dxg, acc, accumulate=True, ws=ws)
    torch.cuda.synchronize()
    print(f"embed bwd deterministic dt={dt} N={N} V={V} top id share {np.bincount(ids).max() / N:.3f}", flush=True)
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    ref = O.embed_backward(dx.astype(np.float64), ids, V)
    # fp32 sums of up to ~10^4 rows per id (the Zipf head): the fp32 bar
    assert_close(outs[0], ref, "f32", "dwte")
    assert_close(acc, ref + 0.5, "f32", "dwte accumulate")


def test_block_bwd_deterministic_bitwise():
    # a d26-width block with value embedding and mixing, backward twice with
    # deterministic = 1 (and repeated ids): every output the same bits
    w = workload("d26").with_(n_layer=2, windows=(-1, -1), vocab=64, mlp_fp8=False)
    B, T, l = 1, 200, 1
    dt = w.dtype
    N, C, KV = B * T, w.C, w.n_kv_head * w.head_dim
    from seeded_inputs import draw_layer
    p = {k: (rounded(v, dt) if np.ndim(v) else np.float32(v)) for k, v in draw_layer(w, l).items()}
    x = rounded(draw_upstream(w, 100, (N, C), 1.0), dt)
    x0 = rounded(draw_upstream(w, 150, (N, C), 1.0), dt)
    dy = rounded(draw_upstream(w, 200, (N, C), 1.0), dt)
    ids = np.random.default_rng(3).integers(0, 8, size=N).astype(np.int32)   # heavy repetition
    cfg = ops.make_cfg(B, T, C, w.n_head, w.n_kv_head, w.head_dim, w.mlp_hidden, -1, TDT[dt], w.eps,
                       deterministic=True)
    sv, wf, wb = ops.block_sizes(cfg)
    saved = torch.empty(sv, dtype=torch.uint8, device=DEV)
    wsf, wsb = torch.empty(wf, dtype=torch.uint8, device=DEV), torch.empty(wb, dtype=torch.uint8, device=DEV)
    W = [dev(p[k], dt) for k in ("w_qkv", "w_o", "w_fc", "w_proj")]
    rope = ops.rope_table(T, w.head_dim, w.rope_base, DEV)
    lam = torch.tensor([p["resid_lambda"], p["x0_lambda"]], dtype=torch.float32, device=DEV)
    xg, x0g, idg = dev(x, dt), dev(x0, dt), torch.from_numpy(ids).to(DEV)
    veg, vgg = dev(p["ve"], dt), dev(p["ve_gate"], dt)      # kept alive: the extras hold raw pointers
    ex = ops.block_extras(lam, x0g, xg, idg, veg, vgg)
    out = empty((N, C), dt)
    ops.block_fwd(cfg, W, rope, xg, out, saved, wsf, ex)
    runs = []
    for rep in range(2):
        dW = [empty(t.shape, torch.float32) for t in W]
        dlam, dx0 = empty((2,), torch.float32), empty((N, C), torch.float32)
        dve, dvg = empty((w.vocab, KV), torch.float32, fill=9.0), empty((w.n_kv_head, w.ve_gate_channels),
                                                                           torch.float32)
        dx = dev(dy, dt)
        ops.block_bwd(cfg, W, rope, saved, dx, dx, dW, wsb, ex, ops.block_extras_grads(dlam, dx0, dve, dvg))
        runs.append([dx, dlam, dx0, dve, dvg] + dW)
    torch.cuda.synchronize()
    for a, b in zip(*runs):
        assert torch.equal(a, b)
    # and the fixed-order table gradient is the oracle's
    cos, sin = O.rope_tables(T, w.head_dim, w.rope_base)
    pp = {k: np.asarray(v, dtype=np.float64) for k, v in p.items()}
    _, c = O.block_forward(x.astype(np.float64).reshape(B, T, C), pp, w, l, cos, sin,
                           x0=x0.astype(np.float64).reshape(B, T, C), ids=ids.reshape(B, T))
    _, gr = O.block_backward(dy.astype(np.float64).reshape(B, T, C), c, pp, w, l, cos, sin, ids=ids.reshape(B, T))
    assert_close(runs[0][3], gr["ve"], dt, "dve")
