"""Parity of each HIP building block (through the C ABI) with the CPU oracle,
element by element, at sizes that span several tiles and a ragged tail."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from gpt_decoder_block_amd import _lib as L, ops
from gpu_util import DEV, TDT, TOL, assert_close, dev, empty, host, rounded

pytestmark = pytest.mark.gpu
RNG = np.random.default_rng(777)


# ------------------------------------------------------------------ RMSNorm
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("N,C", [(37, 1536), (5, 128), (64, 4096), (1, 1664)])
def test_rmsnorm(dt, N, C):
    print(f"rmsnorm dt={dt} N={N} C={C}", flush=True)
    x = rounded(RNG.standard_normal((N, C)) * 3.0, dt)
    dy = rounded(RNG.standard_normal((N, C)), dt)
    dres = rounded(RNG.standard_normal((N, C)), dt)
    xg, dyg, dresg = dev(x, dt), dev(dy, dt), dev(dres, dt)
    xn, r = empty((N, C), dt), empty((N,), torch.float32)
    ops.rmsnorm_fwd(xg, xn, r, 1e-6)
    y_ref, r_ref = O.rms_norm(x.astype(np.float64), 1e-6)
    assert_close(xn, y_ref, dt, "xn")
    assert_close(r, r_ref, "f32", "r", tol=1e-5)
    dx = empty((N, C), dt)
    ops.rmsnorm_bwd(dyg, xn, r, dresg, dx)
    ref = O.rms_norm_backward(dy.astype(np.float64), y_ref, r_ref) + dres
    assert_close(dx, ref, dt, "dx")
    ops.rmsnorm_bwd(dyg, xn, r, None, dx)
    assert_close(dx, O.rms_norm_backward(dy.astype(np.float64), y_ref, r_ref), dt, "dx (no residual)")


# --------------------------------------------------------------------- GEMM
def _store(Mat, kmajor):
    """Mat [rows, K] stored K-major ([rows, K]) or rows-major ([K, rows])."""
    return np.ascontiguousarray(Mat if kmajor else Mat.T)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("ak,bk", [(True, True), (True, False), (False, False), (False, True)])
@pytest.mark.parametrize("epi", [0, 1, 2, 3, 4])
def test_gemm(dt, ak, bk, epi):
    M, N, K = 296, 264, 200
    print(f"gemm dt={dt} ak={ak} bk={bk} epi={epi} M={M} N={N} K={K}", flush=True)
    A = rounded(RNG.standard_normal((M, K)), dt)
    B = rounded(RNG.standard_normal((N, K)), dt)
    R = rounded(RNG.standard_normal((M, N)), dt)
    acc = A.astype(np.float64) @ B.astype(np.float64).T
    Ag, Bg = dev(_store(A, ak), dt), dev(_store(B, bk), dt)
    lda, ldb = (K if ak else M), (K if bk else N)
    if epi == 4:
        for accumulate in (False, True):
            C0 = RNG.standard_normal((M, N)).astype(np.float32)
            C = torch.from_numpy(C0).to(DEV)
            ws = empty((max(1, ops.gemm_ws_bytes(TDT[dt], M, N, K, 4) // 4),), torch.float32)
            ops.gemm(M, N, K, Ag, ak, lda, Bg, bk, ldb, 4, C, N, accumulate=accumulate, ws=ws)
            assert_close(C, acc + (C0 if accumulate else 0.0), "f32", f"fp32 out acc={accumulate}",
                         tol=1e-5 if dt == "f32" else 1e-5)
        return
    C = empty((M, N), dt)
    C2 = empty((M, N), dt)
    Rg = dev(R, dt)
    ops.gemm(M, N, K, Ag, ak, lda, Bg, bk, ldb, epi, C, N, R=Rg if epi in (1, 3) else None, ldr=N,
             C2=C2 if epi == 2 else None)
    if epi == 0:
        assert_close(C, acc, dt, "store")
    elif epi == 1:
        assert_close(C, R + acc, dt, "residual")
    elif epi == 2:
        assert_close(C, acc, dt, "u")
        assert_close(C2, np.maximum(acc, 0) ** 2, dt, "relu2")
    elif epi == 3:
        assert_close(C, acc * 2.0 * np.maximum(R, 0), dt, "relu2 backward")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("ak,bk", [(True, True), (True, False)])
def test_gemm_square_epilogues(dt, ak, bk):
    # epi 6: h = relu(acc)^2 alone; epi 7: acc * 2*sqrt(h) with h saved by 6
    M, N, K = 296, 264, 200
    A = rounded(RNG.standard_normal((M, K)), dt)
    B = rounded(RNG.standard_normal((N, K)), dt)
    acc = A.astype(np.float64) @ B.astype(np.float64).T
    Ag, Bg = dev(_store(A, ak), dt), dev(_store(B, bk), dt)
    lda, ldb = (K if ak else M), (K if bk else N)
    H = rounded(np.maximum(RNG.standard_normal((M, N)), 0) ** 2, dt)
    C = empty((M, N), dt)
    if ak and bk:
        ops.gemm(M, N, K, Ag, ak, lda, Bg, bk, ldb, ops.EPI_SQR, C, N)
        assert_close(C, np.maximum(acc, 0) ** 2, dt, "relu(acc)^2")
    ops.gemm(M, N, K, Ag, ak, lda, Bg, bk, ldb, ops.EPI_DSQR, C, N, R=dev(H, dt), ldr=N)
    assert_close(C, acc * 2.0 * np.sqrt(H), dt, "acc * 2 sqrt(h)")


def test_gemm_square_epilogue_layout_rules():
    # bf16 epi 6 needs both operands K-major, epi 7 a K-major A; 5 is refused
    a = empty((64, 64), "bf16", fill=0.0)
    c = empty((64, 64), "bf16")
    with pytest.raises(L.GdbError, match="epilogue 6"):
        ops.gemm(64, 64, 64, a, True, 64, a, False, 64, ops.EPI_SQR, c, 64)
    with pytest.raises(L.GdbError, match="epilogue 7"):
        ops.gemm(64, 64, 64, a, False, 64, a, True, 64, ops.EPI_DSQR, c, 64, R=c, ldr=64)
    with pytest.raises(L.GdbError, match="unknown epilogue 5"):
        ops.gemm(64, 64, 64, a, True, 64, a, True, 64, 5, c, 64)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_gemm_splitk_large_k(dt):
    # weight-gradient shape: small output, long token contraction -> split-K
    M, N, K = 296, 264, 8192
    A = rounded(RNG.standard_normal((K, M)), dt)   # token-major operands
    B = rounded(RNG.standard_normal((K, N)), dt)
    ws_b = ops.gemm_ws_bytes(TDT[dt], M, N, K, 4)
    if dt == "bf16":
        assert ws_b > 0, "expected split-K for this shape"
    ws = empty((max(1, ws_b // 4),), torch.float32)
    C = empty((M, N), torch.float32)
    ops.gemm(M, N, K, dev(A, dt), False, M, dev(B, dt), False, N, 4, C, N, ws=ws)
    assert_close(C, A.astype(np.float64).T @ B.astype(np.float64), "f32", "split-K", tol=1e-5)


@pytest.mark.parametrize("M,N,K,accumulate", [(1528, 6136, 32704, False), (6136, 1528, 32704, True),
                                               (4600, 1528, 32704, False)])
def test_gemm_bf16_two_phase_splitk(M, N, K, accumulate):
    # weight-gradient shapes (token-major operands, long K) whose split-K plan
    # has two phases: bands of tile columns, of tile rows and a third split
    # pair; ragged M and N, the fp32 output accumulated onto a prior value in
    # one case
    print(f"gemm two-phase split-K M={M} N={N} K={K} accumulate={accumulate}", flush=True)
    g = np.random.default_rng(2024)
    A = rounded(g.standard_normal((K, M), dtype=np.float32), "bf16")
    B = rounded(g.standard_normal((K, N), dtype=np.float32), "bf16")
    ws = empty((max(1, ops.gemm_ws_bytes(TDT["bf16"], M, N, K, 4) // 4),), torch.float32)
    C0 = g.standard_normal((M, N), dtype=np.float32)
    C = torch.from_numpy(C0).to(DEV)
    ops.gemm(M, N, K, dev(A, "bf16"), False, M, dev(B, "bf16"), False, N, 4, C, N, accumulate=accumulate, ws=ws)
    ref = A.astype(np.float64).T @ B.astype(np.float64)
    if accumulate:
        ref += C0
    assert_close(C, ref, "f32", "two-phase split-K", tol=1e-5)


def test_gemm_bf16_multi_tile_exact_shapes():
    # full 256x256 tiles plus XCD remap over many tiles
    M, N, K = 1024, 2048, 768
    A = rounded(RNG.standard_normal((M, K)), "bf16")
    B = rounded(RNG.standard_normal((N, K)), "bf16")
    C = empty((M, N), "bf16")
    ops.gemm(M, N, K, dev(A, "bf16"), True, K, dev(B, "bf16"), True, K, 0, C, N)
    assert_close(C, A.astype(np.float64) @ B.astype(np.float64).T, "bf16", "store")


@pytest.mark.parametrize("epi", [0, 1, 2, 3, 4, 6, 7])
@pytest.mark.parametrize("M,N,K", [(296, 264, 384), (520, 776, 1024)])
def test_gemm_bf16_kmajor_epilogues(epi, M, N, K):
    # both operands K-contiguous with K a multiple of 128 (the shape class of
    # every block product; also the one the ring-fed kernel variant accepts):
    # ragged M and N over several tiles, 6 or 16 K steps, every epilogue
    print(f"gemm kmajor epi={epi} M={M} N={N} K={K}", flush=True)
    A = rounded(RNG.standard_normal((M, K)), "bf16")
    B = rounded(RNG.standard_normal((N, K)), "bf16")
    R = rounded(RNG.standard_normal((M, N)), "bf16")
    acc = A.astype(np.float64) @ B.astype(np.float64).T
    Ag, Bg = dev(A, "bf16"), dev(B, "bf16")
    if epi == 4:
        C0 = RNG.standard_normal((M, N)).astype(np.float32)
        C = torch.from_numpy(C0).to(DEV)
        ws = empty((max(1, ops.gemm_ws_bytes(TDT["bf16"], M, N, K, 4) // 4),), torch.float32)
        ops.gemm(M, N, K, Ag, True, K, Bg, True, K, 4, C, N, accumulate=True, ws=ws)
        assert_close(C, acc + C0, "f32", "fp32 out", tol=1e-5)
        return
    C, C2 = empty((M, N), "bf16"), empty((M, N), "bf16")
    H = rounded(np.maximum(R, 0) ** 2, "bf16")
    Rg = dev(H if epi == 7 else R, "bf16")
    ops.gemm(M, N, K, Ag, True, K, Bg, True, K, epi, C, N, R=Rg if epi in (1, 3, 7) else None, ldr=N,
             C2=C2 if epi == 2 else None)
    want = {0: acc, 1: R + acc, 2: acc, 3: acc * 2.0 * np.maximum(R, 0), 6: np.maximum(acc, 0) ** 2,
            7: acc * 2.0 * np.sqrt(H)}[epi]
    assert_close(C, want, "bf16", f"epilogue {epi}")
    if epi == 2:
        assert_close(C2, np.maximum(acc, 0) ** 2, "bf16", "relu2")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_gemm_token_major_strided(dt):
    # both operands M/N-contiguous (the weight-gradient layout) with leading
    # dimensions wider than the rows, several tiles and a ragged K tail
    M, N, K, lda, ldb = 520, 776, 1000, 528, 800
    A = rounded(RNG.standard_normal((K, lda)), dt)
    B = rounded(RNG.standard_normal((K, ldb)), dt)
    ref = A[:, :M].astype(np.float64).T @ B[:, :N].astype(np.float64)
    print(f"gemm token-major dt={dt} M={M} N={N} K={K} lda={lda} ldb={ldb}", flush=True)
    ws = empty((max(1, ops.gemm_ws_bytes(TDT[dt], M, N, K, 4) // 4),), torch.float32)
    C = empty((M, N), torch.float32)
    ops.gemm(M, N, K, dev(A, dt), False, lda, dev(B, dt), False, ldb, 4, C, N, ws=ws)
    assert_close(C, ref, "f32", "fp32 out", tol=1e-5)
    Cb = empty((M, N), dt)
    ops.gemm(M, N, K, dev(A, dt), False, lda, dev(B, dt), False, ldb, 0, Cb, N)
    assert_close(Cb, ref, dt, "store")


# ---------------------------------------------------------------- attention
def _attn_case(dt, B, T, H, Hkv, D, window, qk_normed=False):
    W3 = (H + 2 * Hkv) * D
    raw = RNG.standard_normal((B * T, W3))
    if qk_normed:
        # q and k heads with unit RMS, as the QK RMS-norm produces
        qk = raw[:, :(H + Hkv) * D].reshape(B * T, H + Hkv, D)
        qk = qk / np.sqrt(np.mean(qk ** 2, axis=-1, keepdims=True))
        raw[:, :(H + Hkv) * D] = qk.reshape(B * T, -1)
    qkv = rounded(raw, dt)
    q = qkv[:, :H * D].reshape(B, T, H, D).astype(np.float64)
    k = qkv[:, H * D:(H + Hkv) * D].reshape(B, T, Hkv, D).astype(np.float64)
    v = qkv[:, (H + Hkv) * D:].reshape(B, T, Hkv, D).astype(np.float64)
    qkvg = dev(qkv, dt)
    o = empty((B * T, H * D), dt)
    lse = empty((B, H, T), torch.float32)
    ops.attention_fwd(B, T, H, Hkv, D, window, qkvg, W3, o, H * D, lse, qk_normed=qk_normed)
    o_ref, P = O.attention(q, k, v, window)
    assert_close(o, o_ref.reshape(B * T, H * D), dt, "o")
    # bf16: lse is the log of the sum of the bf16-rounded weights that also
    # normalise O, so it carries bf16 rounding; fp32: plain fp32 sums
    assert_close(lse, O.attention_logsumexp(q, k, window), "f32", "lse", tol=2e-2 if dt == "bf16" else 1e-5)
    do = rounded(RNG.standard_normal((B * T, H * D)), dt)
    dqkv = empty((B * T, W3), dt, fill=0.0)
    delta = empty((B, H, T), torch.float32)
    ops.attention_bwd(B, T, H, Hkv, D, window, qkvg, W3, o, H * D, lse, dev(do, dt), H * D, dqkv, W3, delta)
    dq, dk, dv = O.attention_backward(do.reshape(B, T, H, D).astype(np.float64), q, k, v, P)
    g = host(dqkv)
    dq_g = g[:, :H * D]
    dk_g = g[:, H * D:(H + Hkv) * D]
    dv_g = g[:, (H + Hkv) * D:]
    assert_close(dq_g, dq.reshape(B * T, -1), dt, "dq")
    assert_close(dk_g, dk.reshape(B * T, -1), dt, "dk")
    assert_close(dv_g, dv.reshape(B * T, -1), dt, "dv")


@pytest.mark.parametrize("qk_normed", [False, True])
@pytest.mark.parametrize("window", [-1, 0, 1, 63, 64, 70, 199, 1000])
def test_attention_bf16_gqa_windows(window, qk_normed):
    print(f"attention bf16 B=2 T=200 H=6 Hkv=2 window={window} qk_normed={qk_normed}", flush=True)
    _attn_case("bf16", 2, 200, 6, 2, 128, window, qk_normed)


@pytest.mark.parametrize("qk_normed", [False, True])
@pytest.mark.parametrize("B,T,H,Hkv,window", [(1, 1, 2, 2, -1), (1, 64, 2, 1, -1), (1, 130, 2, 2, -1),
                                              (1, 384, 3, 1, -1), (1, 640, 2, 1, 300), (2, 333, 4, 4, 65)])
def test_attention_bf16_shapes(B, T, H, Hkv, window, qk_normed):
    print(f"attention bf16 B={B} T={T} H={H} Hkv={Hkv} window={window} qk_normed={qk_normed}", flush=True)
    _attn_case("bf16", B, T, H, Hkv, 128, window, qk_normed)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("window", [-1, 0, 5])
def test_attention_f32(D, window):
    print(f"attention f32 D={D} window={window}", flush=True)
    _attn_case("f32", 2, 50, 4, 2, D, window)


# ------------------------------------------------------------ QK norm + RoPE
@pytest.mark.parametrize("dt,D", [("f32", 64), ("f32", 128), ("bf16", 128)])
def test_qk_norm_rope(dt, D):
    B, T, H, Hkv = 2, 70, 6, 2
    print(f"qk_norm_rope dt={dt} D={D}", flush=True)
    W3 = (H + 2 * Hkv) * D
    qkv = rounded(RNG.standard_normal((B * T, W3)) * RNG.uniform(0.1, 3.0, size=(1, W3)), dt)
    rope = ops.rope_table(T, D, 10000.0, DEV)
    out = empty((B * T, W3), dt)
    rinv = empty((B * T, H + Hkv), torch.float32)
    ops.qk_norm_rope_fwd(B, T, H, Hkv, D, dev(qkv, dt), out, rinv, rope, 1e-6)
    cos, sin = O.rope_tables(T, D, 10000.0)
    x = qkv.astype(np.float64)
    q = x[:, :H * D].reshape(B, T, H, D)
    k = x[:, H * D:(H + Hkv) * D].reshape(B, T, Hkv, D)
    qn, rq = O.rms_norm(q, 1e-6)
    kn, rk = O.rms_norm(k, 1e-6)
    qh, kh = O.rope(qn, cos, sin), O.rope(kn, cos, sin)
    g = host(out)
    assert_close(g[:, :H * D], qh.reshape(B * T, -1), dt, "q^")
    assert_close(g[:, H * D:(H + Hkv) * D], kh.reshape(B * T, -1), dt, "k^")
    np.testing.assert_array_equal(g[:, (H + Hkv) * D:], x[:, (H + Hkv) * D:])
    r_ref = np.concatenate([rq.reshape(B * T, H), rk.reshape(B * T, Hkv)], 1)
    assert_close(rinv, r_ref, "f32", "rinv", tol=1e-5)
    d = rounded(RNG.standard_normal((B * T, W3)), dt)
    dg = dev(d, dt)
    ops.qk_norm_rope_bwd(B, T, H, Hkv, D, dg, out, rinv, rope)
    dd = d.astype(np.float64)
    dq = O.rms_norm_backward(O.rope_backward(dd[:, :H * D].reshape(B, T, H, D), cos, sin), qn, rq)
    dk = O.rms_norm_backward(O.rope_backward(dd[:, H * D:(H + Hkv) * D].reshape(B, T, Hkv, D), cos, sin), kn, rk)
    g = host(dg)
    assert_close(g[:, :H * D], dq.reshape(B * T, -1), dt, "dq")
    assert_close(g[:, H * D:(H + Hkv) * D], dk.reshape(B * T, -1), dt, "dk")
    np.testing.assert_array_equal(g[:, (H + Hkv) * D:], dd[:, (H + Hkv) * D:])


# ------------------------------------------------------------ cross-entropy
@pytest.mark.parametrize("dt,N,V", [("bf16", 37, 32768), ("f32", 64, 512), ("bf16", 5, 40000), ("f32", 3, 32768)])
def test_cross_entropy(dt, N, V):
    print(f"cross_entropy dt={dt} N={N} V={V}", flush=True)
    z = rounded(RNG.standard_normal((N, V)) * 2.0, dt)
    y = RNG.integers(0, V, size=N)
    zg = dev(z, dt)
    tg = torch.from_numpy(y.astype(np.int32)).to(DEV)
    row = empty((N,), torch.float32)
    loss = empty((1,), torch.float32)
    ops.cross_entropy(zg, tg, row, loss)
    l_ref, row_ref, dz_ref, _ = O.cross_entropy(z.astype(np.float64), y)
    assert_close(row, row_ref, "f32", "row loss", tol=1e-5)
    assert abs(float(loss.item()) - l_ref) <= 1e-5 * abs(l_ref)
    assert_close(zg, dz_ref, dt, "dz")


# ---------------------------------------------------------------- embedding
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_embedding(dt):
    N, C, V = 300, 136, 50   # many duplicate ids
    ids = RNG.integers(0, V, size=N)
    wte = rounded(RNG.standard_normal((V, C)), dt)
    idg = torch.from_numpy(ids.astype(np.int32)).to(DEV)
    x = empty((N, C), dt)
    ops.embed_fwd(idg, dev(wte, dt), x)
    np.testing.assert_array_equal(host(x), O.embed_forward(wte.astype(np.float64), ids))
    dx = rounded(RNG.standard_normal((N, C)), dt)
    dw = empty((V, C), torch.float32, fill=float("nan"))
    ops.embed_bwd(idg, dev(dx, dt), dw)
    assert_close(dw, O.embed_backward(dx.astype(np.float64), ids, V), "f32", "dwte", tol=1e-6)
    ops.embed_bwd(idg, dev(dx, dt), dw, accumulate=True)
    assert_close(dw, 2 * O.embed_backward(dx.astype(np.float64), ids, V), "f32", "dwte accumulate", tol=1e-6)


# ---------------------------------------------------------------------- fp8
def _e4m3_values(codes: torch.Tensor) -> np.ndarray:
    """uint8 e4m3fn codes -> float64 values (torch's own e4m3fn decode, on the host)."""
    return codes.cpu().view(torch.float8_e4m3fn).to(torch.float64).numpy()


@pytest.mark.parametrize("R,Cc,Rp,scale", [(130, 96, 144, 1.0), (64, 64, 64, 1e-3), (1, 16, 16, 300.0),
                                            (300, 1664, 304, 1.0), (30001, 1040, 30016, 1.0)])
def test_fp8_quantize_codes_exact(R, Cc, Rp, scale):
    # the codes are integer work: bit-exact against the oracle's float32 decisions;
    # the last shape takes the 128-column tiles (at least 2048 of them), with a
    # partial last column tile and padded transposed rows
    print(f"fp8 quantize R={R} Cc={Cc} Rp={Rp}", flush=True)
    x = rounded(RNG.standard_normal((R, Cc)) * scale, "bf16")
    x[0, :3] = [0.0, -0.0, x[0, 3]]      # zeros and a repeated value
    xg = dev(x, "bf16")
    amax = empty((1,), torch.float32, fill=-5.0)
    xq = torch.full((R, Cc), 0xAA, dtype=torch.uint8, device=DEV)
    xqt = torch.full((Cc, Rp), 0xAA, dtype=torch.uint8, device=DEV)
    ops.fp8_quantize(xg, amax, xq, xqt, Rp)
    torch.cuda.synchronize()
    q_ref, s_ref = O.fp8_quantize(x.astype(np.float64))
    assert float(host(amax)[0]) == float(np.max(np.abs(x)))
    assert float(host(amax)[0]) / 448.0 == pytest.approx(s_ref, rel=1e-7)
    np.testing.assert_array_equal(_e4m3_values(xq), q_ref)
    qt = _e4m3_values(xqt)
    np.testing.assert_array_equal(qt[:, :R], q_ref.T)
    assert not np.any(qt[:, R:])


def test_fp8_quantize_zero_tensor():
    x = torch.zeros((32, 32), dtype=torch.bfloat16, device=DEV)
    amax = empty((1,), torch.float32, fill=3.0)
    xq = torch.full((32, 32), 7, dtype=torch.uint8, device=DEV)
    ops.fp8_quantize(x, amax, xq)
    torch.cuda.synchronize()
    assert host(amax)[0] == 0.0 and not torch.any(xq).item()


@pytest.mark.parametrize("epi", [0, 1, 2, 3, 4, 6, 7])
@pytest.mark.parametrize("M,N,K", [(300, 264, 160), (64, 520, 1664), (2100, 72, 48), (256, 248, 4096)])
def test_gemm_fp8(epi, M, N, K):
    # C = q8(A) q8(B)^T with each operand's own per-tensor scale; both sides
    # quantise the same bf16 inputs, so the codes agree and only the fp32
    # accumulation order (and the bf16 output) differ
    print(f"gemm fp8 epi={epi} M={M} N={N} K={K}", flush=True)
    a = rounded(RNG.standard_normal((M, K)), "bf16")
    b = rounded(RNG.standard_normal((N, K)) * 0.05, "bf16")
    r = rounded(RNG.standard_normal((M, N)), "bf16")
    amax_a, amax_b = empty((1,), torch.float32), empty((1,), torch.float32)
    aq = torch.empty((M, K), dtype=torch.uint8, device=DEV)
    bq = torch.empty((N, K), dtype=torch.uint8, device=DEV)
    ops.fp8_quantize(dev(a, "bf16"), amax_a, aq)
    ops.fp8_quantize(dev(b, "bf16"), amax_b, bq)
    acc = O.fp8_quant_dequant(a.astype(np.float64)) @ O.fp8_quant_dequant(b.astype(np.float64)).T
    rg = dev(r, "bf16")
    if epi == ops.EPI_F32:
        C = empty((M, N), torch.float32, fill=0.5)
        ws = torch.empty(max(ops.gemm_fp8_ws_bytes(M, N, K, epi), 16), dtype=torch.uint8, device=DEV)
        ops.gemm_fp8(M, N, K, aq, K, amax_a, bq, K, amax_b, epi, C, N, accumulate=True, ws=ws)
        torch.cuda.synchronize()
        assert_close(C, acc + 0.5, "f32", "C", tol=1e-3)
        return
    C = empty((M, N), "bf16")
    C2 = empty((M, N), "bf16")
    ops.gemm_fp8(M, N, K, aq, K, amax_a, bq, K, amax_b, epi, C, N, R=rg, ldr=N, C2=C2)
    torch.cuda.synchronize()
    if epi == ops.EPI_STORE:
        assert_close(C, acc, "bf16", "C")
    elif epi == ops.EPI_RESID:
        assert_close(C, acc + r, "bf16", "C")
    elif epi == ops.EPI_RELU2:
        assert_close(C, acc, "bf16", "u")
        assert_close(C2, np.maximum(acc, 0) ** 2, "bf16", "h")
    elif epi == ops.EPI_SQR:
        assert_close(C, np.maximum(acc, 0) ** 2, "bf16", "h")
    elif epi == ops.EPI_DSQR:
        assert_close(C, acc * 2 * np.sqrt(np.maximum(r, 0)), "bf16", "du")
    else:
        assert_close(C, acc * 2 * np.maximum(r, 0), "bf16", "du")
