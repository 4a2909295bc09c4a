"""Pins of the CPU oracle to facts outside itself: closed forms, invariants,
special cases and finite differences (all float64, CPU only)."""
import math

import numpy as np
import pytest

import oracle as O
from seeded_inputs import Workload

RNG = np.random.default_rng(20260101)


def tiny_cfg(**kw):
    base = dict(name="pin", n_layer=2, B=2, T=6, C=16, n_head=2, n_kv_head=1, head_dim=8,
                mlp_hidden=64, vocab=11, windows=(-1, 2), dtype="f32", seed=7)
    base.update(kw)
    return Workload(**base)


# ------------------------------------------------------------------ RMSNorm
def test_rmsnorm_closed_form():
    x = RNG.standard_normal((5, 37)) * 3.0
    eps = 1e-6
    y, r = O.rms_norm(x, eps)
    ms = np.mean(x ** 2, axis=1)
    # output RMS is sqrt(ms / (ms + eps)); r is exactly the inverse RMS
    np.testing.assert_allclose(np.sqrt(np.mean(y ** 2, axis=1)), np.sqrt(ms / (ms + eps)), rtol=1e-14)
    np.testing.assert_allclose(r, 1.0 / np.sqrt(ms + eps), rtol=1e-14)
    # scale invariance (eps -> 0)
    y1, _ = O.rms_norm(x, 0.0)
    y2, _ = O.rms_norm(7.5 * x, 0.0)
    np.testing.assert_allclose(y1, y2, rtol=1e-13)


def test_rmsnorm_backward_orthogonal_at_eps0():
    # with eps = 0 the norm is scale invariant, so <dx, x> = 0 for any dy
    x = RNG.standard_normal((4, 24))
    dy = RNG.standard_normal((4, 24))
    y, r = O.rms_norm(x, 0.0)
    dx = O.rms_norm_backward(dy, y, r)
    assert np.max(np.abs(np.sum(dx * x, axis=1))) < 1e-12


def fd_check(f, x, dx_analytic, h=1e-6, n_dirs=3, rtol=1e-6):
    for _ in range(n_dirs):
        d = RNG.standard_normal(x.shape)
        num = (f(x + h * d) - f(x - h * d)) / (2 * h)
        ana = float(np.sum(dx_analytic * d))
        assert abs(num - ana) <= rtol * max(1.0, abs(ana)), (num, ana)


def test_rmsnorm_backward_fd():
    x = RNG.standard_normal((3, 10))
    w = RNG.standard_normal((3, 10))
    f = lambda z: float(np.sum(O.rms_norm(z, 1e-6)[0] * w))
    y, r = O.rms_norm(x, 1e-6)
    fd_check(f, x, O.rms_norm_backward(w, y, r))


# --------------------------------------------------------------------- RoPE
def test_rope_preserves_norm_and_identity_at_t0():
    T, H, D = 9, 3, 16
    cos, sin = O.rope_tables(T, D, 10000.0)
    x = RNG.standard_normal((2, T, H, D))
    y = O.rope(x, cos, sin)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    np.testing.assert_allclose(y[:, 0], x[:, 0], rtol=0, atol=0)


def test_rope_relative_position():
    # <R_m q, R_n k> depends only on m - n
    T, D = 40, 16
    cos, sin = O.rope_tables(T, D, 10000.0)
    q = RNG.standard_normal(D)
    k = RNG.standard_normal(D)
    X = np.zeros((1, T, 2, D))
    X[0, :, 0] = q
    X[0, :, 1] = k
    Y = O.rope(X, cos, sin)
    for m, n, s in [(5, 2, 11), (9, 9, 20), (3, 7, 30)]:
        a = Y[0, m, 0] @ Y[0, n, 1]
        b = Y[0, m + s, 0] @ Y[0, n + s, 1]
        assert abs(a - b) < 1e-12


def test_rope_closed_form_basis_vector():
    # rotating e_j at position t gives cos(theta) e_j + sin(theta) e_{j+D/2}
    T, D, base = 7, 8, 10000.0
    cos, sin = O.rope_tables(T, D, base)
    for j in range(D // 2):
        x = np.zeros((1, T, 1, D))
        x[..., j] = 1.0
        y = O.rope(x, cos, sin)
        for t in range(T):
            th = t * base ** (-2.0 * j / D)
            expect = np.zeros(D)
            expect[j] = math.cos(th)
            expect[j + D // 2] = math.sin(th)
            np.testing.assert_allclose(y[0, t, 0], expect, atol=1e-15)


def test_rope_backward_is_inverse():
    T, H, D = 5, 2, 8
    cos, sin = O.rope_tables(T, D, 10000.0)
    x = RNG.standard_normal((1, T, H, D))
    np.testing.assert_allclose(O.rope_backward(O.rope(x, cos, sin), cos, sin), x, atol=1e-14)


def test_rms_and_rope_commute():
    T, H, D = 6, 2, 8
    cos, sin = O.rope_tables(T, D, 10000.0)
    x = RNG.standard_normal((1, T, H, D))
    a = O.rope(O.rms_norm(x, 1e-6)[0], cos, sin)
    b = O.rms_norm(O.rope(x, cos, sin), 1e-6)[0]
    np.testing.assert_allclose(a, b, atol=1e-14)


# ---------------------------------------------------------------- attention
def _qkv(B=2, T=12, H=4, Hkv=2, D=8):
    return (RNG.standard_normal((B, T, H, D)), RNG.standard_normal((B, T, Hkv, D)),
            RNG.standard_normal((B, T, Hkv, D)))


@pytest.mark.parametrize("window", [-1, 0, 1, 3, 11, 40])
def test_softmax_rows_sum_to_one_and_mask(window):
    q, k, v = _qkv()
    T = q.shape[1]
    _, P = O.attention(q, k, v, window)
    np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-14)
    m = O.visible_mask(T, window)
    assert np.all(P[..., ~m] == 0.0)
    assert np.all(P[..., m] > 0.0)
    # the visible set is exactly the keys with 0 <= i - j <= W
    i, j = np.nonzero(m)
    assert np.all(i - j >= 0)
    if window >= 0:
        assert np.all(i - j <= window)
        assert m.sum() == sum(min(t, window) + 1 for t in range(T))


def test_window_zero_gives_v_and_no_qk_grad():
    q, k, v = _qkv()
    o, P = O.attention(q, k, v, 0)
    G = q.shape[2] // k.shape[2]
    np.testing.assert_allclose(o, np.repeat(v, G, axis=2), atol=1e-15)
    do = RNG.standard_normal(o.shape)
    dq, dk, dv = O.attention_backward(do, q, k, v, P)
    assert np.max(np.abs(dq)) < 1e-15 and np.max(np.abs(dk)) < 1e-15


def test_window_ge_T_minus_1_is_full_causal():
    q, k, v = _qkv(T=10)
    o_full, _ = O.attention(q, k, v, -1)
    o_w, _ = O.attention(q, k, v, 9)
    o_w2, _ = O.attention(q, k, v, 500)
    np.testing.assert_array_equal(o_full, o_w)
    np.testing.assert_array_equal(o_full, o_w2)
    o_w8, _ = O.attention(q, k, v, 8)
    assert np.max(np.abs(o_w8 - o_full)) > 1e-6  # one key fewer on the last row


def test_gqa_equals_mha_on_repeated_kv():
    q, k, v = _qkv(H=6, Hkv=2)
    G = 3
    kr, vr = np.repeat(k, G, axis=2), np.repeat(v, G, axis=2)
    o_g, P_g = O.attention(q, k, v, 3)
    o_m, P_m = O.attention(q, kr, vr, 3)
    np.testing.assert_allclose(o_g, o_m, atol=1e-15)
    do = RNG.standard_normal(o_g.shape)
    dq_g, dk_g, dv_g = O.attention_backward(do, q, k, v, P_g)
    dq_m, dk_m, dv_m = O.attention_backward(do, q, kr, vr, P_m)
    np.testing.assert_allclose(dq_g, dq_m, atol=1e-14)
    B, T = q.shape[:2]
    np.testing.assert_allclose(dk_g, dk_m.reshape(B, T, 2, G, -1).sum(3), atol=1e-13)
    np.testing.assert_allclose(dv_g, dv_m.reshape(B, T, 2, G, -1).sum(3), atol=1e-13)


def test_mha_head_independence():
    # n_kv_head = n_head: head h of the output depends only on head h inputs
    q, k, v = _qkv(H=3, Hkv=3)
    o, _ = O.attention(q, k, v, -1)
    for h in range(3):
        oh, _ = O.attention(q[:, :, h:h + 1], k[:, :, h:h + 1], v[:, :, h:h + 1], -1)
        np.testing.assert_allclose(o[:, :, h:h + 1], oh, atol=1e-15)


@pytest.mark.parametrize("window", [-1, 2])
def test_causality_under_perturbation(window):
    q, k, v = _qkv(T=14)
    o, _ = O.attention(q, k, v, window)
    j = 6
    k2, v2 = k.copy(), v.copy()
    k2[:, j] += 1.0
    v2[:, j] -= 2.0
    o2, _ = O.attention(q, k2, v2, window)
    np.testing.assert_array_equal(o[:, :j], o2[:, :j])
    if window >= 0:
        np.testing.assert_array_equal(o[:, j + window + 1:], o2[:, j + window + 1:])
    assert np.max(np.abs(o[:, j] - o2[:, j])) > 1e-3


@pytest.mark.parametrize("window", [-1, 0, 3])
def test_attention_backward_fd(window):
    q, k, v = _qkv(B=1, T=7, H=4, Hkv=2, D=4)
    w = RNG.standard_normal(q.shape)
    o, P = O.attention(q, k, v, window)
    dq, dk, dv = O.attention_backward(w, q, k, v, P)
    fd_check(lambda z: float(np.sum(O.attention(z, k, v, window)[0] * w)), q, dq)
    fd_check(lambda z: float(np.sum(O.attention(q, z, v, window)[0] * w)), k, dk)
    fd_check(lambda z: float(np.sum(O.attention(q, k, z, window)[0] * w)), v, dv)


# ------------------------------------------------------------ cross-entropy
def test_ce_zero_head_closed_form():
    N, C, V = 9, 12, 17
    x = RNG.standard_normal((N, C))
    y = RNG.integers(0, V, size=N)
    loss, dx, dw, c = O.lm_head_ce(x, np.zeros((V, C)), y, 1e-6)
    assert loss == pytest.approx(math.log(V), rel=1e-15)
    onehot = np.zeros((N, V))
    onehot[np.arange(N), y] = 1.0
    np.testing.assert_allclose(c["dz"], (1.0 / V - onehot) / N, atol=1e-16)
    assert np.all(dx == 0.0)


def test_ce_rows_of_dz_sum_to_zero_and_fd():
    N, C, V = 6, 10, 13
    x = RNG.standard_normal((N, C))
    W = RNG.standard_normal((V, C)) * 0.3
    y = RNG.integers(0, V, size=N)
    loss, dx, dw, c = O.lm_head_ce(x, W, y, 1e-6)
    np.testing.assert_allclose(c["dz"].sum(1), 0.0, atol=1e-16)
    fd_check(lambda z: O.lm_head_ce(z, W, y, 1e-6)[0], x, dx, rtol=1e-7)
    fd_check(lambda z: O.lm_head_ce(x, z, y, 1e-6)[0], W, dw, rtol=1e-7)


def test_ce_init_statistics():
    # at init the normalised stream has unit RMS so logits are ~N(0, 0.02^2 C);
    # E[loss] ~= ln V + 0.0002 C
    N, C, V = 256, 128, 512
    x = RNG.standard_normal((N, C))
    W = RNG.standard_normal((V, C)) * 0.02
    y = RNG.integers(0, V, size=N)
    loss = O.lm_head_ce(x, W, y, 1e-6)[0]
    assert abs(loss - (math.log(V) + 0.0002 * C)) < 0.05


# --------------------------------------------------------------------- fp8
def test_e4m3_grid_special_values():
    vals = np.array([0.0, 1.0, 1.0625, 1.125, 1.1875, 448.0, 464.0, 470.0, 1e9, 2 ** -9,
                     2 ** -10, 3 * 2 ** -11, -1.0625, 2 ** -6, 0.0009765625])
    exp = np.array([0.0, 1.0, 1.0, 1.125, 1.25, 448.0, 448.0, 448.0, 448.0, 2 ** -9,
                    0.0, 2 ** -9, -1.0, 2 ** -6, 0.0])
    np.testing.assert_array_equal(O.e4m3_round(vals), exp)


def test_e4m3_matches_torch_cast_on_all_bf16_in_range():
    torch = pytest.importorskip("torch")
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    f = (bits << 16).view(np.float32).astype(np.float64)
    ok = np.isfinite(f) & (np.abs(f) <= 464.0)   # torch's cast overflows to NaN above 464
    f = f[ok]
    ref = torch.from_numpy(f).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.e4m3_round(f), ref)


def test_bf16_round_matches_torch_cast():
    torch = pytest.importorskip("torch")
    x = np.concatenate([RNG.standard_normal(4096) * 10.0 ** RNG.integers(-8, 8, 4096),
                        # exact ties between two bfloat16 values: 1 + 2^-8 -> 1, 1 + 3*2^-8 -> 1 + 2^-6
                        [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 0.0, 65504.0]])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.bf16_round(x), ref)
    assert O.bf16_round(np.array([1.0 + 2.0 ** -8]))[0] == 1.0


def test_fp8_quant_dequant_error_bound():
    x = RNG.standard_normal((64, 64)) * 5.0
    y = O.fp8_quant_dequant(x)
    s = np.max(np.abs(x)) / 448.0
    # relative half-ulp 2^-4 on normals, absolute half-ulp 2^-10 * s on subnormals
    assert np.all(np.abs(y - x) <= np.maximum(np.abs(x) * 2.0 ** -4, s * 2.0 ** -10) + 1e-15)
    # amax lands on the top code 448: back to amax up to the float32 scale
    assert np.max(np.abs(y)) == pytest.approx(np.max(np.abs(x)), rel=2 ** -22)


def test_fp8_quantize_codes_are_float32_decisions():
    # an input exactly halfway between two e4m3 steps after a float32 division
    # rounds to even; codes depend only on float32 arithmetic
    x = np.array([448.0, -224.0, 1.0, 0.0, 3.5, 7.0, 15.0])
    q, s = O.fp8_quantize(x)
    assert s == float(np.float32(448.0) / np.float32(448.0)) == 1.0
    np.testing.assert_array_equal(q, [448.0, -224.0, 1.0, 0.0, 3.5, 7.0, 15.0])
    q, s = O.fp8_quantize(x * 3.0)          # s = 3: 3.5*3/3 = 3.5 exactly, etc.
    assert s == 3.0
    np.testing.assert_array_equal(q, [448.0, -224.0, 1.0, 0.0, 3.5, 7.0, 15.0])
    q, s = O.fp8_quantize(np.zeros(5))
    assert s == 0.0 and not np.any(q)
    # 17 = 16 * 1.0625 is a tie between 16 and 18 (3 mantissa bits): even -> 16
    q, _ = O.fp8_quantize(np.array([448.0, 17.0, 19.0]))
    np.testing.assert_array_equal(q, [448.0, 16.0, 20.0])


# ------------------------------------------------------ whole-step FD pins
def _params(cfg, rng):
    Q, KV = cfg.n_head * cfg.head_dim, cfg.n_kv_head * cfg.head_dim
    C, F, V = cfg.C, cfg.mlp_hidden, cfg.vocab
    s = 0.3
    glob = {"wte": rng.standard_normal((V, C)), "w_lm": rng.standard_normal((V, C)) * s}
    layers = []
    for l in range(cfg.n_layer):
        p = {"w_qkv": rng.standard_normal((Q + 2 * KV, C)) * s, "w_o": rng.standard_normal((C, Q)) * s,
             "w_fc": rng.standard_normal((F, C)) * s, "w_proj": rng.standard_normal((C, F)) * s}
        if cfg.extras:
            p["resid_lambda"] = rng.uniform(0.5, 1.5)
            p["x0_lambda"] = rng.uniform(0.5, 1.5)
            if l % 2 == 1:
                p["ve"] = rng.standard_normal((V, KV))
                p["ve_gate"] = rng.standard_normal((cfg.n_kv_head, cfg.ve_gate_channels)) * s
        layers.append(p)
    if cfg.extras:
        glob["smear_lambda"] = rng.uniform(0.5, 1.5)
        glob["backout_lambda"] = rng.uniform(0.5, 1.5)
        glob["smear_gate"] = rng.standard_normal(cfg.smear_channels) * s
    ids = rng.integers(0, V, size=(cfg.B, cfg.T + 1))
    return ids, glob, layers


def _loss(cfg, ids, glob, layers):
    return O.stack_forward_backward(cfg, ids, glob, layers)[0]


def _fd_all(cfg, seed, h=1e-6, rtol=2e-6):
    rng = np.random.default_rng(seed)
    ids, glob, layers = _params(cfg, rng)
    loss, grads, _ = O.stack_forward_backward(cfg, ids, glob, layers)
    checked = 0

    def check(get, setv, g):
        nonlocal checked
        base = np.array(get(), dtype=np.float64)
        d = rng.standard_normal(base.shape)
        setv(base + h * d)
        lp = _loss(cfg, ids, glob, layers)
        setv(base - h * d)
        lm = _loss(cfg, ids, glob, layers)
        setv(base)
        num = (lp - lm) / (2 * h)
        ana = float(np.sum(np.asarray(g) * d))
        assert abs(num - ana) <= rtol * max(abs(ana), 1e-3), (num, ana)
        checked += 1

    for key in list(glob.keys()):
        g = grads[key]
        check(lambda k=key: glob[k], lambda v, k=key: glob.__setitem__(k, v), g)
    for l, p in enumerate(layers):
        for key in list(p.keys()):
            g = grads["layers"][l][key]
            check(lambda k=key, p=p: p[k], lambda v, k=key, p=p: p.__setitem__(k, v), g)
    return checked


def test_fd_whole_step_gqa_window():
    assert _fd_all(tiny_cfg(), 1) == 2 + 2 * 4


def test_fd_whole_step_mha_full():
    assert _fd_all(tiny_cfg(n_kv_head=2, windows=(-1, -1), T=5), 2) == 10


def test_fd_whole_step_window0_and_T1():
    _fd_all(tiny_cfg(windows=(0, 1), T=4), 3)
    _fd_all(tiny_cfg(T=1, B=3), 4)


def test_fd_whole_step_extras():
    cfg = tiny_cfg(C=48, n_head=3, n_kv_head=1, head_dim=16, mlp_hidden=96, vocab=13, T=5,
                   n_layer=2, windows=(-1, 2), extras=True)
    n = _fd_all(cfg, 5)
    assert n == 5 + (4 + 2) + (4 + 2 + 2)


def test_fd_whole_step_extras_four_layers():
    # backout taken after block L/2 - 1 = 1, value embeddings on layers 1 and 3
    cfg = tiny_cfg(C=48, n_head=3, n_kv_head=3, head_dim=16, mlp_hidden=96, vocab=9, T=4, B=1,
                   n_layer=4, windows=(-1, 1, -1, 2), extras=True)
    _fd_all(cfg, 6)


def test_attention_logsumexp_matches_softmax_denominator():
    q, k, v = _qkv(T=9)
    for window in (-1, 0, 2):
        lse = O.attention_logsumexp(q, k, window)
        _, P = O.attention(q, k, v, window)
        # P_ij = exp(s_ij - lse_i) on visible pairs
        B, T, H, D = q.shape
        for b in range(B):
            for h in range(H):
                s = q[b, :, h] @ k[b, :, h // (H // k.shape[2])].T / math.sqrt(D)
                m = O.visible_mask(T, window)
                np.testing.assert_allclose(P[b, h][m], np.exp(s - lse[b, h][:, None])[m], rtol=1e-12)


def test_cross_entropy_against_torch():
    torch = pytest.importorskip("torch")
    z = RNG.standard_normal((7, 23)) * 2.0
    y = RNG.integers(0, 23, size=7)
    zt = torch.tensor(z, requires_grad=True)
    lt = torch.nn.functional.cross_entropy(zt, torch.tensor(y))
    lt.backward()
    loss, row_loss, dz, lse = O.cross_entropy(z, y)
    assert abs(loss - float(lt)) < 1e-13
    np.testing.assert_allclose(dz, zt.grad.numpy(), atol=1e-15)
    np.testing.assert_allclose(lse, torch.logsumexp(torch.tensor(z), 1).numpy(), rtol=1e-14)


# ----------------------------------------------------------- decode attention
def _decode_inputs(B=3, Tmax=20, H=4, Hkv=2, D=8, seed=5):
    g = np.random.default_rng(seed)
    return (g.standard_normal((B, H, D)), g.standard_normal((B, Tmax, Hkv, D)),
            g.standard_normal((B, Tmax, Hkv, D)))


@pytest.mark.parametrize("window", [-1, 0, 3, 30])
def test_decode_is_last_row_of_attention(window):
    # decode of a sequence of length L equals row L-1 of the training attention
    # on that sequence with the new query in its last row
    q, k, v = _decode_inputs()
    lens = np.array([1, 7, 20])
    o, lse = O.attention_decode(q, k, v, lens, window)
    for b, L in enumerate(lens):
        qs = np.zeros((1, L, 4, 8))
        qs[0, L - 1] = q[b]
        oa, _ = O.attention(qs, k[b:b + 1, :L], v[b:b + 1, :L], window)
        np.testing.assert_allclose(o[b], oa[0, L - 1], rtol=1e-12, atol=1e-14)
        la = O.attention_logsumexp(qs, k[b:b + 1, :L], window)
        np.testing.assert_allclose(lse[b], la[0, :, L - 1], rtol=1e-12)


@pytest.mark.parametrize("window", [-1, 4])
def test_decode_against_torch_sdpa(window):
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    q, k, v = _decode_inputs(B=2, Tmax=16, H=6, Hkv=2, D=16, seed=9)
    lens = np.array([16, 9])
    o, _ = O.attention_decode(q, k, v, lens, window)
    for b, L in enumerate(lens):
        i = L - 1
        vis = np.array([(j <= i) and (window < 0 or i - j <= window) for j in range(16)])
        kk = torch.from_numpy(np.repeat(k[b], 3, axis=1)).permute(1, 0, 2)   # [H, T, D]
        vv = torch.from_numpy(np.repeat(v[b], 3, axis=1)).permute(1, 0, 2)
        qq = torch.from_numpy(q[b])[:, None, :]                               # [H, 1, D]
        ref = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=torch.from_numpy(vis)[None, None, :])
        np.testing.assert_allclose(o[b], ref[:, 0, :].numpy(), rtol=1e-12, atol=1e-14)


def test_decode_closed_forms():
    q, k, v = _decode_inputs()
    lens = np.array([1, 7, 20])
    # zero query: uniform weights, o = mean of the visible values, lse = log(count)
    for window in (-1, 2):
        o, lse = O.attention_decode(np.zeros_like(q), k, v, lens, window)
        for b, L in enumerate(lens):
            lo = max(0, L - 1 - window) if window >= 0 else 0
            for h in range(4):
                np.testing.assert_allclose(o[b, h], v[b, lo:L, h // 2].mean(axis=0), rtol=1e-13)
                assert lse[b, h] == pytest.approx(math.log(L - lo), rel=1e-14)
    # one visible key (length 1, or window 0): o is that value, lse its score
    o, lse = O.attention_decode(q, k, v, lens, 0)
    for b, L in enumerate(lens):
        for h in range(4):
            np.testing.assert_allclose(o[b, h], v[b, L - 1, h // 2], rtol=1e-14)
            assert lse[b, h] == pytest.approx(float(q[b, h] @ k[b, L - 1, h // 2]) / math.sqrt(8), rel=1e-13)
    # empty sequence
    o, lse = O.attention_decode(q, k, v, np.array([0, 3, 3]), -1)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))


# ----------------------------------------------------------------- optimizer
PE_PRINTED = [(8.156, -22.483, 15.879), (4.043, -2.809, 0.500)]   # the two triples the pages print


def _svd_closed_form(G, coeffs, norm_scale=1.0, eps=1e-7):
    U, S, Vt = np.linalg.svd(G, full_matrices=False)
    s = S / (np.linalg.norm(G) * norm_scale + eps)
    for a, b, c in coeffs:
        s = a * s + b * s ** 3 + c * s ** 5
    return (U * s) @ Vt


@pytest.mark.parametrize("shape", [(7, 5), (5, 7), (12, 12)])
@pytest.mark.parametrize("coeffs", [PE_PRINTED, [(3.0, -3.2, 1.2)] * 3, [(1.5, -0.5, 0.0)]])
def test_newton_schulz_svd_closed_form(shape, coeffs):
    G = np.random.default_rng(3).standard_normal(shape)
    X = O.newton_schulz(G, coeffs, norm_scale=1.02)
    np.testing.assert_allclose(X, _svd_closed_form(G, coeffs, 1.02), rtol=1e-10, atol=1e-12)
    # transpose identity of the exact map (the Gram can be taken on either side)
    np.testing.assert_allclose(O.newton_schulz(G.T, coeffs, 1.02), X.T, rtol=1e-10, atol=1e-12)


def test_newton_schulz_cubic_converges_to_polar_factor():
    G = np.random.default_rng(4).standard_normal((9, 6))
    U, S, Vt = np.linalg.svd(G, full_matrices=False)
    X = O.newton_schulz(G, [(1.5, -0.5, 0.0)] * 60)
    np.testing.assert_allclose(X, U @ Vt, atol=1e-9)


def test_adamw_against_torch():
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(5)
    p0 = g.standard_normal(37)
    grads = [g.standard_normal(37) for _ in range(4)]
    kw = dict(lr=3e-3, betas=(0.8, 0.95), eps=1e-8, weight_decay=0.1)
    tp = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    opt = torch.optim.AdamW([tp], **kw)
    p, m, v = p0.copy(), np.zeros(37), np.zeros(37)
    for t, gr in enumerate(grads, 1):
        tp.grad = torch.from_numpy(gr.copy())
        opt.step()
        p, m, v = O.adamw_step(p, gr, m, v, t, 3e-3, 0.8, 0.95, 1e-8, 0.1)
        np.testing.assert_allclose(p, tp.detach().numpy(), rtol=1e-13, atol=1e-15)


def test_muon_without_momentum_is_a_newton_schulz_step():
    g = np.random.default_rng(6)
    p, gr = g.standard_normal((8, 5)), g.standard_normal((8, 5))
    p1, buf = O.muon_step(p, gr, np.zeros((8, 5)), 0.02, 0.0, True, 0.0, 1.5, PE_PRINTED)
    np.testing.assert_allclose(p1, p - 0.02 * 1.5 * _svd_closed_form(gr, PE_PRINTED), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(buf, gr)
    # Nesterov with momentum mu orthogonalises g + mu * (mu * buf + g)
    b0 = g.standard_normal((8, 5))
    p2, buf2 = O.muon_step(p, gr, b0, 0.02, 0.9, True, 0.1, 1.0, PE_PRINTED)
    np.testing.assert_allclose(buf2, 0.9 * b0 + gr)
    u = gr + 0.9 * buf2
    np.testing.assert_allclose(p2, p * (1 - 0.002) - 0.02 * _svd_closed_form(u, PE_PRINTED), rtol=1e-10, atol=1e-12)


def test_newton_schulz_bf16_storage_option():
    # the bf16-storage variant only rounds: zero steps give the rounded
    # normalised input, and its distance from the exact map shrinks with the
    # number of bits (an fp32-like rounding would be ~2^16 times closer)
    G = np.random.default_rng(8).standard_normal((40, 24))
    x0 = O.newton_schulz(G, [], 1.0)
    np.testing.assert_array_equal(O.newton_schulz(G, [], 1.0, round_to="bf16"), O.bf16_round(x0))
    d = np.max(np.abs(O.newton_schulz(G, PE_PRINTED, round_to="bf16") - O.newton_schulz(G, PE_PRINTED)))
    assert 1e-5 < d < 0.1 * np.max(np.abs(O.newton_schulz(G, PE_PRINTED)))
    # the rounding follows the given orientation (no side is chosen for it):
    # the transposed problem has the same exact map but rounds other values
    dT = np.max(np.abs(O.newton_schulz(G.T, PE_PRINTED, round_to="bf16").T - O.newton_schulz(G, PE_PRINTED)))
    assert 1e-5 < dT < 0.1 * np.max(np.abs(O.newton_schulz(G, PE_PRINTED)))
    assert not np.array_equal(O.newton_schulz(G.T, PE_PRINTED, round_to="bf16").T,
                              O.newton_schulz(G, PE_PRINTED, round_to="bf16"))


# ------------------------------------------------------------------ NorMuon
def test_normuon_keeps_the_update_norm():
    # the final scale v_norm / v_norm_new rescales the per-neuron normalised
    # update back to the orthogonalised update's Frobenius norm, whatever the
    # state v and beta2
    g = np.random.default_rng(21)
    for m, n, beta2 in ((12, 7, 0.95), (5, 9, 0.0), (16, 16, 0.5)):
        o = g.standard_normal((m, n)) * g.uniform(0.1, 3.0, size=(m, 1))
        v0 = g.uniform(0.01, 2.0, size=m)
        out, v1 = O.normuon_scale(o, v0, beta2)
        assert np.linalg.norm(out) == pytest.approx(np.linalg.norm(o), rel=1e-12)
        # each row is only rescaled (the direction of every neuron's update is kept)
        cos = np.sum(out * o, axis=1) / (np.linalg.norm(out, axis=1) * np.linalg.norm(o, axis=1))
        np.testing.assert_allclose(cos, 1.0, rtol=1e-12)


def test_normuon_equalises_rows_without_history():
    # beta2 = 0: v is the current per-row mean square, so every output neuron's
    # update ends with the same RMS (the mean of the rows' mean squares); the
    # columns are not equalised
    g = np.random.default_rng(22)
    o = g.standard_normal((10, 6)) * np.linspace(0.2, 5.0, 10)[:, None]
    out, v1 = O.normuon_scale(o, np.zeros(10), 0.0)
    ms = np.mean(out * out, axis=1)
    np.testing.assert_allclose(ms, np.mean(np.mean(o * o, axis=1)), rtol=1e-12)
    np.testing.assert_allclose(v1, np.mean(o * o, axis=1), rtol=1e-15)
    assert np.std(np.mean(out * out, axis=0)) > 1e-3


def test_normuon_is_muon_when_rows_already_agree():
    # rows of one RMS with the state holding that value: the per-neuron scale
    # is uniform and cancels against the norm ratio, so the update is Muon's
    g = np.random.default_rng(23)
    o = g.standard_normal((8, 12))
    o /= np.sqrt(np.mean(o * o, axis=1, keepdims=True)) / 0.3
    out, _ = O.normuon_scale(o, np.full(8, 0.09), 0.9)
    np.testing.assert_allclose(out, o, rtol=1e-12, atol=1e-15)
    p, gr, buf = g.standard_normal((8, 5)), g.standard_normal((8, 5)), g.standard_normal((8, 5))
    pm, bm = O.muon_step(p, gr, buf, 0.02, 0.9, True, 0.1, 1.5, PE_PRINTED)
    # a uniform state cancels too; a state that differs across rows does not
    pu, _, _ = O.normuon_step(p, gr, buf, np.full(8, 1e3), 0.02, 0.9, True, 0.1, 1.5, 0.9, PE_PRINTED)
    vrow = np.where(np.arange(8) % 2 == 0, 1e-2, 1e2)
    pn, bn, _ = O.normuon_step(p, gr, buf, vrow, 0.02, 0.9, True, 0.1, 1.5, 0.9, PE_PRINTED)
    np.testing.assert_allclose(bn, bm)
    assert np.max(np.abs(pu - pm)) < 1e-5 * np.max(np.abs(pm))
    assert np.max(np.abs(pn - pm)) > 1e-3


def test_normuon_state_tracks_the_row_statistics():
    # repeated steps on the same update: v converges to the rows' mean squares
    # (an exponential moving average), and the output to the beta2 = 0 one
    g = np.random.default_rng(24)
    o = g.standard_normal((6, 9)) * np.array([0.5, 1, 2, 3, 4, 8])[:, None]
    v = np.full(6, 7.0)
    for _ in range(400):
        out, v = O.normuon_scale(o, v, 0.9)
    np.testing.assert_allclose(v, np.mean(o * o, axis=1), rtol=1e-12)
    np.testing.assert_allclose(out, O.normuon_scale(o, np.zeros(6), 0.0)[0], rtol=1e-10)
    # one step from v = 0 weighs the new statistic by 1 - beta2
    _, v1 = O.normuon_scale(o, np.zeros(6), 0.75)
    np.testing.assert_allclose(v1, 0.25 * np.mean(o * o, axis=1), rtol=1e-15)


# ------------------------------------------- bf16 storage of the streams
@pytest.mark.parametrize("extras", [False, True])
def test_stack_bf16_stream_storage_option(extras):
    """The option that measures how bf16 storage of the residual streams moves
    the result (the full-depth parity bound): off, the exact oracle bit for
    bit; on, every stream entering a block is a bf16 value, and the loss and
    every gradient move by more than nothing and by no more than a few bf16
    unit roundoffs per stored stream."""
    cfg = tiny_cfg(C=48, n_head=3, n_kv_head=1, head_dim=16, mlp_hidden=96, vocab=13, T=5, n_layer=4,
                   windows=(-1, 2, -1, 1), extras=extras)
    ids, glob, layers = _params(cfg, np.random.default_rng(31))
    l0, g0, _ = O.stack_forward_backward(cfg, ids, glob, layers)
    la, ga, _ = O.stack_forward_backward(cfg, ids, glob, layers, stream_dtype=None)
    assert la == l0 and np.array_equal(ga["wte"], g0["wte"]) and np.array_equal(ga["w_lm"], g0["w_lm"])
    l1, g1, o1 = O.stack_forward_backward(cfg, ids, glob, layers, keep=True, stream_dtype="bf16")
    for a in o1["acts"]:
        assert np.array_equal(O.bf16_round(a), a)
    u = 2.0 ** -9  # bf16 unit roundoff
    stores = 2 * (cfg.n_layer + 1)
    rel = lambda a, b: float(np.max(np.abs(a - b))) / float(np.max(np.abs(b)))
    assert 0 < abs(l1 - l0) / abs(l0) < stores * u
    for k in ("wte", "w_lm"):
        assert 0 < rel(g1[k], g0[k]) < 10 * stores * u
    for l in range(cfg.n_layer):
        for k in ("w_qkv", "w_o", "w_fc", "w_proj"):
            assert 0 < rel(g1["layers"][l][k], g0["layers"][l][k]) < 10 * stores * u
    with pytest.raises(ValueError):
        O.stack_forward_backward(cfg, ids, glob, layers, stream_dtype="fp16")


def test_smear_gate_term_magnitudes_bound_the_gradient():
    """sum_abs of the smear gate's gradient is the magnitude sum of its terms:
    it bounds the gradient (triangle inequality) and equals it when every
    term has one sign (dx = x_prev with the gate's derivative positive)."""
    cfg = tiny_cfg(C=48, n_head=3, n_kv_head=1, head_dim=16, mlp_hidden=96, vocab=13, T=5, n_layer=2,
                   windows=(-1, 2), extras=True)
    ids, glob, layers = _params(cfg, np.random.default_rng(41))
    _, g, o = O.stack_forward_backward(cfg, ids, glob, layers)
    sa = o["sum_abs"]["smear_gate"]
    assert sa.shape == g["smear_gate"].shape and np.all(sa >= np.abs(g["smear_gate"]) * (1 - 1e-12))
    assert np.all(sa < 1e3 * (np.abs(g["smear_gate"]) + 1e-300))
    # one sign: with the embedding rows positive and dx parallel to x_prev the
    # two nested sums have no cancellation, so the bound is attained
    e = np.abs(np.random.default_rng(3).standard_normal((1, 4, 8))) + 0.1
    c = {"prev": np.concatenate([np.zeros((1, 1, 8)), e[:, :-1]], axis=1)}
    c["sg"] = np.full((1, 4), 0.3)
    c["gate"] = 0.5 * c["sg"]
    dx = c["prev"].copy()
    _, dws, _ = O.smear_backward(dx, e, np.ones(3), 0.5, c)
    inner = np.sum(np.abs(dx * c["prev"]), axis=-1)
    inner[:, 0] = 0.0
    ref = np.einsum("bt,btc->c", inner * np.abs(0.5 * c["sg"] * (1 - c["sg"])), np.abs(e[..., :3]))
    assert np.allclose(dws, ref, rtol=1e-14, atol=0)
