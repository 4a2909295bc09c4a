"""The oracle against torch float64 autograd on library primitives.

The torch model below computes the same step with F.rms_norm, F.linear,
F.scaled_dot_product_attention (boolean window mask, enable_gqa),
F.embedding and F.cross_entropy, and takes every gradient from autograd.  It
shares nothing with the oracle's hand-written backward, so it pins the
oracle's forward to the library routines and its backward to autograd.  Only
RoPE and the d26 extras are written out here (RoPE is pinned separately by
its invariants in test_oracle_pins.py).

The fp8 MLP is checked the same way: torch's own float8_e4m3fn cast makes the
codes, a straight-through wrapper passes gradients through the quantiser, and
an identity whose backward quantises the incoming gradient puts the output
gradient of each MLP product on fp8 as well, so autograd yields the six fp8
products without any hand-written backward."""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")
F = torch.nn.functional

import oracle as O
from seeded_inputs import Workload, draw_all, workload

from test_oracle_pins import _params, tiny_cfg


def _rope_t(x, T, D, base):
    j = torch.arange(D // 2, dtype=torch.float64)
    th = torch.arange(T, dtype=torch.float64)[:, None] * base ** (-2.0 * j / D)[None, :]
    c, s = torch.cos(th)[None, :, None, :], torch.sin(th)[None, :, None, :]
    a, b = x[..., : D // 2], x[..., D // 2:]
    return torch.cat([a * c - b * s, a * s + b * c], dim=-1)


def _q8_t(x, storage):
    """Per-tensor e4m3 quantise-dequantise with torch's cast (float32 scale and division)."""
    if storage == "bf16":
        x = x.to(torch.bfloat16).to(torch.float64)
    amax = x.abs().max().to(torch.float32)
    if float(amax) == 0.0:
        return torch.zeros_like(x)
    s = amax / torch.tensor(448.0, dtype=torch.float32)
    q = (x.to(torch.float32) / s).to(torch.float8_e4m3fn).to(torch.float64)
    return q * s.to(torch.float64)


class _GradQ(torch.autograd.Function):
    """Identity whose backward quantises the incoming gradient."""

    @staticmethod
    def forward(ctx, x, storage):
        ctx.storage = storage
        return x.view_as(x)

    @staticmethod
    def backward(ctx, g):
        return _q8_t(g, ctx.storage), None


def _fp8_linear(x, w, storage):
    st = lambda a: a + (_q8_t(a.detach(), storage) - a).detach()   # value q8(a), gradient 1
    return _GradQ.apply(F.linear(st(x), st(w)), storage)


def torch_step(cfg, ids, glob, layers):
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True)
    G = {k: t(v) for k, v in glob.items()}
    Ls = [{k: t(v) for k, v in p.items()} for p in layers]
    ids_t = torch.tensor(ids)
    B, T1 = ids.shape
    T = T1 - 1
    inp, tgt = ids_t[:, :T], ids_t[:, 1:]
    H, Hkv, D, C = cfg.n_head, cfg.n_kv_head, cfg.head_dim, cfg.C
    Q, KV = H * D, Hkv * D
    eps = cfg.eps
    x = F.embedding(inp, G["wte"])
    if cfg.extras:
        n = cfg.smear_channels
        gate = G["smear_lambda"] * torch.sigmoid(x[..., :n] @ G["smear_gate"])
        prev = torch.cat([torch.zeros_like(x[:, :1]), x[:, :-1]], dim=1)
        gate = torch.cat([torch.zeros_like(gate[:, :1]), gate[:, 1:]], dim=1)
        x = x + gate[..., None] * prev
    x0 = x
    x_bo = None
    for l, p in enumerate(Ls):
        if cfg.extras:
            x = p["resid_lambda"] * x + p["x0_lambda"] * x0
        xn = F.rms_norm(x, (C,), eps=eps)
        qkv = F.linear(xn, p["w_qkv"])
        q = qkv[..., :Q].reshape(B, T, H, D)
        k = qkv[..., Q:Q + KV].reshape(B, T, Hkv, D)
        v = qkv[..., Q + KV:].reshape(B, T, Hkv, D)
        if cfg.extras and "ve" in p:
            g = 3.0 * torch.sigmoid(F.linear(xn[..., :cfg.ve_gate_channels], p["ve_gate"]))
            v = v + g[..., None] * F.embedding(inp, p["ve"]).reshape(B, T, Hkv, D)
        q = _rope_t(F.rms_norm(q, (D,), eps=eps), T, D, cfg.rope_base)
        k = _rope_t(F.rms_norm(k, (D,), eps=eps), T, D, cfg.rope_base)
        mask = torch.ones(T, T, dtype=torch.bool).tril()
        if cfg.windows[l] >= 0:
            mask = mask.triu(-cfg.windows[l])
        o = F.scaled_dot_product_attention(q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2),
                                           attn_mask=mask, enable_gqa=True)
        o = o.transpose(1, 2).reshape(B, T, Q)
        x = x + F.linear(o, p["w_o"])
        if getattr(cfg, "mlp_fp8", False):
            h = F.relu(_fp8_linear(F.rms_norm(x, (C,), eps=eps), p["w_fc"], cfg.dtype)) ** 2
            x = x + _fp8_linear(h, p["w_proj"], cfg.dtype)
        else:
            h = F.relu(F.linear(F.rms_norm(x, (C,), eps=eps), p["w_fc"])) ** 2
            x = x + F.linear(h, p["w_proj"])
        if cfg.extras and l == cfg.n_layer // 2 - 1:
            x_bo = x
    if cfg.extras:
        x = x - G["backout_lambda"] * x_bo
    z = F.linear(F.rms_norm(x, (C,), eps=eps), G["w_lm"])
    loss = F.cross_entropy(z.reshape(-1, z.shape[-1]), tgt.reshape(-1))
    loss.backward()
    grads = {k: v.grad.numpy() for k, v in G.items()}
    grads["layers"] = [{k: v.grad.numpy() for k, v in p.items()} for p in Ls]
    return float(loss), grads


def _compare(cfg, ids, glob, layers, tol=1e-11):
    loss_o, g_o, _ = O.stack_forward_backward(cfg, ids, glob, layers)
    loss_t, g_t = torch_step(cfg, ids, glob, layers)
    assert abs(loss_o - loss_t) <= tol * abs(loss_t)
    rel = lambda a, b: float(np.max(np.abs(np.asarray(a) - np.asarray(b))) / max(np.max(np.abs(b)), 1e-300))
    for k in g_t:
        if k == "layers":
            continue
        assert rel(g_o[k], g_t[k]) <= tol, k
    for l in range(cfg.n_layer):
        for k in g_t["layers"][l]:
            assert rel(g_o["layers"][l][k], g_t["layers"][l][k]) <= tol, (l, k)


@pytest.mark.parametrize("kw", [
    dict(),
    dict(n_kv_head=2, windows=(-1, -1)),
    dict(windows=(0, 5), T=9),
    dict(n_head=4, n_kv_head=2, head_dim=4, windows=(3, -1), T=11),
])
def test_oracle_matches_torch_autograd(kw):
    cfg = tiny_cfg(**kw)
    ids, glob, layers = _params(cfg, np.random.default_rng(11))
    _compare(cfg, ids, glob, layers)


def test_oracle_matches_torch_autograd_extras():
    cfg = tiny_cfg(C=48, n_head=3, n_kv_head=1, head_dim=16, mlp_hidden=96, vocab=13, T=7,
                   n_layer=4, windows=(-1, 2, -1, 3), extras=True)
    ids, glob, layers = _params(cfg, np.random.default_rng(12))
    _compare(cfg, ids, glob, layers)


def test_oracle_matches_torch_on_tiny_workload():
    # the tiny single-block workload exactly as specified (B=1, T=64, C=128,
    # 2 query heads sharing 1 K/V head of 64, vocab 512), seeded draws
    w = workload("tiny")
    d = draw_all(w)
    _compare(w, d["ids"], d["globals"], d["layers"], tol=1e-10)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_oracle_matches_torch_autograd_fp8_mlp(dtype):
    # fp8 MLP with and without the other extras; "bf16" also rounds every
    # quantised tensor to bfloat16 first (on both sides, by different code)
    cfg = tiny_cfg(C=48, n_head=3, n_kv_head=1, head_dim=16, mlp_hidden=96, vocab=13, T=7,
                   n_layer=4, windows=(-1, 2, -1, 3), extras=True, mlp_fp8=True, dtype=dtype)
    ids, glob, layers = _params(cfg, np.random.default_rng(13))
    _compare(cfg, ids, glob, layers)
    cfg = tiny_cfg(mlp_fp8=True, dtype=dtype)
    ids, glob, layers = _params(cfg, np.random.default_rng(14))
    _compare(cfg, ids, glob, layers)
