"""Plain float64 CPU oracle: forward and hand-written backward of the decoder
stack, the fused next-token cross-entropy and the embedding.

TEST INFRASTRUCTURE ONLY (see the package docstring): never called by the
product path.  Slow on purpose: no blocking, fusion or reordering beyond each
definition, so every function can be checked against the pages by eye.

Sources (page title, then section):
  [FR] "Comment Entraîner Votre Propre ChatGPT Pour 50€ ?", section
       "1. Le modèle GPT (nanochat/gpt.py)": RoPE without learned positions,
       QK normalisation, untied token embedding and output projection, ReLU²
       MLP, grouped-query attention, sliding-window attention; the value-
       embedding snippet and the three "astuces d'efficacité" snippets
       (per-layer residual scaling, smear, backout); section "3. Gestion de la
       précision": bias-free Linear computing F.linear(x, W) with W stored
       [out, in]; section "5. Unification de Flash Attention": the attention
       call takes (B, T, H, D) tensors with causal=True and a window_size.
  [JA] the same article on dev.to (Japanese), section "1. GPTモデル".
  [ZH] "nanochat：仅需73美元，3小时训练GPT-2级别大语言模型", section "排行榜"
       (the d24 run: batch 16 per device, sequence 2048).
  [FR] section "6. Moteur d'inférence": generation against a prefilled KV
       cache (`attention_decode`).

Readings taken where the pages are silent:
  * pre-norm blocks x += Attn(rms(x)); x += MLP(rms(x)); final rms before the
    head; no biases; RMSNorm has no affine and eps = 1e-6 everywhere;
  * QK norm is an RMSNorm over head_dim per (token, head), applied before
    RoPE (the two commute: RoPE is a rotation and the norm has no affine);
  * RoPE pairs dimension j with j + D/2, angle t * base^(-2j/D), positions
    restart at 0 on every row;
  * softmax scale 1/sqrt(D); window W >= 0 makes key j visible from query i
    iff 0 <= i - j <= W; W < 0 is plain causal attention;
  * query head h reads K/V head h // (H / Hkv);
  * the loss is the mean over all B*T positions, no ignore index;
  * fp8 operands (d26 MLP) are OCP e4m3fn with a per-tensor scale
    amax/448, round-to-nearest-even, saturating; gradients pass straight
    through the quantiser; all six MLP products (forward, data and weight
    gradients) take fp8 operands; scale and division in float32, and in
    bf16 mode the quantised tensors are bf16 values.

Pins (tests/test_oracle_*.py): finite differences of every gradient on tiny
shapes; RoPE preserves norms, is the identity at t = 0 and depends only on
relative position; softmax rows sum to one and vanish off the mask; W = 0 gives
o = v and zero dq, dk; W >= T - 1 equals full causal; Hkv = H equals MHA and
GQA equals MHA on repeated K/V; causality under perturbation; the whole
forward/backward against torch float64 autograd on library primitives
(F.rms_norm, F.linear, F.scaled_dot_product_attention, F.cross_entropy);
cross-entropy closed form at W_lm = 0; the e4m3 quantiser against torch's
float8_e4m3fn cast; decode attention against torch's scaled_dot_product_attention
with an explicit mask, the last row of `attention`, and the uniform-weight and
single-key closed forms.  Parity with nanochat's own numerics is unpinned: the
pages print no forward or backward value.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Tuple

import numpy as np

__all__ = [
    "rms_norm", "rms_norm_backward", "rope_tables", "rope", "rope_backward",
    "visible_mask", "attention", "attention_logsumexp", "attention_backward", "attention_decode",
    "cross_entropy", "e4m3_round",
    "bf16_round", "fp8_quantize", "fp8_quant_dequant", "mm_nt", "relu2", "relu2_grad", "block_forward", "block_backward", "lm_head_ce",
    "embed_forward", "embed_backward", "smear_forward", "smear_backward",
    "mix_forward", "mix_backward", "ve_forward", "ve_backward", "backout_forward", "backout_backward",
    "stack_forward_backward", "FP8_E4M3_MAX",
]

FP8_E4M3_MAX = 448.0


# ----------------------------------------------------------------- RMSNorm
def rms_norm(x: np.ndarray, eps: float) -> Tuple[np.ndarray, np.ndarray]:
    """y = x / sqrt(mean(x^2) + eps) over the last axis (no affine).
    Returns y and r = 1/sqrt(mean(x^2) + eps) (shape x.shape[:-1])."""
    ms = np.mean(x * x, axis=-1)
    r = 1.0 / np.sqrt(ms + eps)
    return x * r[..., None], r


def rms_norm_backward(dy: np.ndarray, y: np.ndarray, r: np.ndarray) -> np.ndarray:
    """Chain rule through y = x*r, r = (mean(x^2)+eps)^(-1/2):
    dx = r * (dy - y * mean(dy * y))."""
    return r[..., None] * (dy - y * np.mean(dy * y, axis=-1, keepdims=True))


# -------------------------------------------------------------------- RoPE
def rope_tables(T: int, D: int, base: float) -> Tuple[np.ndarray, np.ndarray]:
    """cos and sin of theta[t, j] = t * base^(-2j/D), t < T, j < D/2 (float64)."""
    j = np.arange(D // 2, dtype=np.float64)
    inv_freq = base ** (-2.0 * j / D)
    theta = np.arange(T, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.cos(theta), np.sin(theta)


def rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate each pair (x[j], x[j + D/2]) of x [B, T, H, D] by theta[t, j]:
    (a, b) -> (a cos - b sin, a sin + b cos)."""
    D = x.shape[-1]
    a, b = x[..., : D // 2], x[..., D // 2:]
    c, s = cos[None, :, None, :], sin[None, :, None, :]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def rope_backward(dy: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Transpose of the rotation (= rotation by -theta)."""
    D = dy.shape[-1]
    da, db = dy[..., : D // 2], dy[..., D // 2:]
    c, s = cos[None, :, None, :], sin[None, :, None, :]
    return np.concatenate([da * c + db * s, -da * s + db * c], axis=-1)


# --------------------------------------------------------------- attention
def visible_mask(T: int, window: int) -> np.ndarray:
    """[T, T] bool: query i sees key j iff j <= i and (window < 0 or i - j <= window)."""
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    m = j <= i
    if window >= 0:
        m &= (i - j) <= window
    return m


def _kv_head(h: int, H: int, Hkv: int) -> int:
    return h // (H // Hkv)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, window: int
              ) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention on q [B,T,H,D], k/v [B,T,Hkv,D]; scale 1/sqrt(D).
    Returns o [B,T,H,D] and the probabilities P [B,H,T,T] (zero off-mask)."""
    B, T, H, D = q.shape
    Hkv = k.shape[2]
    mask = visible_mask(T, window)
    scale = 1.0 / math.sqrt(D)
    o = np.zeros_like(q)
    P = np.zeros((B, H, T, T))
    for b in range(B):
        for h in range(H):
            g = _kv_head(h, H, Hkv)
            s = (q[b, :, h, :] @ k[b, :, g, :].T) * scale
            s = np.where(mask, s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            e = np.exp(s)
            p = e / e.sum(axis=1, keepdims=True)
            P[b, h] = p
            o[b, :, h, :] = p @ v[b, :, g, :]
    return o, P


def attention_logsumexp(q: np.ndarray, k: np.ndarray, window: int) -> np.ndarray:
    """log of the softmax denominator of each query row, [B, H, T]:
    lse[b, h, i] = log sum over visible j of exp(q_i . k_j / sqrt(D))."""
    B, T, H, D = q.shape
    Hkv = k.shape[2]
    mask = visible_mask(T, window)
    out = np.zeros((B, H, T))
    for b in range(B):
        for h in range(H):
            s = (q[b, :, h, :] @ k[b, :, _kv_head(h, H, Hkv), :].T) / math.sqrt(D)
            s = np.where(mask, s, -np.inf)
            m = s.max(axis=1)
            out[b, h] = m + np.log(np.sum(np.exp(s - m[:, None]), axis=1))
    return out


def attention_decode(q: np.ndarray, k: np.ndarray, v: np.ndarray, lens: np.ndarray, window: int
                     ) -> Tuple[np.ndarray, np.ndarray]:
    """One generation step against a key/value cache ([FR] section "6. Moteur
    d'inférence": the prompt is prefilled into a KV cache, then each new token
    attends to it).  q [B, H, D] is the query of position i = lens[b] - 1 of
    sequence b; k, v [B, Tmax, Hkv, D] hold positions 0 .. lens[b] - 1 (the new
    token's own key and value included).  Key j is visible iff j <= i and
    (window < 0 or i - j <= window) -- the rule of `attention`, for its last
    row.  Scale 1/sqrt(D); query head h reads K/V head h // (H / Hkv).
    Returns o [B, H, D] and lse [B, H] (natural log of the softmax
    denominator).  A length of 0 gives o = 0 and lse = -inf."""
    B, H, D = q.shape
    Hkv = k.shape[2]
    o = np.zeros((B, H, D))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        L = int(lens[b])
        if L <= 0:
            continue
        i = L - 1
        lo = max(0, i - window) if window >= 0 else 0
        for h in range(H):
            g = _kv_head(h, H, Hkv)
            s = (k[b, lo:L, g, :] @ q[b, h, :]) / math.sqrt(D)
            m = s.max()
            e = np.exp(s - m)
            o[b, h] = (e / e.sum()) @ v[b, lo:L, g, :]
            lse[b, h] = m + math.log(e.sum())
    return o, lse


def attention_backward(do: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray,
                       P: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Backward of `attention`: dP = dO V^T, dS = P*(dP - rowsum(dP*P)),
    dQ = dS K * scale, dK = dS^T Q * scale, dV = P^T dO; K/V gradients are summed
    over the query heads that share a K/V head."""
    B, T, H, D = q.shape
    Hkv = k.shape[2]
    scale = 1.0 / math.sqrt(D)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            g = _kv_head(h, H, Hkv)
            p = P[b, h]
            dv[b, :, g, :] += p.T @ do[b, :, h, :]
            dp = do[b, :, h, :] @ v[b, :, g, :].T
            ds = p * (dp - np.sum(dp * p, axis=1, keepdims=True))
            dq[b, :, h, :] = (ds @ k[b, :, g, :]) * scale
            dk[b, :, g, :] += (ds.T @ q[b, :, h, :]) * scale
    return dq, dk, dv


# --------------------------------------------------------------------- fp8
def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Round to the nearest OCP e4m3fn value (ties to even), saturating at
    +-448.  e4m3fn: 3 mantissa bits, exponent bias 7, smallest normal 2^-6,
    subnormal spacing 2^-9, no infinities."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, e = np.frexp(ax)                       # ax = m * 2^e, m in [0.5, 1)
    quantum = np.ldexp(1.0, np.maximum(e - 4, -9))  # 2^(floor(log2 ax) - 3), >= 2^-9
    q = np.round(ax / quantum) * quantum      # np.round: half to even
    q = np.minimum(q, FP8_E4M3_MAX)
    return np.where(x < 0, -q, q)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even, via float32), as float64."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    b = f.view(np.uint32)
    b = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return b.view(np.float32).astype(np.float64)


def fp8_quantize(x: np.ndarray, storage: Optional[str] = None) -> Tuple[np.ndarray, float]:
    """Per-tensor dynamic scaling: s = amax|x| / 448 and codes e4m3(x / s).
    The pages fix no precision for the scale and the division; both are taken
    in float32 (amax rounded to float32, s = amax / 448 and x / s each one
    correctly rounded float32 operation), so an input that is exactly
    representable in float32 gets the same code whatever computes it.
    storage="bf16": the quantised tensor is a bfloat16 activation (explicit
    dtypes, section "3. Gestion de la précision"), so its values are rounded
    to bfloat16 before the codes are chosen.
    Returns (the e4m3 values as float64, s as a float)."""
    x = np.asarray(x, dtype=np.float64)
    if storage == "bf16":
        x = bf16_round(x)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    if amax == 0.0:
        return np.zeros_like(x), 0.0
    s = np.float32(amax / np.float32(FP8_E4M3_MAX))
    q = x.astype(np.float32) / s
    return e4m3_round(q.astype(np.float64)), float(s)


def fp8_quant_dequant(x: np.ndarray, storage: Optional[str] = None) -> np.ndarray:
    """x ~ e4m3(x / s) * s with the per-tensor scale of `fp8_quantize`."""
    q, s = fp8_quantize(x, storage)
    return q * s


def mm_nt(a, b, fp8: bool = False, storage: Optional[str] = None) -> np.ndarray:
    """The bias-free Linear's product a @ b^T ([FR] section "3. Gestion de la
    précision": F.linear(x, W) with W [out, in]); with fp8, both operands go
    through the per-tensor e4m3 quantiser first (each with its own scale)."""
    if fp8:
        a, b = fp8_quant_dequant(a, storage), fp8_quant_dequant(b, storage)
    return a @ b.T


def relu2(u: np.ndarray) -> np.ndarray:
    """The MLP activation ([FR] section "1. Le modèle GPT": ReLU²): max(u, 0)^2."""
    return np.maximum(u, 0.0) ** 2


def relu2_grad(u: np.ndarray) -> np.ndarray:
    """d relu2 / du = 2 max(u, 0)."""
    return 2.0 * np.maximum(u, 0.0)


# ------------------------------------------------------------------ extras
def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def mix_forward(x: np.ndarray, x0: np.ndarray, a: float, b: float) -> np.ndarray:
    """Per-layer residual mixing ([FR] the per-layer residual scaling snippet):
    the block runs on a*x + b*x0, x0 the stream after embedding and smear."""
    return a * x + b * x0


def mix_backward(dy: np.ndarray, x: np.ndarray, x0: np.ndarray, a: float, b: float) -> dict:
    """Gradients of y = a*x + b*x0 given dy: dx = a*dy, dx0 = b*dy,
    da = sum(dy*x), db = sum(dy*x0); sum_abs holds each scalar sum's terms'
    magnitudes (the scale of its forward error bound)."""
    return {"dx": a * dy, "dx0": b * dy, "da": float(np.sum(dy * x)), "db": float(np.sum(dy * x0)),
            "sum_abs": {"da": float(np.sum(np.abs(dy * x))), "db": float(np.sum(np.abs(dy * x0)))}}


def ve_forward(xn: np.ndarray, v: np.ndarray, ids: np.ndarray, ve: np.ndarray, wg: np.ndarray
               ) -> Tuple[np.ndarray, dict]:
    """Value embedding ([FR] the value-embedding snippet): per token and K/V
    head g, s = xn[..., :nc] . wg[g], v[..., g, :] += 3*sigmoid(s) * VE[id, g, :].
    xn [B, T, C], v [B, T, Hkv, D], ids [B, T], ve [V, Hkv*D], wg [Hkv, nc]."""
    B, T, Hkv, D = v.shape
    nc = wg.shape[1]
    s = xn[..., :nc] @ wg.T                 # [B, T, Hkv]
    gate = 3.0 * _sigmoid(s)
    rows = ve[ids].reshape(B, T, Hkv, D)
    return v + gate[..., None] * rows, {"ve_s": s, "ve_gate": gate, "ve_rows": rows}


def ve_backward(dv: np.ndarray, xn: np.ndarray, ids: np.ndarray, wg: np.ndarray, V: int, c: dict) -> dict:
    """Backward of `ve_forward` given dv (the gradient w.r.t. the updated v,
    which also flows unchanged to the projection's v): the gate logits'
    gradient ds, dwg = sum over tokens of ds (x) xn[..., :nc], the extra
    gradient of xn, and the table's rows dve (repeated ids add up)."""
    B, T, Hkv, D = dv.shape
    nc = wg.shape[1]
    dgate = np.sum(dv * c["ve_rows"], axis=-1)                   # [B, T, Hkv]
    sg = _sigmoid(c["ve_s"])
    ds = dgate * 3.0 * sg * (1.0 - sg)
    dwg = np.einsum("bth,btc->hc", ds, xn[..., :nc])
    dxn = np.zeros_like(xn)
    dxn[..., :nc] = ds @ wg
    dve = np.zeros((V, Hkv * D))
    np.add.at(dve, ids.reshape(-1), (dv * c["ve_gate"][..., None]).reshape(B * T, Hkv * D))
    # per element, the sum over tokens of the summed terms' magnitudes (the
    # scale of that sum's forward error bound)
    dwg_abs = np.einsum("bth,btc->hc", np.abs(ds), np.abs(xn[..., :nc]))
    return {"ds": ds, "dwg": dwg, "dxn": dxn, "dve": dve, "dwg_sum_abs": dwg_abs}


def backout_forward(x: np.ndarray, x_bo: np.ndarray, lam: float) -> np.ndarray:
    """Backout ([FR] the backout snippet): x - lam * x_bo before the final norm."""
    return x - lam * x_bo


def backout_backward(dy: np.ndarray, x_bo: np.ndarray, lam: float) -> dict:
    """Gradients of y = x - lam*x_bo: dx = dy, dx_bo = -lam*dy, dlam = -sum(dy*x_bo)."""
    return {"dx_bo": -lam * dy, "dlam": -float(np.sum(dy * x_bo)), "sum_abs": float(np.sum(np.abs(dy * x_bo)))}


# ------------------------------------------------------------------- block


def block_forward(x: np.ndarray, p: Dict[str, np.ndarray], cfg, l: int,
                  cos: np.ndarray, sin: np.ndarray,
                  x0: Optional[np.ndarray] = None,
                  ids: Optional[np.ndarray] = None) -> Tuple[np.ndarray, dict]:
    """One pre-norm decoder block on x [B, T, C] (all float64).

    [d26 extras: x <- resid_lambda*x + x0_lambda*x0 first; on odd layers
    v += 3*sigmoid(xn1[..., :32] @ W_g^T) * VE[ids] per K/V head.]
    xn1 = rms(x); q,k,v = xn1 W_qkv^T; qh = rope(rms_D(q)), kh = rope(rms_D(k));
    o = attn(qh, kh, v); x_mid = x + o W_o^T; xn2 = rms(x_mid);
    u = xn2 W_fc^T; h = relu(u)^2; out = x_mid + h W_proj^T.
    """
    B, T, C = x.shape
    H, Hkv, D = cfg.n_head, cfg.n_kv_head, cfg.head_dim
    Q, KV = H * D, Hkv * D
    eps, window = cfg.eps, cfg.windows[l]
    fp8 = bool(getattr(cfg, "mlp_fp8", False))
    c = {}
    if cfg.extras:
        c["x_premix"], c["x0"] = x, x0
        x = mix_forward(x, x0, p["resid_lambda"], p["x0_lambda"])
    c["x_in"] = x
    xn1, r1 = rms_norm(x, eps)
    qkv = xn1 @ p["w_qkv"].T
    q = qkv[..., :Q].reshape(B, T, H, D)
    k = qkv[..., Q:Q + KV].reshape(B, T, Hkv, D)
    v = qkv[..., Q + KV:].reshape(B, T, Hkv, D)
    if cfg.extras and "ve" in p:
        v, cv = ve_forward(xn1, v, ids, p["ve"], p["ve_gate"])
        c.update(cv)
    qn, rq = rms_norm(q, eps)
    kn, rk = rms_norm(k, eps)
    qh, kh = rope(qn, cos, sin), rope(kn, cos, sin)
    o, P = attention(qh, kh, v, window)
    o2 = o.reshape(B, T, Q)
    x_mid = x + o2 @ p["w_o"].T
    xn2, r2 = rms_norm(x_mid, eps)
    st = getattr(cfg, "dtype", None)
    u = mm_nt(xn2, p["w_fc"], fp8, st)
    h = relu2(u)
    out = x_mid + mm_nt(h, p["w_proj"], fp8, st)
    c.update(xn1=xn1, r1=r1, qn=qn, rq=rq, kn=kn, rk=rk, qh=qh, kh=kh, v=v, o=o2,
             P=P, x_mid=x_mid, xn2=xn2, r2=r2, u=u, h=h)
    return out, c


def block_backward(dout: np.ndarray, c: dict, p: Dict[str, np.ndarray], cfg, l: int,
                   cos: np.ndarray, sin: np.ndarray,
                   ids: Optional[np.ndarray] = None) -> Tuple[np.ndarray, dict]:
    """Reverse of `block_forward`.  Returns dx (w.r.t. the block input; with
    the extras, w.r.t. the pre-mix stream) and a dict of float64 gradients
    (w_qkv, w_o, w_fc, w_proj[, resid_lambda, x0_lambda, x0, ve, ve_gate])."""
    B, T, C = dout.shape
    H, Hkv, D = cfg.n_head, cfg.n_kv_head, cfg.head_dim
    Q, KV = H * D, Hkv * D
    fp8 = bool(getattr(cfg, "mlp_fp8", False))
    g = {}
    st = getattr(cfg, "dtype", None)
    q8 = (lambda a: fp8_quant_dequant(a, st)) if fp8 else (lambda a: a)
    # MLP: out = x_mid + h W_proj^T, h = relu(u)^2, u = xn2 W_fc^T
    dh = q8(dout) @ q8(p["w_proj"])
    g["w_proj"] = np.einsum("btc,btf->cf", q8(dout), q8(c["h"]))
    du = dh * relu2_grad(c["u"])
    dxn2 = q8(du) @ q8(p["w_fc"])
    g["w_fc"] = np.einsum("btf,btc->fc", q8(du), q8(c["xn2"]))
    dx_mid = dout + rms_norm_backward(dxn2, c["xn2"], c["r2"])
    # attention output projection
    do2 = dx_mid @ p["w_o"]
    g["w_o"] = np.einsum("btc,btq->cq", dx_mid, c["o"])
    dqh, dkh, dv = attention_backward(do2.reshape(B, T, H, D), c["qh"], c["kh"], c["v"], c["P"])
    dq = rms_norm_backward(rope_backward(dqh, cos, sin), c["qn"], c["rq"])
    dk = rms_norm_backward(rope_backward(dkh, cos, sin), c["kn"], c["rk"])
    dxn1_extra = 0.0
    if cfg.extras and "ve" in p:
        gv = ve_backward(dv, c["xn1"], ids, p["ve_gate"], p["ve"].shape[0], c)
        g["ve_gate"], g["ve"], dxn1_extra = gv["dwg"], gv["dve"], gv["dxn"]
        ve_gate_sum_abs = gv["dwg_sum_abs"]
    dqkv = np.concatenate([dq.reshape(B, T, Q), dk.reshape(B, T, KV), dv.reshape(B, T, KV)], -1)
    dxn1 = dqkv @ p["w_qkv"] + dxn1_extra
    g["w_qkv"] = np.einsum("btk,btc->kc", dqkv, c["xn1"])
    dx = dx_mid + rms_norm_backward(dxn1, c["xn1"], c["r1"])
    if cfg.extras:
        gm = mix_backward(dx, c["x_premix"], c["x0"], p["resid_lambda"], p["x0_lambda"])
        g["resid_lambda"], g["x0_lambda"] = gm["da"], gm["db"]
        g["sum_abs"] = {"resid_lambda": gm["sum_abs"]["da"], "x0_lambda": gm["sum_abs"]["db"]}
        if "ve" in p:
            g["sum_abs"]["ve_gate"] = ve_gate_sum_abs
        g["x0"] = gm["dx0"]
        dx = gm["dx"]
    return dx, g


# ------------------------------------------------------- head + loss, embed
def cross_entropy(z: np.ndarray, y: np.ndarray) -> Tuple[float, np.ndarray, np.ndarray, np.ndarray]:
    """Mean next-token cross-entropy on logits z [N, V] with targets y [N]:
    row_loss = logsumexp(z_n) - z_n[y_n]; loss = mean(row_loss);
    dz = (softmax(z) - onehot(y)) / N.  Returns loss, row_loss, dz, lse."""
    N = z.shape[0]
    m = z.max(axis=1)
    lse = m + np.log(np.sum(np.exp(z - m[:, None]), axis=1))
    row_loss = lse - z[np.arange(N), y]
    dz = np.exp(z - lse[:, None])
    dz[np.arange(N), y] -= 1.0
    dz /= N
    return float(np.mean(row_loss)), row_loss, dz, lse


def lm_head_ce(x: np.ndarray, w_lm: np.ndarray, targets: np.ndarray, eps: float
               ) -> Tuple[float, np.ndarray, np.ndarray, dict]:
    """xf = rms(x); z = xf W_lm^T; loss = mean_n(logsumexp(z_n) - z_n[y_n]).
    Returns loss, dx (w.r.t. the pre-norm x), dW_lm and a cache
    (z, lse, dz = (softmax(z) - onehot(y)) / N)."""
    shp = x.shape
    x2 = x.reshape(-1, shp[-1])
    y = targets.reshape(-1)
    N = x2.shape[0]
    xf, rf = rms_norm(x2, eps)
    z = xf @ w_lm.T
    loss, row_loss, dz, lse = cross_entropy(z, y)
    dxf = dz @ w_lm
    dw = dz.T @ xf
    dx = rms_norm_backward(dxf, xf, rf).reshape(shp)
    return loss, dx, dw, {"z": z, "lse": lse, "dz": dz, "xf": xf, "rf": rf}


def embed_forward(wte: np.ndarray, ids: np.ndarray) -> np.ndarray:
    return wte[ids]


def embed_backward(dx: np.ndarray, ids: np.ndarray, V: int) -> np.ndarray:
    """dWte[v] = sum of dx rows whose id is v."""
    C = dx.shape[-1]
    dw = np.zeros((V, C))
    np.add.at(dw, ids.reshape(-1), dx.reshape(-1, C))
    return dw


def smear_forward(e: np.ndarray, w_s: np.ndarray, lam: float) -> Tuple[np.ndarray, dict]:
    """x_t = e_t + lam * sigmoid(w_s . e_t[:n]) * e_{t-1} for t >= 1; x_0 = e_0.
    e [B, T, C]; the gate reads the current token, the mixed vector is the
    previous token's embedding."""
    n = w_s.shape[0]
    s = e[..., :n] @ w_s                     # [B, T]
    sg = _sigmoid(s)
    prev = np.zeros_like(e)
    prev[:, 1:] = e[:, :-1]
    gate = lam * sg
    gate[:, 0] = 0.0
    return e + gate[..., None] * prev, {"s": s, "sg": sg, "prev": prev, "gate": gate}


def smear_backward(dx: np.ndarray, e: np.ndarray, w_s: np.ndarray, lam: float, c: dict
                   ) -> Tuple[np.ndarray, np.ndarray, float]:
    n = w_s.shape[0]
    de = dx.copy()
    de[:, :-1] += c["gate"][:, 1:, None] * dx[:, 1:]
    dgate = np.sum(dx * c["prev"], axis=-1)           # [B, T]
    dgate[:, 0] = 0.0
    dlam = float(np.sum(dgate * c["sg"]))
    ds = dgate * lam * c["sg"] * (1.0 - c["sg"])
    dws = np.einsum("bt,btc->c", ds, e[..., :n])
    de[..., :n] += ds[..., None] * w_s
    return de, dws, dlam


# ------------------------------------------------------------------- stack
def stack_forward_backward(cfg, ids: np.ndarray, glob: Dict[str, np.ndarray],
                           layers: List[Dict[str, np.ndarray]], keep: bool = False,
                           stream_dtype: Optional[str] = None):
    """Full step on ids [B, T+1]: embedding [-> smear], L blocks [with residual
    mixing, value embeddings, backout], final rms, lm_head, mean next-token
    cross-entropy; then the backward of all of it.  Returns (loss, grads,
    acts) where grads has 'wte', 'w_lm', 'layers' (list of dicts) [and the
    extras' scalars], and acts (if keep) holds each block's input stream.

    stream_dtype="bf16" stores the residual streams between blocks as bf16
    values, as a model with explicit bf16 activations does (section "3.
    Gestion de la précision"): the stream entering the first block, every
    block's output, the head's input gradient and every block's input
    gradient are rounded to bf16; everything else stays exact.  Used only to
    measure how far that storage alone moves each result over depth (the
    bound of the full-depth parity tests); the default is the exact oracle."""
    if stream_dtype not in (None, "bf16"):
        raise ValueError(f"stream_dtype {stream_dtype!r}")
    store = bf16_round if stream_dtype == "bf16" else (lambda a: a)
    B, T1 = ids.shape
    T = T1 - 1
    inp, tgt = ids[:, :T], ids[:, 1:]
    L = cfg.n_layer
    cos, sin = rope_tables(T, cfg.head_dim, cfg.rope_base)
    f64 = lambda a: np.asarray(a, dtype=np.float64)
    glob = {k: f64(v) for k, v in glob.items()}
    layers = [{k: f64(v) for k, v in p.items()} for p in layers]
    e = embed_forward(glob["wte"], inp)
    x0 = None
    if cfg.extras:
        x, sc = smear_forward(e, glob["smear_gate"], float(np.ravel(glob["smear_lambda"])[0]))
        x = store(x)
        x0 = x
    else:
        x = store(e)
    caches, acts = [], []
    i_bo = L // 2 - 1
    x_bo = None
    for l in range(L):
        acts.append(x)
        x, c = block_forward(x, layers[l], cfg, l, cos, sin, x0=x0, ids=inp)
        x = store(x)
        caches.append(c)
        if cfg.extras and l == i_bo:
            x_bo = x
    acts.append(x)
    if cfg.extras:
        x_final = backout_forward(x, x_bo, glob["backout_lambda"])
    else:
        x_final = x
    loss, dx, dw_lm, hc = lm_head_ce(x_final, glob["w_lm"], tgt, cfg.eps)
    dx = store(dx)
    grads = {"w_lm": dw_lm, "layers": [None] * L}
    if cfg.extras:
        gb = backout_backward(dx, x_bo, glob["backout_lambda"])
        grads["backout_lambda"] = gb["dlam"]
        sum_abs = {"backout_lambda": gb["sum_abs"]}
        dx_bo = gb["dx_bo"]
        dx0 = np.zeros_like(dx)
    for l in reversed(range(L)):
        if cfg.extras and l == i_bo:
            dx = dx + dx_bo
        dx, g = block_backward(dx, caches[l], layers[l], cfg, l, cos, sin, ids=inp)
        dx = store(dx)
        if cfg.extras:
            dx0 += g.pop("x0")
        grads["layers"][l] = g
    if cfg.extras:
        dx = dx + dx0
        de, dws, dlam = smear_backward(dx, e, glob["smear_gate"], float(np.ravel(glob["smear_lambda"])[0]), sc)
        grads["smear_gate"] = dws
        grads["smear_lambda"] = dlam
        sum_abs["smear_lambda"] = float(np.sum(np.abs(np.sum(dx * sc["prev"], axis=-1) * sc["sg"])))
        # the gate weight gradient nests two sums (over channels into each
        # token's gate input, then over tokens): the magnitudes of both levels'
        # terms, per gate channel
        lam_s = float(np.ravel(glob["smear_lambda"])[0])
        inner = np.sum(np.abs(dx * sc["prev"]), axis=-1)
        inner[:, 0] = 0.0
        n_s = glob["smear_gate"].shape[0]
        sum_abs["smear_gate"] = np.einsum("bt,btc->c", inner * np.abs(lam_s * sc["sg"] * (1.0 - sc["sg"])),
                                          np.abs(e[..., :n_s]))
    else:
        de = dx
    grads["wte"] = embed_backward(de, inp, glob["wte"].shape[0])
    out = {"head": hc, "x_final": x_final}
    if cfg.extras:
        out["sum_abs"] = sum_abs
    if keep:
        out["acts"] = acts
        out["caches"] = caches
    return loss, grads, out
