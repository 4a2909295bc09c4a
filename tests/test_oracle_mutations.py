"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch each one: a dropped term, a wrong sign, an off-by-one, a transposed
operand.  Every mutant must fail the torch-autograd cross-check or the
finite-difference check."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle.reference as R
from test_oracle_pins import _params, tiny_cfg
from test_oracle_vs_torch import _compare


def _mut_rms_bwd(dy, y, r):          # dropped projection term
    return r[..., None] * dy


def _mut_rope(x, cos, sin):          # wrong rotation sign in the forward only
    D = x.shape[-1]
    a, b = x[..., : D // 2], x[..., D // 2:]
    c, s = cos[None, :, None, :], sin[None, :, None, :]
    return np.concatenate([a * c + b * s, -a * s + b * c], axis=-1)


def _mut_mask(T, window):            # window off by one (i - j < W)
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    m = j <= i
    if window >= 0:
        m &= (i - j) < window
    return m


_orig_attn_bwd = R.attention_backward


def _mut_attn_bwd(do, q, k, v, P):  # transposed P in dV
    dq, dk, dv = _orig_attn_bwd(do, q, k, v, P)
    B, T, H, D = q.shape
    Hkv = k.shape[2]
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            dv[b, :, h // (H // Hkv)] += P[b, h] @ do[b, :, h]
    return dq, dk, dv


def _mut_kv_head(h, H, Hkv):         # interleaved instead of contiguous head groups
    return h % Hkv


_orig_ce = R.lm_head_ce


def _mut_ce(x, w, t, eps):           # loss not divided by N in the gradient
    loss, dx, dw, c = _orig_ce(x, w, t, eps)
    n = x.reshape(-1, x.shape[-1]).shape[0]
    return loss, dx * n, dw * n, c


MUTANTS = [("rms_norm_backward", _mut_rms_bwd), ("rope", _mut_rope),
           ("visible_mask", _mut_mask), ("attention_backward", _mut_attn_bwd),
           ("_kv_head", _mut_kv_head), ("lm_head_ce", _mut_ce)]


@pytest.mark.parametrize("name,fn", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(monkeypatch, name, fn):
    cfg = tiny_cfg(n_head=4, n_kv_head=2, head_dim=4, windows=(3, -1), T=9)
    ids, glob, layers = _params(cfg, np.random.default_rng(13))
    _compare(cfg, ids, glob, layers)            # unmutated: passes
    monkeypatch.setattr(R, name, fn)
    with pytest.raises(AssertionError):
        _compare(cfg, ids, glob, layers)


# decode attention: each mutant must fail the torch SDPA pin
_orig_decode = R.attention_decode


def _mut_decode_window(q, k, v, lens, window):   # window lower bound off by one
    return _orig_decode(q, k, v, lens, window + 1 if window >= 0 else window)


def _mut_decode_scale(q, k, v, lens, window):    # softmax scale 1/D instead of 1/sqrt(D)
    return _orig_decode(q / np.sqrt(q.shape[-1]), k, v, lens, window)


def _mut_decode_last_key(q, k, v, lens, window):  # the query's own key left out
    o, lse = _orig_decode(q, k, v, np.asarray(lens) - 1, window - 1 if window > 0 else window)
    return o, lse


DECODE_MUTANTS = [_mut_decode_window, _mut_decode_scale, _mut_decode_last_key]


@pytest.mark.parametrize("fn", DECODE_MUTANTS, ids=[f.__name__ for f in DECODE_MUTANTS])
def test_decode_pins_catch_mutant(monkeypatch, fn):
    import test_oracle_pins as P
    P.test_decode_against_torch_sdpa(4)          # unmutated: passes
    monkeypatch.setattr(R, "attention_decode", fn)
    monkeypatch.setattr(P.O, "attention_decode", fn)
    with pytest.raises(AssertionError):
        P.test_decode_against_torch_sdpa(4)


# optimizer: each mutant must fail its closed-form or torch pin
import oracle.optim as OPT

_orig_ns = OPT.newton_schulz


def _mut_ns_gram_side(G, coeffs, norm_scale=1.0, eps=1e-7):   # X B replaced by B X (square case)
    X = np.asarray(G, dtype=np.float64)
    X = X / (np.linalg.norm(X) * norm_scale + eps)
    for a, b, c in coeffs:
        A = X.T @ X
        X = a * X + (b * A + c * (A @ A)) @ X
    return X


def _mut_ns_no_norm(G, coeffs, norm_scale=1.0, eps=1e-7):      # missing the Frobenius normalisation
    return _orig_ns(np.asarray(G) * np.linalg.norm(G), coeffs, norm_scale, eps)


_orig_adamw = OPT.adamw_step


def _mut_adamw_no_bias_corr(p, g, m, v, t, lr, beta1, beta2, eps, wd):
    return _orig_adamw(p, g, m, v, 10 ** 6, lr, beta1, beta2, eps, wd)


def _mut_adamw_coupled_decay(p, g, m, v, t, lr, beta1, beta2, eps, wd):   # L2 penalty instead of decoupled decay
    return _orig_adamw(p, g + wd * np.asarray(p), m, v, t, lr, beta1, beta2, eps, 0.0)


@pytest.mark.parametrize("fn", [_mut_ns_gram_side, _mut_ns_no_norm], ids=["gram_side", "no_norm"])
def test_newton_schulz_pin_catches_mutant(monkeypatch, fn):
    import test_oracle_pins as P
    P.test_newton_schulz_svd_closed_form((12, 12), P.PE_PRINTED)
    monkeypatch.setattr(P.O, "newton_schulz", fn)
    with pytest.raises(AssertionError):
        P.test_newton_schulz_svd_closed_form((12, 12), P.PE_PRINTED)


@pytest.mark.parametrize("fn", [_mut_adamw_no_bias_corr, _mut_adamw_coupled_decay], ids=["bias_corr", "decay"])
def test_adamw_pin_catches_mutant(monkeypatch, fn):
    import test_oracle_pins as P
    P.test_adamw_against_torch()
    monkeypatch.setattr(P.O, "adamw_step", fn)
    with pytest.raises(AssertionError):
        P.test_adamw_against_torch()
