"""Plain float64 CPU oracle of the optimizer step that follows the backward.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (page title, then section):
  [JA] the Japanese version of the French article on dev.to, section
       "2. Muonオプティマイザー（nanochat/optim.py）": embeddings, lm_head and
       scalar parameters take AdamW, 2-D matrices take Muon; the Polar Express
       Newton-Schulz loop (A = X^T X; B = b A + c A^2; X = a X + X B) with the
       first two of its coefficient triples.
  [FR] "Comment Entraîner Votre Propre ChatGPT Pour 50€ ?", section "2.
       L'optimiseur Muon (nanochat/optim.py)": the same loop, five iterations,
       Muon read as momentum orthogonalised by that iteration.

Readings taken where the pages are silent:
  * the iteration starts from X0 = G / (||G||_F * norm_scale + eps): the
    polynomial steps only act as intended on singular values in (0, 1], and
    the Frobenius norm bounds the largest one; norm_scale and eps are inputs;
  * the coefficient table is an input (the pages print two of the five
    triples); tests use the two printed ones and synthetic tables;
  * Muon: buf <- momentum * buf + g; the orthogonalised matrix is that of
    g + momentum * buf (Nesterov) or of buf; p <- p * (1 - lr * wd) -
    lr * scale * NS(.), with the shape-dependent scale an input;
  * AdamW is the decoupled-weight-decay Adam with bias correction (the
    textbook method, as torch.optim.AdamW computes it);
  * NorMuon ([FR] and [JA], the "variance reduction" snippet: four printed
    lines in which `red_dim`, `step_size` and `v_norm_new` are not defined):
    g is the orthogonalised update; the statistic is per output neuron, i.e.
    the mean of g^2 over the input dimension of each row of a [out, in]
    weight (red_dim = the last axis); step_size is per neuron, the inverse
    square root of a second moment v kept across steps (v <- beta2 v +
    (1 - beta2) v_mean, floored at 1e-10) -- the snippet's final scale must
    vary per neuron for the update to be "normalised per neuron"; v_norm_new
    is v_norm's formula applied to the rescaled update, sqrt(sum v_mean *
    step^2), so the final scale keeps the update's Frobenius norm.

Pins (tests/test_oracle_pins.py): NorMuon keeps the Frobenius norm of the
orthogonalised update, gives every row the same RMS when beta2 = 0, and is
Muon when the rows already share one RMS and v holds it; Newton-Schulz against the SVD closed form
(singular vectors kept, each singular value through the composed
polynomial), the transpose identity NS(G^T) = NS(G)^T, the classic cubic
iteration converging to the polar factor U V^T; AdamW against
torch.optim.AdamW over several steps; Muon with momentum 0 and no decay
reduces to a Newton-Schulz step.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

from .reference import bf16_round

__all__ = ["newton_schulz", "adamw_step", "muon_step", "normuon_scale", "normuon_step"]


def newton_schulz(G: np.ndarray, coeffs: Sequence[Tuple[float, float, float]], norm_scale: float = 1.0,
                  eps: float = 1e-7, round_to: Optional[str] = None) -> np.ndarray:
    """The pages' orthogonalisation loop on G [m, n], one (a, b, c) triple per
    iteration, starting from the Frobenius-normalised G.

    round_to="bf16" rounds the normalised input and the result of each of the
    three lines to bfloat16 (an iteration run in bf16 storage with exact
    arithmetic inside each line), in the pages' orientation (Gram X^T X of the
    given G); used only to measure how far bf16 storage alone moves the exact
    map, never as the reference.  The exact map is the same for G and for the
    transposed problem, the storage rounding is not, so a bar built from this
    takes the larger move over both orientations."""
    X = np.asarray(G, dtype=np.float64)
    rnd = bf16_round if round_to == "bf16" else (lambda a: a)
    if round_to not in (None, "bf16"):
        raise ValueError(f"round_to must be None or 'bf16' (got {round_to!r})")
    X = rnd(X / (np.linalg.norm(X) * norm_scale + eps))
    for a, b, c in coeffs:
        A = rnd(X.T @ X)
        B = rnd(b * A + c * (A @ A))
        X = rnd(a * X + X @ B)
    return X


def adamw_step(p, g, m, v, t: int, lr: float, beta1: float, beta2: float, eps: float, wd: float):
    """One AdamW step (decoupled weight decay, bias-corrected moments); t >= 1
    counts steps including this one.  Returns the new (p, m, v)."""
    p = np.asarray(p, dtype=np.float64) * (1.0 - lr * wd)
    m = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * np.square(g)
    mhat = m / (1.0 - beta1 ** t)
    vhat = v / (1.0 - beta2 ** t)
    p = p - lr * mhat / (np.sqrt(vhat) + eps)
    return p, m, v


def muon_step(p, g, buf, lr: float, momentum: float, nesterov: bool, wd: float, scale: float,
              coeffs: Sequence[Tuple[float, float, float]], norm_scale: float = 1.0, eps: float = 1e-7):
    """One Muon step on a matrix parameter p [m, n] with gradient g and
    momentum buffer buf.  Returns the new (p, buf)."""
    buf = momentum * np.asarray(buf, dtype=np.float64) + g
    u = g + momentum * buf if nesterov else buf
    o = newton_schulz(u, coeffs, norm_scale, eps)
    p = np.asarray(p, dtype=np.float64) * (1.0 - lr * wd) - lr * scale * o
    return p, buf


def normuon_scale(o: np.ndarray, v: np.ndarray, beta2: float) -> Tuple[np.ndarray, np.ndarray]:
    """The per-neuron variance normalisation of an orthogonalised update o
    [m, n] (rows = output neurons) with per-neuron second moment v [m].
    Returns (the normalised update, the new v)."""
    o = np.asarray(o, dtype=np.float64)
    v_mean = np.mean(o * o, axis=-1)                     # per neuron
    v_norm = math.sqrt(float(np.sum(v_mean)))
    v = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * v_mean
    step = 1.0 / np.sqrt(np.maximum(v, 1e-10))
    v_norm_new = math.sqrt(float(np.sum(v_mean * step * step)))
    final = step * (v_norm / max(v_norm_new, 1e-10))
    return o * final[:, None], v


def normuon_step(p, g, buf, v, lr: float, momentum: float, nesterov: bool, wd: float, scale: float, beta2: float,
                 coeffs: Sequence[Tuple[float, float, float]], norm_scale: float = 1.0, eps: float = 1e-7):
    """One Muon step whose orthogonalised update goes through
    `normuon_scale` first.  Returns the new (p, buf, v)."""
    buf = momentum * np.asarray(buf, dtype=np.float64) + g
    u = g + momentum * buf if nesterov else buf
    o, v = normuon_scale(newton_schulz(u, coeffs, norm_scale, eps), v, beta2)
    p = np.asarray(p, dtype=np.float64) * (1.0 - lr * wd) - lr * scale * o
    return p, buf, v
