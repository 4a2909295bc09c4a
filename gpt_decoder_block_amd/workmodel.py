"""Algorithmic work of one training step: FLOPs of the contractions and bytes
of the bandwidth-bound kernels, per workload.

Two FLOP conventions are provided:
  * algorithmic (primary): 2*M*N*K per GEMM, forward + 2x for the backward;
    attention counts only the visible (query, key) pairs of the causal
    triangle or the window band: 4*D per pair per head forward (QK^T and PV),
    8*D backward (dV, dP, dQ, dK); the backward's recompute of S is hardware
    work and is not counted;
  * the pages' convention: 6 * (matrix parameters) + 12 * H * D * W per token
    per layer with W the window (T for a full layer), no causal halving.  This
    is the convention that reproduces the total training FLOPs printed in the
    run summary of "nanochat：仅需73美元，3小时训练GPT-2级别大语言模型", section
    "排行榜" (d24, 16 704 steps of 2^19 tokens).
"""
from __future__ import annotations

from typing import Dict, Sequence


def attn_pairs(T: int, W: int) -> int:
    """Visible (i, j) pairs of one sequence: j <= i and (W < 0 or i - j <= W)."""
    if W < 0 or W >= T - 1:
        return T * (T + 1) // 2
    # rows i < W see i + 1 keys, rows i >= W see W + 1 keys
    return W * (W + 1) // 2 + (T - W) * (W + 1)


def matrix_params(n_layer: int, C: int, H: int, Hkv: int, D: int, F: int, V: int) -> int:
    """Block matrices plus lm_head (the token embedding is a lookup, not a matmul)."""
    Q, KV = H * D, Hkv * D
    return n_layer * (C * (Q + 2 * KV) + Q * C + 2 * C * F) + V * C


def flops_per_token(n_layer, C, H, Hkv, D, F, V, T, windows: Sequence[int]) -> float:
    """Algorithmic fwd+bwd FLOPs per token (causal-exact attention)."""
    mm = 6 * matrix_params(n_layer, C, H, Hkv, D, F, V)
    att = sum(12 * D * H * attn_pairs(T, w) for w in windows) / T
    return mm + att


def flops_per_token_pages(n_layer, C, H, Hkv, D, F, V, T, windows: Sequence[int],
                          extra_params: int = 0) -> int:
    """The pages' convention: 6 * params + sum over layers of 12*H*D*W_eff."""
    mm = 6 * (matrix_params(n_layer, C, H, Hkv, D, F, V) + extra_params)
    att = sum(12 * H * D * (T if (w < 0 or w >= T) else w) for w in windows)
    return mm + att


def step_flops(w) -> Dict[str, float]:
    """Split of algorithmic FLOPs per step for a workload `w` (seeded_inputs.Workload
    or anything with the same fields)."""
    N = w.B * w.T
    Q, KV = w.n_head * w.head_dim, w.n_kv_head * w.head_dim
    C, F, V, L = w.C, w.mlp_hidden, w.vocab, w.n_layer
    gemm_fwd = 2 * N * (C * (Q + 2 * KV) + Q * C + 2 * C * F)
    head_fwd = 2 * N * V * C
    att_fwd = [4 * w.head_dim * w.n_head * w.B * attn_pairs(w.T, win) for win in w.windows]
    return {
        "block_gemm": 3.0 * L * gemm_fwd,
        "lm_head": 3.0 * head_fwd,
        "attention": 3.0 * sum(att_fwd),
        "attention_fwd_per_layer": att_fwd,
        "total": 3.0 * (L * gemm_fwd + head_fwd + sum(att_fwd)),
    }


def bytes_rmsnorm_fwd(N: int, C: int, s: int) -> int:
    """read x, write xn (s bytes each element) + write the fp32 inverse RMS."""
    return 2 * N * C * s + 4 * N


def bytes_rmsnorm_bwd(N: int, C: int, s: int, residual: bool = True) -> int:
    """read dxn, xn, (residual grad), write dx; read r."""
    return (4 if residual else 3) * N * C * s + 4 * N


def bytes_ce(N: int, V: int, s: int) -> int:
    """read logits once, write dlogits once, read targets, write per-row loss."""
    return N * V * 2 * s + 8 * N
