"""Seeded synthetic workloads for the decoder-block training step.

This module describes the workload shapes and draws their random inputs
(token ids, weight matrices, per-layer scalars).  It is the only code shared by
the HIP path (via tests and bench) and the CPU oracle, and it holds none of the
method's arithmetic: it only draws numbers and rounds them to the storage dtype.

Shapes follow the decoder described in "nanochat: обучи GPT-2 уровня за $48"
and "Comment Entraîner Votre Propre ChatGPT Pour 50€ ?" (section "1. Le modèle
GPT": RoPE, QK norm, untied embedding/lm_head, ReLU² MLP, GQA, sliding window),
at the depths the pages train (d12 trial runs, the d24 leaderboard run and the
d26 fp8 run), plus the d24 record run's own model (the sliding-window pattern
"SSSL" of section "1. Le modèle GPT" with every extra).  Every weight matrix is drawn N(0, 0.02^2); per-layer scalars of
the d26 extras are drawn U(0.5, 1.5); token ids are uniform over the vocabulary.

Each tensor has its own random stream keyed by (seed, tensor kind, layer), so a
caller can draw layer l alone, and a workload cut to fewer layers or a smaller
batch gets exactly the same values for what remains.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Dict, Optional, Tuple

import numpy as np

__all__ = ["Workload", "WORKLOADS", "workload", "draw_ids", "draw_layer",
           "draw_globals", "draw_all", "to_dtype", "draw_normal", "draw_ids_zipf", "sssl_windows"]

# stream ids for SeedSequence keys
_K_IDS, _K_WTE, _K_WLM, _K_QKV, _K_O, _K_FC, _K_PROJ = 1, 2, 3, 4, 5, 6, 7
_K_VE, _K_VEGATE, _K_SCAL, _K_SMEAR, _K_DX = 8, 9, 10, 11, 12
INIT_STD = 0.02


@dataclass(frozen=True)
class Workload:
    name: str
    n_layer: int
    B: int
    T: int
    C: int
    n_head: int
    n_kv_head: int
    head_dim: int
    mlp_hidden: int
    vocab: int
    windows: Tuple[int, ...]  # per layer; -1 means full causal attention
    dtype: str                # "f32" or "bf16": storage/compute dtype of the path
    seed: int
    rope_base: float = 10000.0
    eps: float = 1e-6
    extras: bool = False      # residual mixing, value embeddings, smear, backout
    mlp_fp8: bool = False     # MLP GEMM operands in OCP e4m3 with per-tensor scales
    ve_gate_channels: int = 32
    smear_channels: int = 24

    @property
    def N(self) -> int:
        return self.B * self.T

    @property
    def qkv_width(self) -> int:
        return (self.n_head + 2 * self.n_kv_head) * self.head_dim

    def with_(self, **kw) -> "Workload":
        if "n_layer" in kw and "windows" not in kw:
            kw["windows"] = self.windows[: kw["n_layer"]]
        return dataclasses.replace(self, **kw)


def _alt_windows(n_layer: int, w: int) -> Tuple[int, ...]:
    # odd (0-based) layers windowed, even layers full causal
    return tuple(w if (l % 2 == 1) else -1 for l in range(n_layer))


def sssl_windows(n_layer: int, short: int) -> Tuple[int, ...]:
    """The repeating short-short-short-long layer pattern: layers l with
    l % 4 < 3 get the short window, every fourth layer and the last one full
    causal attention (the long context equals T here)."""
    return tuple(-1 if (l % 4 == 3 or l == n_layer - 1) else short for l in range(n_layer))


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 1, 1, 64, 128, 2, 1, 64, 512, 512, (-1,), "f32", 1001),
    "d12": Workload("d12", 12, 16, 2048, 768, 6, 6, 128, 3072, 32768,
                    (-1,) * 12, "bf16", 1002),
    "d12_gqa_swa": Workload("d12_gqa_swa", 12, 16, 2048, 768, 6, 2, 128, 3072, 32768,
                            _alt_windows(12, 1024), "bf16", 1003),
    "d24": Workload("d24", 24, 16, 2048, 1536, 12, 12, 128, 6144, 32768,
                    _alt_windows(24, 1024), "bf16", 1004),
    "d26": Workload("d26", 26, 16, 2048, 1664, 13, 13, 128, 6656, 32768,
                    (-1,) * 26, "bf16", 1005, extras=True, mlp_fp8=True),
    # the d24 record run's model: SSSL windows (short 1024, long = T), value
    # embeddings on alternating layers, residual mixing, smear and backout, bf16
    "d24_record": Workload("d24_record", 24, 16, 2048, 1536, 12, 12, 128, 6144, 32768,
                           sssl_windows(24, 1024), "bf16", 1006, extras=True),
}


def workload(name: str, **overrides) -> Workload:
    return WORKLOADS[name].with_(**overrides) if overrides else WORKLOADS[name]


def _rng(seed: int, kind: int, layer: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, kind, layer]))


def draw_normal(seed: int, kind: int, layer: int, shape, std: float = INIT_STD) -> np.ndarray:
    """float32 draws of N(0, std^2) from the stream (seed, kind, layer)."""
    g = _rng(seed, kind, layer)
    out = g.standard_normal(size=shape, dtype=np.float32)
    out *= np.float32(std)
    return out


def draw_ids(w: Workload) -> np.ndarray:
    """Token ids [B, T+1], uniform on [0, vocab).  Inputs are ids[:, :T] and
    next-token targets ids[:, 1:].  Row b is the same for any B > b."""
    rows = [_rng(w.seed, _K_IDS, b).integers(0, w.vocab, size=w.T + 1, dtype=np.int64)
            for b in range(w.B)]
    return np.stack(rows, 0)


def draw_ids_zipf(w: Workload, a: float = 1.0) -> np.ndarray:
    """Zipf(a)-distributed ids [B, T+1] (a stand-in for natural-text contention in
    the embedding scatter), ranks mapped to ids by a seeded permutation."""
    g = _rng(w.seed, _K_IDS, 10_000)
    ranks = np.arange(1, w.vocab + 1, dtype=np.float64)
    p = ranks ** (-a)
    p /= p.sum()
    perm = g.permutation(w.vocab)
    return perm[g.choice(w.vocab, size=(w.B, w.T + 1), p=p)].astype(np.int64)


def draw_layer(w: Workload, l: int) -> Dict[str, np.ndarray]:
    """float32 draws for block l: w_qkv [Q+2KV, C] (rows q; k; v, head-major),
    w_o [C, Q], w_fc [F, C], w_proj [C, F]; plus the extras of the d26 shape."""
    C, F = w.C, w.mlp_hidden
    Q, KV = w.n_head * w.head_dim, w.n_kv_head * w.head_dim
    out = {
        "w_qkv": draw_normal(w.seed, _K_QKV, l, (Q + 2 * KV, C)),
        "w_o": draw_normal(w.seed, _K_O, l, (C, Q)),
        "w_fc": draw_normal(w.seed, _K_FC, l, (F, C)),
        "w_proj": draw_normal(w.seed, _K_PROJ, l, (C, F)),
    }
    if w.extras:
        g = _rng(w.seed, _K_SCAL, l)
        out["resid_lambda"] = np.float32(g.uniform(0.5, 1.5))
        out["x0_lambda"] = np.float32(g.uniform(0.5, 1.5))
        if l % 2 == 1:
            out["ve"] = draw_normal(w.seed, _K_VE, l, (w.vocab, KV))
            out["ve_gate"] = draw_normal(w.seed, _K_VEGATE, l, (w.n_kv_head, w.ve_gate_channels))
    return out


def draw_globals(w: Workload) -> Dict[str, np.ndarray]:
    """float32 draws for wte [V, C] and lm_head [V, C]; plus smear/backout params."""
    out = {
        "wte": draw_normal(w.seed, _K_WTE, 0, (w.vocab, w.C)),
        "w_lm": draw_normal(w.seed, _K_WLM, 0, (w.vocab, w.C)),
    }
    if w.extras:
        g = _rng(w.seed, _K_SCAL, 100_000)
        out["smear_lambda"] = np.float32(g.uniform(0.5, 1.5))
        out["backout_lambda"] = np.float32(g.uniform(0.5, 1.5))
        out["smear_gate"] = draw_normal(w.seed, _K_SMEAR, 0, (w.smear_channels,))
    return out


def draw_all(w: Workload) -> Dict[str, object]:
    return {"ids": draw_ids(w), "globals": draw_globals(w),
            "layers": [draw_layer(w, l) for l in range(w.n_layer)]}


def draw_upstream(w: Workload, key: int, shape, std: float = 1.0) -> np.ndarray:
    """A seeded upstream gradient (used to test one block's backward alone)."""
    return draw_normal(w.seed, _K_DX, key, shape, std)


def to_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 draws to the storage dtype; returns float32 values that are
    exactly representable in `dtype` ("f32": unchanged, "bf16": round to nearest
    even on the bit pattern, which these finite draws never overflow)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f32":
        return a
    if dtype != "bf16":
        raise ValueError(dtype)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)
