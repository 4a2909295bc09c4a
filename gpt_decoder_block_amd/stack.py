"""One training step of the decoder stack through the C ABI.

    embed_fwd -> L x block_fwd -> lm_head_ce_fwd_bwd -> L x block_bwd -> embed_bwd

With `extras` (the largest model of "Comment Entraîner Votre Propre ChatGPT
Pour 50€ ?", section "1. Le modèle GPT"): smear after the embedding, residual
mixing with x0 in every block, value embeddings in the odd blocks, backout of
the output of block L/2 - 1 before the head.

torch allocates every buffer once (weights, fp32 weight gradients, per-layer
saved activations, the residual stream of every layer, workspaces) and
provides the stream; all arithmetic runs in libgdb's HIP kernels.  On a
288 GB MI355X the whole d24 step at B=16, T=2048 (about 45 GB) stays resident,
so nothing is chunked or recomputed.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

from . import _lib, ops

L_EXTRAS_WS = _lib.GDB_EXTRAS_WS_BYTES
_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


class DecoderStack:
    def __init__(self, *, n_layer: int, B: int, T: int, C: int, n_head: int, n_kv_head: int, head_dim: int,
                 mlp_hidden: int, vocab: int, windows: Sequence[int], dtype: str, eps: float = 1e-6,
                 rope_base: float = 10000.0, device: str = "cuda:0", extras: bool = False,
                 ve_gate_channels: int = 32, smear_channels: int = 24, mlp_fp8: bool = False,
                 deterministic: bool = False):
        if len(windows) != n_layer:
            raise ValueError("one window per layer")
        if extras and n_layer < 2:
            raise ValueError("the extras need at least 2 layers (backout reads block L/2 - 1)")
        self.L, self.B, self.T, self.C, self.V = n_layer, B, T, C, vocab
        self.N = B * T
        self.dt = _TORCH_DT[dtype]
        self.eps = eps
        self.extras = extras
        self.device = torch.device(device)
        self.deterministic = deterministic
        self.cfgs = [ops.make_cfg(B, T, C, n_head, n_kv_head, head_dim, mlp_hidden, w, self.dt, eps,
                                  mlp_fp8=mlp_fp8, deterministic=deterministic) for w in windows]
        Q, KV = n_head * head_dim, n_kv_head * head_dim
        self.shapes = {"w_qkv": (Q + 2 * KV, C), "w_o": (C, Q), "w_fc": (mlp_hidden, C), "w_proj": (C, mlp_hidden)}
        dev, dt = self.device, self.dt
        f32 = torch.float32
        self.rope = ops.rope_table(T, head_dim, rope_base, dev)
        sizes = [ops.block_sizes(c) for c in self.cfgs]
        self.saved = [torch.empty(s[0], dtype=torch.uint8, device=dev) for s in sizes]
        self.ws_f = torch.empty(max(s[1] for s in sizes), dtype=torch.uint8, device=dev)
        self.ws_b = torch.empty(max(s[2] for s in sizes), dtype=torch.uint8, device=dev)
        self.ws_h = torch.empty(ops.lm_head_ce_sizes(self.N, C, vocab, dt), dtype=torch.uint8, device=dev)
        self.xs = [torch.empty((self.N, C), dtype=dt, device=dev) for _ in range(n_layer + 1)]
        self.dx = torch.empty((self.N, C), dtype=dt, device=dev)
        self.loss = torch.zeros((1,), dtype=f32, device=dev)
        self.wte = torch.empty((vocab, C), dtype=dt, device=dev)
        self.w_lm = torch.empty((vocab, C), dtype=dt, device=dev)
        self.layers = [[torch.empty(self.shapes[k], dtype=dt, device=dev) for k in self.shapes]
                       for _ in range(n_layer)]
        self.dwte = torch.empty((vocab, C), dtype=f32, device=dev)
        self.dw_lm = torch.empty((vocab, C), dtype=f32, device=dev)
        self.dlayers = [[torch.empty(self.shapes[k], dtype=f32, device=dev) for k in self.shapes]
                        for _ in range(n_layer)]
        self.ids = torch.zeros((self.N,), dtype=torch.int32, device=dev)
        # deterministic: the embedding gradient adds its tokens in a fixed order (sort scratch)
        self.ws_e = (torch.empty(max(ops.embed_bwd_ws_bytes(self.N, True), 16), dtype=torch.uint8, device=dev)
                     if deterministic else None)
        self.tgt = torch.zeros((self.N,), dtype=torch.int32, device=dev)
        if extras:
            self.i_bo = n_layer // 2 - 1
            self.ve_layers = [l % 2 == 1 for l in range(n_layer)]
            self.e = torch.empty((self.N, C), dtype=dt, device=dev)          # embedding before smear
            self.x_final = torch.empty((self.N, C), dtype=dt, device=dev)    # after backout
            self.dhead = torch.empty((self.N, C), dtype=dt, device=dev)      # head gradient, kept for backout
            self.de = torch.empty((self.N, C), dtype=dt, device=dev)
            self.dx0 = torch.empty((self.N, C), dtype=f32, device=dev)
            self.s_smear = torch.empty((self.N,), dtype=f32, device=dev)
            self.ws_x = torch.empty(L_EXTRAS_WS, dtype=torch.uint8, device=dev)
            self.smear_lambda = torch.zeros((1,), dtype=f32, device=dev)
            self.backout_lambda = torch.zeros((1,), dtype=f32, device=dev)
            self.smear_gate = torch.empty((smear_channels,), dtype=dt, device=dev)
            self.d_smear_lambda = torch.zeros((1,), dtype=f32, device=dev)
            self.d_backout_lambda = torch.zeros((1,), dtype=f32, device=dev)
            self.d_smear_gate = torch.zeros((smear_channels,), dtype=f32, device=dev)
            self.lambdas = [torch.zeros((2,), dtype=f32, device=dev) for _ in range(n_layer)]
            self.dlambdas = [torch.zeros((2,), dtype=f32, device=dev) for _ in range(n_layer)]
            self.ve = [torch.empty((vocab, KV), dtype=dt, device=dev) if v else None for v in self.ve_layers]
            self.ve_gate = [torch.empty((n_kv_head, ve_gate_channels), dtype=dt, device=dev) if v else None
                            for v in self.ve_layers]
            self.dve = [torch.empty((vocab, KV), dtype=f32, device=dev) if v else None for v in self.ve_layers]
            self.dve_gate = [torch.empty((n_kv_head, ve_gate_channels), dtype=f32, device=dev) if v else None
                             for v in self.ve_layers]
            self.ex = [ops.block_extras(self.lambdas[l], self.xs[0], self.xs[l], self.ids, self.ve[l],
                                        self.ve_gate[l]) for l in range(n_layer)]
            self.dex = [ops.block_extras_grads(self.dlambdas[l], self.dx0, self.dve[l], self.dve_gate[l],
                                               accumulate_dx0=l != n_layer - 1) for l in range(n_layer)]

    # ------------------------------------------------------------ inputs
    def _put(self, dst: torch.Tensor, a: np.ndarray) -> None:
        dst.copy_(torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32).reshape(dst.shape)).to(dst.dtype))

    def load(self, glob: Dict[str, np.ndarray], layers: List[Dict[str, np.ndarray]]) -> None:
        """Copy float32 host arrays (already representable in the compute dtype)."""
        self._put(self.wte, glob["wte"])
        self._put(self.w_lm, glob["w_lm"])
        for l, p in enumerate(layers):
            for t, k in zip(self.layers[l], self.shapes):
                self._put(t, p[k])
        if self.extras:
            self._put(self.smear_lambda, np.array([glob["smear_lambda"]]))
            self._put(self.backout_lambda, np.array([glob["backout_lambda"]]))
            self._put(self.smear_gate, glob["smear_gate"])
            for l, p in enumerate(layers):
                self._put(self.lambdas[l], np.array([p["resid_lambda"], p["x0_lambda"]]))
                if self.ve_layers[l]:
                    self._put(self.ve[l], p["ve"])
                    self._put(self.ve_gate[l], p["ve_gate"])

    def set_ids(self, ids: np.ndarray) -> None:
        """ids [B, T+1]: inputs ids[:, :T], next-token targets ids[:, 1:]."""
        ids = np.asarray(ids)
        self.ids.copy_(torch.from_numpy(np.ascontiguousarray(ids[:, :-1].reshape(-1), dtype=np.int32)))
        self.tgt.copy_(torch.from_numpy(np.ascontiguousarray(ids[:, 1:].reshape(-1), dtype=np.int32)))

    # -------------------------------------------------------------- step
    def forward(self) -> None:
        if self.extras:
            ops.embed_fwd(self.ids, self.wte, self.e)
            ops.smear_fwd(self.B, self.T, self.e, self.smear_gate, self.smear_lambda, self.xs[0], self.s_smear)
        else:
            ops.embed_fwd(self.ids, self.wte, self.xs[0])
        for l in range(self.L):
            ops.block_fwd(self.cfgs[l], self.layers[l], self.rope, self.xs[l], self.xs[l + 1], self.saved[l],
                          self.ws_f, self.ex[l] if self.extras else None)
        if self.extras:
            ops.backout_fwd(self.xs[self.L], self.xs[self.i_bo + 1], self.backout_lambda, self.x_final)

    def head(self) -> None:
        if self.extras:
            ops.lm_head_ce_fwd_bwd(self.x_final, self.w_lm, self.tgt, self.loss, self.dhead, self.dw_lm, self.ws_h,
                                   eps=self.eps)
        else:
            ops.lm_head_ce_fwd_bwd(self.xs[self.L], self.w_lm, self.tgt, self.loss, self.dx, self.dw_lm, self.ws_h,
                                   eps=self.eps)

    def backward(self) -> None:
        if not self.extras:
            for l in reversed(range(self.L)):
                ops.block_bwd(self.cfgs[l], self.layers[l], self.rope, self.saved[l], self.dx, self.dx,
                              self.dlayers[l], self.ws_b)
            ops.embed_bwd(self.ids, self.dx, self.dwte, ws=self.ws_e)
            return
        for l in reversed(range(self.L)):
            if l == self.i_bo:
                # the gradient w.r.t. block i_bo's output also receives the backout share
                ops.backout_bwd(self.dhead, self.xs[self.i_bo + 1], self.backout_lambda, self.dx,
                                self.d_backout_lambda, self.ws_x)
            dy = self.dhead if l == self.L - 1 else self.dx
            ops.block_bwd(self.cfgs[l], self.layers[l], self.rope, self.saved[l], dy, self.dx, self.dlayers[l],
                          self.ws_b, self.ex[l], self.dex[l])
        ops.smear_bwd(self.B, self.T, self.e, self.smear_gate, self.smear_lambda, self.s_smear, self.dx, self.dx0,
                      self.de, self.d_smear_lambda, self.d_smear_gate, self.ws_x)
        ops.embed_bwd(self.ids, self.de, self.dwte, ws=self.ws_e)

    def step(self) -> torch.Tensor:
        self.forward()
        self.head()
        self.backward()
        return self.loss
