"""One training step of the decoder stack through the C ABI.

    embed_fwd -> L x block_fwd -> lm_head_ce_fwd_bwd -> L x block_bwd -> embed_bwd

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

from . import ops

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


class DecoderStack:
    def __init__(self, *, n_layer: int, B: int, T: int, C: int, n_head: int, n_kv_head: int, head_dim: int,
                 mlp_hidden: int, vocab: int, windows: Sequence[int], dtype: str, eps: float = 1e-6,
                 rope_base: float = 10000.0, device: str = "cuda:0"):
        if len(windows) != n_layer:
            raise ValueError("one window per layer")
        self.L, self.B, self.T, self.C, self.V = n_layer, B, T, C, vocab
        self.N = B * T
        self.dt = _TORCH_DT[dtype]
        self.eps = eps
        self.device = torch.device(device)
        self.cfgs = [ops.make_cfg(B, T, C, n_head, n_kv_head, head_dim, mlp_hidden, w, self.dt, eps)
                     for w in windows]
        Q, KV = n_head * head_dim, n_kv_head * head_dim
        self.shapes = {"w_qkv": (Q + 2 * KV, C), "w_o": (C, Q), "w_fc": (mlp_hidden, C), "w_proj": (C, mlp_hidden)}
        dev, dt = self.device, self.dt
        self.rope = ops.rope_table(T, head_dim, rope_base, dev)
        sizes = [ops.block_sizes(c) for c in self.cfgs]
        self.saved = [torch.empty(s[0], dtype=torch.uint8, device=dev) for s in sizes]
        self.ws_f = torch.empty(max(s[1] for s in sizes), dtype=torch.uint8, device=dev)
        self.ws_b = torch.empty(max(s[2] for s in sizes), dtype=torch.uint8, device=dev)
        self.ws_h = torch.empty(ops.lm_head_ce_sizes(self.N, C, vocab, dt), dtype=torch.uint8, device=dev)
        self.xs = [torch.empty((self.N, C), dtype=dt, device=dev) for _ in range(n_layer + 1)]
        self.dx = torch.empty((self.N, C), dtype=dt, device=dev)
        self.loss = torch.zeros((1,), dtype=torch.float32, device=dev)
        self.wte = torch.empty((vocab, C), dtype=dt, device=dev)
        self.w_lm = torch.empty((vocab, C), dtype=dt, device=dev)
        self.layers = [[torch.empty(self.shapes[k], dtype=dt, device=dev) for k in self.shapes]
                       for _ in range(n_layer)]
        self.dwte = torch.empty((vocab, C), dtype=torch.float32, device=dev)
        self.dw_lm = torch.empty((vocab, C), dtype=torch.float32, device=dev)
        self.dlayers = [[torch.empty(self.shapes[k], dtype=torch.float32, device=dev) for k in self.shapes]
                        for _ in range(n_layer)]
        self.ids = torch.zeros((self.N,), dtype=torch.int32, device=dev)
        self.tgt = torch.zeros((self.N,), dtype=torch.int32, device=dev)

    # ------------------------------------------------------------ inputs
    def _put(self, dst: torch.Tensor, a: np.ndarray) -> None:
        dst.copy_(torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dst.dtype))

    def load(self, glob: Dict[str, np.ndarray], layers: List[Dict[str, np.ndarray]]) -> None:
        """Copy float32 host arrays (already representable in the compute dtype)."""
        self._put(self.wte, glob["wte"])
        self._put(self.w_lm, glob["w_lm"])
        for l, p in enumerate(layers):
            for t, k in zip(self.layers[l], self.shapes):
                self._put(t, p[k])

    def set_ids(self, ids: np.ndarray) -> None:
        """ids [B, T+1]: inputs ids[:, :T], next-token targets ids[:, 1:]."""
        ids = np.asarray(ids)
        self.ids.copy_(torch.from_numpy(np.ascontiguousarray(ids[:, :-1].reshape(-1), dtype=np.int32)))
        self.tgt.copy_(torch.from_numpy(np.ascontiguousarray(ids[:, 1:].reshape(-1), dtype=np.int32)))

    # -------------------------------------------------------------- step
    def forward(self) -> None:
        ops.embed_fwd(self.ids, self.wte, self.xs[0])
        for l in range(self.L):
            ops.block_fwd(self.cfgs[l], self.layers[l], self.rope, self.xs[l], self.xs[l + 1], self.saved[l],
                          self.ws_f)

    def head(self) -> None:
        ops.lm_head_ce_fwd_bwd(self.xs[self.L], self.w_lm, self.tgt, self.loss, self.dx, self.dw_lm, self.ws_h,
                               eps=self.eps)

    def backward(self) -> None:
        for l in reversed(range(self.L)):
            ops.block_bwd(self.cfgs[l], self.layers[l], self.rope, self.saved[l], self.dx, self.dx,
                          self.dlayers[l], self.ws_b)
        ops.embed_bwd(self.ids, self.dx, self.dwte)

    def step(self) -> torch.Tensor:
        self.forward()
        self.head()
        self.backward()
        return self.loss
