"""Parity at the full d24 training size, in the launch configuration bench.py
times (B=16, T=2048, C=1536): the kernels run on the whole batch and the
oracle checks sampled outputs it can compute on its own.

* Block: x_out and dx_in of whole sampled sequences (a sequence's outputs
  depend only on that sequence), and the weight gradients of a backward whose
  upstream gradient is non-zero only on the sampled sequences (so dW is the
  sum of those sequences' contributions, which the oracle computes).
* Head: every token except a few sampled ones has x = 0, so its normalised
  row is 0, its logits are 0 and its loss is exactly ln V; each sampled row's
  loss, the mean loss, the sampled rows of dx (the oracle's one-row gradient
  times 1/N) and dW_lm (only sampled rows contribute) are then known from the
  sampled rows alone.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from gpt_decoder_block_amd import ops
from gpu_util import DEV, TDT, assert_close, dev, empty, host, rounded
from seeded_inputs import draw_globals, draw_ids, draw_layer, draw_upstream, workload

pytestmark = pytest.mark.gpu


def _block_fullsize(w, l, rows):
    dt, B, T, C = w.dtype, w.B, w.T, w.C
    N = B * T
    print(f"full-size block {w.name} l={l} B={B} T={T} window={w.windows[l]} rows={rows}", flush=True)
    p = {k: rounded(v, dt) for k, v in draw_layer(w, l).items()}
    x = rounded(draw_upstream(w, 100 + l, (N, C), 1.0), dt)
    dy_all = rounded(draw_upstream(w, 200 + l, (N, C), 1.0), dt).reshape(B, T, C)
    dy = np.zeros_like(dy_all)
    dy[rows] = dy_all[rows]
    cfg = ops.make_cfg(B, T, C, w.n_head, w.n_kv_head, w.head_dim, w.mlp_hidden, w.windows[l], TDT[dt], w.eps)
    sv, wf, wb = ops.block_sizes(cfg)
    saved = torch.empty(sv, dtype=torch.uint8, device=DEV)
    wsf = torch.empty(wf, dtype=torch.uint8, device=DEV)
    wsb = torch.empty(wb, dtype=torch.uint8, device=DEV)
    W = [dev(p[k], dt) for k in ("w_qkv", "w_o", "w_fc", "w_proj")]
    dW = [empty(t.shape, torch.float32) for t in W]
    rope = ops.rope_table(T, w.head_dim, w.rope_base, DEV)
    out = empty((N, C), dt)
    ops.block_fwd(cfg, W, rope, dev(x, dt), out, saved, wsf)
    dx = dev(dy.reshape(N, C), dt)
    ops.block_bwd(cfg, W, rope, saved, dx, dx, dW, wsb)
    torch.cuda.synchronize()
    out_h = host(out).reshape(B, T, C)
    dx_h = host(dx).reshape(B, T, C)
    cos, sin = O.rope_tables(T, w.head_dim, w.rope_base)
    pp = {k: v.astype(np.float64) for k, v in p.items()}
    gsum = {k: 0.0 for k in ("w_qkv", "w_o", "w_fc", "w_proj")}
    errs = {}
    x3 = x.reshape(B, T, C)
    for b in rows:
        o_out, c = O.block_forward(x3[b:b + 1].astype(np.float64), pp, w, l, cos, sin)
        o_dx, g = O.block_backward(dy[b:b + 1].astype(np.float64), c, pp, w, l, cos, sin)
        errs[f"x_out[{b}]"] = assert_close(out_h[b], o_out[0], dt, f"x_out row {b}")
        errs[f"dx_in[{b}]"] = assert_close(dx_h[b], o_dx[0], dt, f"dx_in row {b}")
        for k in gsum:
            gsum[k] = gsum[k] + g[k]
        del c
    for k, t in zip(gsum, dW):
        errs[k] = assert_close(t, gsum[k], dt, "d" + k)
    print(f"full-size block errs={errs}", flush=True)


@pytest.mark.parametrize("l", [0, 1])
def test_block_d24_full_size(l):
    # l=0: full causal attention; l=1: window 1024 over T=2048
    w = workload("d24")
    _block_fullsize(w, l, [0, w.B - 1])


def test_lm_head_ce_d24_full_size():
    w = workload("d24")
    dt, N, C, V = w.dtype, w.B * w.T, w.C, w.vocab
    rows = np.array([0, 1, 4097, 20000, N - 1])
    print(f"full-size head N={N} C={C} V={V} rows={rows.tolist()}", flush=True)
    g = draw_globals(w)
    w_lm = rounded(g["w_lm"], dt)
    x = np.zeros((N, C), dtype=np.float32)
    x[rows] = rounded(draw_upstream(w, 300, (len(rows), C), 1.0), dt)
    y = draw_ids(w)[:, 1:].reshape(-1)
    ws = torch.empty(ops.lm_head_ce_sizes(N, C, V, TDT[dt]), dtype=torch.uint8, device=DEV)
    loss = empty((1,), torch.float32)
    row_loss = empty((N,), torch.float32)
    dx = empty((N, C), dt)
    dw = empty((V, C), torch.float32)
    ops.lm_head_ce_fwd_bwd(dev(x, dt), dev(w_lm, dt), torch.from_numpy(y.astype(np.int32)).to(DEV), loss, dx, dw,
                           ws, eps=w.eps, row_loss=row_loss)
    torch.cuda.synchronize()
    l_rows, dx_rows, dw_rows, hc = O.lm_head_ce(x[rows].astype(np.float64), w_lm.astype(np.float64), y[rows], w.eps)
    # each sampled row's own loss (the oracle's per-row losses), every other
    # row exactly ln V; then the mean over N, which those rows fix
    z = hc["z"]
    row_ref = hc["lse"] - z[np.arange(len(rows)), y[rows]]
    rl = host(row_loss)
    e_rows = assert_close(rl[rows], row_ref, dt, "row losses (sampled rows)")
    others = np.setdiff1d(np.arange(N), rows)
    assert np.max(np.abs(rl[others] - math.log(V))) <= 1e-5 * math.log(V)
    n = len(rows)
    loss_ref = (l_rows * n + (N - n) * math.log(V)) / N
    assert abs(loss.item() - loss_ref) <= 2e-2 * abs(loss_ref)
    e_dx = assert_close(host(dx)[rows], dx_rows * n / N, dt, "dx (sampled rows)")
    e_dw = assert_close(dw, dw_rows * n / N, dt, "dw_lm")
    print(f"full-size head row losses {e_rows:.3e}", flush=True)
    print(f"full-size head loss {loss.item():.6f} ref {loss_ref:.6f} dx {e_dx:.3e} dw {e_dw:.3e}", flush=True)
