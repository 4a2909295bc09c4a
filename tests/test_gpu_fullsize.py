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


def test_block_d26_full_size_fp8_mixing():
    """The d26 block (layer 0: residual mixing, fp8 MLP products; no value
    embedding on even layers) at the full batch B=16, T=2048.  Only the
    sampled sequences carry non-zero inputs (x, x0 and the upstream gradient),
    so every other token's activations and gradients are exactly zero: the
    per-tensor fp8 scales of the whole batch equal those of the sampled
    sequences, which the oracle computes alone.  Bars: the fp8 bound 2q of the
    block tests (q measured on the oracle with the quantiser off)."""
    from gpu_util import fp8_bars
    w = workload("d26")
    l, rows = 0, [0, w.B - 1]
    dt, B, T, C = w.dtype, w.B, w.T, w.C
    N = B * T
    print(f"full-size d26 block l={l} B={B} T={T} fp8={w.mlp_fp8} rows={rows}", flush=True)
    p = {k: (rounded(v, dt) if np.ndim(v) else np.float32(v)) for k, v in draw_layer(w, l).items()}
    assert "ve" not in p
    def sampled(key, std):
        a = np.zeros((B, T, C), dtype=np.float32)
        a[rows] = rounded(draw_upstream(w, key, (len(rows), T, C), std), dt)
        return a
    x, x0, dy = sampled(100, 1.0), sampled(150, 1.0), sampled(200, 1.0)
    ids = draw_ids(w)[:, :T]
    cfg = ops.make_cfg(B, T, C, w.n_head, w.n_kv_head, w.head_dim, w.mlp_hidden, w.windows[l], TDT[dt], w.eps,
                       mlp_fp8=w.mlp_fp8)
    sv, wf, wb = ops.block_sizes(cfg)
    saved = torch.empty(sv, dtype=torch.uint8, device=DEV)
    wsf = torch.empty(wf, dtype=torch.uint8, device=DEV)
    wsb = torch.empty(wb, dtype=torch.uint8, device=DEV)
    W = [dev(p[k], dt) for k in ("w_qkv", "w_o", "w_fc", "w_proj")]
    dW = [empty(t.shape, torch.float32) for t in W]
    rope = ops.rope_table(T, w.head_dim, w.rope_base, DEV)
    xg, x0g, out = dev(x.reshape(N, C), dt), dev(x0.reshape(N, C), dt), empty((N, C), dt)
    lam = torch.tensor([p["resid_lambda"], p["x0_lambda"]], dtype=torch.float32, device=DEV)
    idsg = torch.from_numpy(ids.reshape(-1).astype(np.int32)).to(DEV)
    dlam = empty((2,), torch.float32)
    dx0 = empty((N, C), torch.float32, fill=0.0)
    ex = ops.block_extras(lam, x0g, xg, idsg, None, None)
    dex = ops.block_extras_grads(dlam, dx0, None, None, accumulate_dx0=True)
    ops.block_fwd(cfg, W, rope, xg, out, saved, wsf, ex)
    dx = dev(dy.reshape(N, C), dt)
    ops.block_bwd(cfg, W, rope, saved, dx, dx, dW, wsb, ex, dex)
    torch.cuda.synchronize()
    out_h, dx_h, dx0_h = host(out).reshape(B, T, C), host(dx).reshape(B, T, C), host(dx0).reshape(B, T, C)
    others = np.setdiff1d(np.arange(B), rows)
    assert not np.any(out_h[others]) and not np.any(dx_h[others]) and not np.any(dx0_h[others])
    cos, sin = O.rope_tables(T, w.head_dim, w.rope_base)
    pp = {k: np.asarray(v, dtype=np.float64) for k, v in p.items()}
    s = np.array(rows)
    x64, x064, dy64 = x[s].astype(np.float64), x0[s].astype(np.float64), dy[s].astype(np.float64)
    o_out, c = O.block_forward(x64, pp, w, l, cos, sin, x0=x064, ids=ids[s])
    o_dx, g = O.block_backward(dy64, c, pp, w, l, cos, sin, ids=ids[s])
    we = w.with_(mlp_fp8=False)
    oe, ce = O.block_forward(x64, pp, we, l, cos, sin, x0=x064, ids=ids[s])
    dxe, ge = O.block_backward(dy64, ce, pp, we, l, cos, sin, ids=ids[s])
    names = ("w_qkv", "w_o", "w_fc", "w_proj")
    bars = fp8_bars({"x_out": (o_out, oe), "dx_in": (o_dx, dxe), "dx0": (g["x0"], ge["x0"]),
                     "dlambdas": ([g["resid_lambda"], g["x0_lambda"]], [ge["resid_lambda"], ge["x0_lambda"]]),
                     **{k: (g[k], ge[k]) for k in names}}, dt)
    print("fp8 bars", {k: round(v, 4) for k, v in bars.items()}, flush=True)
    errs = {"x_out": assert_close(out_h[s], o_out, dt, "x_out (sampled sequences)", bars["x_out"]),
            "dx_in": assert_close(dx_h[s], o_dx, dt, "dx_in (sampled sequences)", bars["dx_in"]),
            "dx0": assert_close(dx0_h[s], g["x0"], dt, "dx0 (sampled sequences)", bars["dx0"]),
            "dlambdas": assert_close(dlam, [g["resid_lambda"], g["x0_lambda"]], dt, "dlambdas", bars["dlambdas"])}
    for k, t in zip(names, dW):
        errs[k] = assert_close(t, g[k], dt, "d" + k, bars[k])
    print(f"full-size d26 block errs={errs}", flush=True)
