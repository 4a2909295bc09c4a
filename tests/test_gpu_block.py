"""Parity of block_fwd / block_bwd / lm_head_ce_fwd_bwd and of the whole
training step (through the C ABI) with the CPU oracle on the same seeded
inputs.  Bars: max relative error <= 1e-4 in fp32 mode, <= 2e-2 in bf16 mode,
per output and per gradient tensor."""
import numpy as np
import pytest
import torch

import oracle as O
from gpt_decoder_block_amd import ops
from gpt_decoder_block_amd.stack import DecoderStack
from gpu_util import DEV, TDT, assert_close, dev, empty, host, rounded
from seeded_inputs import draw_all, draw_layer, draw_upstream, workload

pytestmark = pytest.mark.gpu


def _block_case(w, l, B, T, x_std=1.0):
    dt = w.dtype
    N, C = B * T, w.C
    p = {k: rounded(v, dt) for k, v in draw_layer(w, l).items()}
    x = rounded(draw_upstream(w, 100 + l, (N, C), x_std), dt)
    dy = rounded(draw_upstream(w, 200 + l, (N, C), 1.0), dt)
    cfg = ops.make_cfg(B, T, C, w.n_head, w.n_kv_head, w.head_dim, w.mlp_hidden, w.windows[l], TDT[dt], w.eps)
    sv, wf, wb = ops.block_sizes(cfg)
    saved = torch.empty(sv, dtype=torch.uint8, device=DEV)
    wsf = torch.empty(wf, dtype=torch.uint8, device=DEV)
    wsb = torch.empty(wb, dtype=torch.uint8, device=DEV)
    W = [dev(p[k], dt) for k in ("w_qkv", "w_o", "w_fc", "w_proj")]
    dW = [empty(t.shape, torch.float32) for t in W]
    rope = ops.rope_table(T, w.head_dim, w.rope_base, DEV)
    xg, out = dev(x, dt), empty((N, C), dt)
    ops.block_fwd(cfg, W, rope, xg, out, saved, wsf)
    dx = dev(dy, dt)
    ops.block_bwd(cfg, W, rope, saved, dx, dx, dW, wsb)      # dx_in aliases dx_out
    torch.cuda.synchronize()
    # oracle
    cos, sin = O.rope_tables(T, w.head_dim, w.rope_base)
    pp = {k: v.astype(np.float64) for k, v in p.items()}
    o_out, c = O.block_forward(x.astype(np.float64).reshape(B, T, C), pp, w, l, cos, sin)
    o_dx, g = O.block_backward(dy.astype(np.float64).reshape(B, T, C), c, pp, w, l, cos, sin)
    errs = {"x_out": assert_close(out, o_out.reshape(N, C), dt, "x_out"),
            "dx_in": assert_close(dx, o_dx.reshape(N, C), dt, "dx_in")}
    for name, t in zip(("w_qkv", "w_o", "w_fc", "w_proj"), dW):
        errs[name] = assert_close(t, g[name], dt, "d" + name)
    print(f"block {w.name} l={l} B={B} T={T} window={w.windows[l]} errs={errs}", flush=True)
    return errs


@pytest.mark.parametrize("l", [0, 1])
def test_block_d24_shape(l):
    # d24 widths (C=1536, 12 heads of 128, MLP 6144); odd layer windowed (1024 -> 64 here)
    w = workload("d24").with_(n_layer=2, windows=(-1, 64))
    _block_case(w, l, 2, 160)


def test_block_d12_gqa_window():
    w = workload("d12_gqa_swa").with_(n_layer=2, windows=(-1, 100))
    _block_case(w, 1, 1, 300)
    _block_case(w, 0, 2, 64)


def test_block_d26_widths_ragged_tiles():
    # C = 1664 = 13 heads of 128: output tiles of 256 are ragged
    w = workload("d26").with_(n_layer=1, windows=(-1,), extras=False, mlp_fp8=False)
    _block_case(w, 0, 1, 130)


@pytest.mark.parametrize("B,T", [(1, 64), (2, 37)])
def test_block_tiny_fp32(B, T):
    w = workload("tiny")
    _block_case(w, 0, B, T)


@pytest.mark.parametrize("name,N", [("d24", 256), ("tiny", 64)])
def test_lm_head_ce(name, N):
    w = workload(name)
    dt = w.dtype
    glob = draw_globals_rounded(w)
    x = rounded(draw_upstream(w, 300, (N, w.C), 1.0), dt)
    y = np.random.default_rng(5).integers(0, w.vocab, size=N)
    ws = torch.empty(ops.lm_head_ce_sizes(N, w.C, w.vocab, TDT[dt]), dtype=torch.uint8, device=DEV)
    loss = empty((1,), torch.float32)
    dx = empty((N, w.C), dt)
    dw = empty((w.vocab, w.C), torch.float32)
    ops.lm_head_ce_fwd_bwd(dev(x, dt), dev(glob["w_lm"], dt), torch.from_numpy(y.astype(np.int32)).to(DEV),
                           loss, dx, dw, ws, eps=w.eps)
    torch.cuda.synchronize()
    l_ref, dx_ref, dw_ref, _ = O.lm_head_ce(x.astype(np.float64), glob["w_lm"].astype(np.float64), y, w.eps)
    tol = 1e-4 if dt == "f32" else 2e-2
    assert abs(loss.item() - l_ref) <= tol * abs(l_ref)
    assert_close(dx, dx_ref, dt, "dx")
    assert_close(dw, dw_ref, dt, "dw_lm")


def draw_globals_rounded(w):
    from seeded_inputs import draw_globals
    return {k: rounded(v, w.dtype) for k, v in draw_globals(w).items()}


def _stack_case(w):
    d = draw_all(w)
    glob = {k: rounded(v, w.dtype) for k, v in d["globals"].items()}
    layers = [{k: rounded(v, w.dtype) for k, v in p.items()} for p in d["layers"]]
    st = DecoderStack(n_layer=w.n_layer, B=w.B, T=w.T, C=w.C, n_head=w.n_head, n_kv_head=w.n_kv_head,
                      head_dim=w.head_dim, mlp_hidden=w.mlp_hidden, vocab=w.vocab, windows=w.windows,
                      dtype=w.dtype, eps=w.eps, rope_base=w.rope_base, device=DEV)
    st.load(glob, layers)
    st.set_ids(d["ids"])
    loss = st.step()
    torch.cuda.synchronize()
    l_ref, g, _ = O.stack_forward_backward(w, d["ids"], glob, layers)
    dt = w.dtype
    tol = 1e-4 if dt == "f32" else 2e-2
    errs = {"loss": abs(loss.item() - l_ref) / abs(l_ref)}
    assert errs["loss"] <= tol
    errs["wte"] = assert_close(st.dwte, g["wte"], dt, "dwte")
    errs["w_lm"] = assert_close(st.dw_lm, g["w_lm"], dt, "dw_lm")
    for l in range(w.n_layer):
        for t, k in zip(st.dlayers[l], ("w_qkv", "w_o", "w_fc", "w_proj")):
            errs[f"{l}.{k}"] = assert_close(t, g["layers"][l][k], dt, f"layer {l} d{k}")
    print(f"stack {w.name} L={w.n_layer} B={w.B} T={w.T} errs={errs}", flush=True)


def test_stack_tiny_exact_workload():
    # the tiny single-block fp32 workload exactly as specified
    _stack_case(workload("tiny"))


def test_stack_d12_gqa_window_two_layers():
    _stack_case(workload("d12_gqa_swa").with_(n_layer=2, B=1, T=256, windows=(-1, 100)))


def test_stack_d24_two_layers():
    _stack_case(workload("d24").with_(n_layer=2, B=1, T=256, windows=(-1, 128)))
