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
from gpu_util import (DEV, TDT, TOL, assert_close, dev, empty, fp8_alternative, fp8_alternatives, fp8_bars, sum_close,
                      host, rounded)
from seeded_inputs import draw_all, draw_ids, draw_layer, draw_upstream, sssl_windows, workload

pytestmark = pytest.mark.gpu


def _block_case(w, l, B, T, x_std=1.0):
    dt = w.dtype
    N, C = B * T, w.C
    p = {k: rounded(v, dt) for k, v in draw_layer(w, l).items()}
    x = rounded(draw_upstream(w, 100 + l, (N, C), x_std), dt)
    dy = rounded(draw_upstream(w, 200 + l, (N, C), 1.0), dt)
    cfg = ops.make_cfg(B, T, C, w.n_head, w.n_kv_head, w.head_dim, w.mlp_hidden, w.windows[l], TDT[dt], w.eps,
                       mlp_fp8=w.mlp_fp8)
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
    bars = {}
    if w.mlp_fp8:
        alts = []
        for seed in fp8_alternatives(dt):
            with fp8_alternative(dt, seed) as alt_dt:
                w32 = w.with_(dtype=alt_dt)
                o2, c2 = O.block_forward(x.astype(np.float64).reshape(B, T, C), pp, w32, l, cos, sin)
                dx2, g2 = O.block_backward(dy.astype(np.float64).reshape(B, T, C), c2, pp, w32, l, cos, sin)
            alts.append((o2, dx2, g2))
        bars = fp8_bars({"x_out": (o_out, [a[0] for a in alts]), "dx_in": (o_dx, [a[1] for a in alts]),
                         **{k: (g[k], [a[2][k] for a in alts]) for k in ("w_qkv", "w_o", "w_fc", "w_proj")}}, dt)
        print("fp8 bars", bars, flush=True)
    errs = {"x_out": assert_close(out, o_out.reshape(N, C), dt, "x_out", bars.get("x_out")),
            "dx_in": assert_close(dx, o_dx.reshape(N, C), dt, "dx_in", bars.get("dx_in"))}
    for name, t in zip(("w_qkv", "w_o", "w_fc", "w_proj"), dW):
        errs[name] = assert_close(t, g[name], dt, "d" + name, bars.get(name))
    print(f"block {w.name} l={l} B={B} T={T} window={w.windows[l]} fp8={w.mlp_fp8} errs={errs}", flush=True)
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


def test_block_mlp_width_not_tile_multiple():
    # MLP width 1000 (a multiple of 8, not of 64): the backward's transposed
    # weight copies end in partial 64x64 tiles on both sides
    w = workload("d12_gqa_swa").with_(n_layer=1, windows=(-1,), mlp_hidden=1000)
    _block_case(w, 0, 1, 96)


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
                      dtype=w.dtype, eps=w.eps, rope_base=w.rope_base, device=DEV, extras=w.extras,
                      ve_gate_channels=w.ve_gate_channels, smear_channels=w.smear_channels, mlp_fp8=w.mlp_fp8)
    st.load(glob, layers)
    st.set_ids(d["ids"])
    loss = st.step()
    torch.cuda.synchronize()
    l_ref, g, o_out = O.stack_forward_backward(w, d["ids"], glob, layers)
    dt = w.dtype
    tol = 1e-4 if dt == "f32" else 2e-2
    bars = {}
    if w.mlp_fp8:
        alts = []
        for seed in fp8_alternatives(dt):
            with fp8_alternative(dt, seed) as alt_dt:
                alts.append(O.stack_forward_backward(w.with_(dtype=alt_dt), d["ids"], glob, layers)[:2])
        pairs = {"loss": (l_ref, [a[0] for a in alts]), "wte": (g["wte"], [a[1]["wte"] for a in alts]),
                 "w_lm": (g["w_lm"], [a[1]["w_lm"] for a in alts])}
        for l in range(w.n_layer):
            for k in g["layers"][l]:
                if k != "sum_abs":
                    pairs[f"{l}.{k}"] = (g["layers"][l][k], [a[1]["layers"][l][k] for a in alts])
        if w.extras:
            for k in ("smear_gate", "smear_lambda", "backout_lambda"):
                pairs[k] = (g[k], [a[1][k] for a in alts])
        bars = fp8_bars(pairs, dt)
        print("fp8 bars", {k: round(v, 4) for k, v in bars.items()}, flush=True)
    errs = {"loss": abs(loss.item() - l_ref) / abs(l_ref)}
    assert errs["loss"] <= bars.get("loss", tol)
    errs["wte"] = assert_close(st.dwte, g["wte"], dt, "dwte", bars.get("wte"))
    errs["w_lm"] = assert_close(st.dw_lm, g["w_lm"], dt, "dw_lm", bars.get("w_lm"))
    for l in range(w.n_layer):
        for t, k in zip(st.dlayers[l], ("w_qkv", "w_o", "w_fc", "w_proj")):
            errs[f"{l}.{k}"] = assert_close(t, g["layers"][l][k], dt, f"layer {l} d{k}", bars.get(f"{l}.{k}"))
        if w.extras:
            gl = g["layers"][l]
            if st.ve_layers[l]:
                errs[f"{l}.ve"] = assert_close(st.dve[l], gl["ve"], dt, f"layer {l} dve", bars.get(f"{l}.ve"))
                errs[f"{l}.ve_gate"] = sum_close(st.dve_gate[l], gl["ve_gate"], gl["sum_abs"]["ve_gate"], dt,
                                                 f"layer {l} dve_gate", bars.get(f"{l}.ve_gate"))
    if w.extras:
        # The residual, smear and backout scalars' gradients are sums over all
        # B*T*C activations with heavy cancellation (the sum of the terms'
        # magnitudes is 10^2..10^3 times the sum at these shapes), so a
        # per-element error e of the bf16 activations moves them by up to
        # e * sum|terms|, not e * |sum|.  The bar is the tensor bar applied to
        # that forward error bound: |gpu - oracle| <= TOL * sum|terms|.  In fp32
        # mode the plain relative bar holds as well.
        sa = o_out["sum_abs"]
        dl = np.stack([host(t) for t in st.dlambdas])

        def scalar_close(gpu, ref, bound, what, key):
            # with fp8 products, the fp8 bar (relative) is a third way to pass
            err = abs(float(gpu) - float(ref))
            rel = err / max(abs(float(ref)), 1e-300)
            ok = rel <= TOL[dt] or (dt == "bf16" and err <= TOL[dt] * bound) or rel <= bars.get(key, 0.0)
            assert ok, f"{what}: |d| {err:.3e} (rel {rel:.3e}, sum|terms| {bound:.3e}, fp8 bar {bars.get(key)})"
            return err / bound

        for l in range(w.n_layer):
            gl = g["layers"][l]
            errs[f"{l}.resid_lambda"] = scalar_close(dl[l, 0], gl["resid_lambda"], gl["sum_abs"]["resid_lambda"],
                                                     f"layer {l} d resid_lambda", f"{l}.resid_lambda")
            errs[f"{l}.x0_lambda"] = scalar_close(dl[l, 1], gl["x0_lambda"], gl["sum_abs"]["x0_lambda"],
                                                  f"layer {l} d x0_lambda", f"{l}.x0_lambda")
        errs["smear_lambda"] = scalar_close(host(st.d_smear_lambda)[0], g["smear_lambda"], sa["smear_lambda"],
                                            "d smear_lambda", "smear_lambda")
        errs["backout_lambda"] = scalar_close(host(st.d_backout_lambda)[0], g["backout_lambda"],
                                              sa["backout_lambda"], "d backout_lambda", "backout_lambda")
        errs["smear_gate"] = assert_close(st.d_smear_gate, g["smear_gate"], dt, "d smear_gate",
                                          bars.get("smear_gate"))
    print(f"stack {w.name} L={w.n_layer} B={w.B} T={w.T} extras={w.extras} fp8={w.mlp_fp8} errs={errs}",
          flush=True)


def test_stack_tiny_exact_workload():
    # the tiny single-block fp32 workload exactly as specified
    _stack_case(workload("tiny"))


def test_stack_d12_gqa_window_two_layers():
    _stack_case(workload("d12_gqa_swa").with_(n_layer=2, B=1, T=256, windows=(-1, 100)))


def test_stack_d24_two_layers():
    _stack_case(workload("d24").with_(n_layer=2, B=1, T=256, windows=(-1, 128)))


# ------------------------------------------------------------ extras (d26)
def _block_extras_case(w, l, B, T):
    """One block with residual mixing (and, on odd l, the value embedding);
    dx0 is pre-filled to check that the x0 share is added to it."""
    w = w.with_(B=B, T=T)
    dt = w.dtype
    N, C, KV = B * T, w.C, w.n_kv_head * w.head_dim
    p = {k: (rounded(v, dt) if np.ndim(v) else np.float32(v)) for k, v in draw_layer(w, l).items()}
    x = rounded(draw_upstream(w, 100 + l, (N, C), 1.0), dt)
    x0 = rounded(draw_upstream(w, 150 + l, (N, C), 1.0), dt)
    dy = rounded(draw_upstream(w, 200 + l, (N, C), 1.0), dt)
    dx0_prev = draw_upstream(w, 250 + l, (N, C), 0.1).astype(np.float32)
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
    xg, x0g, out = dev(x, dt), dev(x0, dt), empty((N, C), dt)
    lam = torch.tensor([p["resid_lambda"], p["x0_lambda"]], dtype=torch.float32, device=DEV)
    idsg = torch.from_numpy(ids.reshape(-1).astype(np.int32)).to(DEV)
    has_ve = "ve" in p
    ve = dev(p["ve"], dt) if has_ve else None
    vg = dev(p["ve_gate"], dt) if has_ve else None
    dlam = empty((2,), torch.float32)
    dx0 = torch.from_numpy(dx0_prev).to(DEV)
    dve = empty((w.vocab, KV), torch.float32, fill=7.0) if has_ve else None   # overwritten (no accumulate)
    dvg = empty((w.n_kv_head, w.ve_gate_channels), torch.float32) if has_ve else None
    ex = ops.block_extras(lam, x0g, xg, idsg, ve, vg)
    dex = ops.block_extras_grads(dlam, dx0, dve, dvg, accumulate_dx0=True)
    ops.block_fwd(cfg, W, rope, xg, out, saved, wsf, ex)
    dx = dev(dy, dt)
    ops.block_bwd(cfg, W, rope, saved, dx, dx, dW, wsb, ex, dex)
    torch.cuda.synchronize()
    cos, sin = O.rope_tables(T, w.head_dim, w.rope_base)
    pp = {k: np.asarray(v, dtype=np.float64) for k, v in p.items()}
    x64, x064 = x.astype(np.float64).reshape(B, T, C), x0.astype(np.float64).reshape(B, T, C)
    o_out, c = O.block_forward(x64, pp, w, l, cos, sin, x0=x064, ids=ids)
    o_dx, g = O.block_backward(dy.astype(np.float64).reshape(B, T, C), c, pp, w, l, cos, sin, ids=ids)
    names = ["w_qkv", "w_o", "w_fc", "w_proj"] + (["ve", "ve_gate"] if has_ve else [])
    bars = {}
    if w.mlp_fp8:
        alts = []
        for seed in fp8_alternatives(dt):
            with fp8_alternative(dt, seed) as alt_dt:
                w32 = w.with_(dtype=alt_dt)
                o2, c2 = O.block_forward(x64, pp, w32, l, cos, sin, x0=x064, ids=ids)
                dx2, g2 = O.block_backward(dy.astype(np.float64).reshape(B, T, C), c2, pp, w32, l, cos, sin,
                                           ids=ids)
            alts.append((o2, dx2, g2))
        bars = fp8_bars({"x_out": (o_out, [a[0] for a in alts]), "dx_in": (o_dx, [a[1] for a in alts]),
                         "dx0": (g["x0"], [a[2]["x0"] for a in alts]),
                         "dlambdas": ([g["resid_lambda"], g["x0_lambda"]],
                                      [[a[2]["resid_lambda"], a[2]["x0_lambda"]] for a in alts]),
                         **{k: (g[k], [a[2][k] for a in alts]) for k in names}}, dt)
        print("fp8 bars", bars, flush=True)
    errs = {"x_out": assert_close(out, o_out.reshape(N, C), dt, "x_out", bars.get("x_out")),
            "dx_in": assert_close(dx, o_dx.reshape(N, C), dt, "dx_in", bars.get("dx_in")),
            "dx0": assert_close(dx0, dx0_prev + g["x0"].reshape(N, C), dt, "dx0", bars.get("dx0")),
            "dlambdas": assert_close(dlam, [g["resid_lambda"], g["x0_lambda"]], dt, "dlambdas",
                                     bars.get("dlambdas"))}
    for name, t in zip(("w_qkv", "w_o", "w_fc", "w_proj"), dW):
        errs[name] = assert_close(t, g[name], dt, "d" + name, bars.get(name))
    if has_ve:
        errs["ve"] = assert_close(dve, g["ve"], dt, "dve", bars.get("ve"))
        errs["ve_gate"] = sum_close(dvg, g["ve_gate"], g["sum_abs"]["ve_gate"], dt, "dve_gate", bars.get("ve_gate"))
    print(f"block+extras {w.name} l={l} B={B} T={T} ve={has_ve} fp8={w.mlp_fp8} errs={errs}", flush=True)


@pytest.mark.parametrize("l", [0, 1])
def test_block_extras_d26_widths(l):
    # d26 widths (C=1664, 13 heads), vocabulary cut to 512 so the oracle's
    # value-embedding table stays small; l=1 carries a value embedding
    w = workload("d26").with_(n_layer=2, windows=(-1, -1), vocab=512, mlp_fp8=False)
    _block_extras_case(w, l, 1, 130)


@pytest.mark.parametrize("l", [0, 1])
def test_block_extras_tiny_fp32(l):
    w = workload("tiny").with_(n_layer=2, windows=(-1, -1), extras=True)
    _block_extras_case(w, l, 2, 37)


def test_stack_extras_tiny_fp32():
    _stack_case(workload("tiny").with_(n_layer=4, windows=(-1,) * 4, extras=True))


def test_stack_d24_record_pattern():
    # the d24 record model at d24 widths: SSSL windows (short window 40 at
    # T=130, so the window edge falls inside tiles), value embeddings on odd
    # layers, residual mixing, smear and backout, bf16
    w = workload("d24_record")
    _stack_case(w.with_(n_layer=4, B=1, T=130, vocab=512, windows=sssl_windows(4, 40)))


def test_stack_extras_d26_four_layers():
    # smear, residual mixing, value embeddings on layers 1 and 3, backout of block 1
    _stack_case(workload("d26").with_(n_layer=4, B=1, T=128, vocab=512, windows=(-1,) * 4, mlp_fp8=False))


# ------------------------------------------------------------- fp8 MLP (d26)
@pytest.mark.parametrize("B,T", [(1, 130), (2, 64)])
def test_block_fp8_mlp_d26_widths(B, T):
    # all four MLP products of the forward and the two of each backward GEMM on
    # e4m3 codes; T=130 leaves a ragged token count (padded to 144 for the
    # weight gradients)
    w = workload("d26").with_(n_layer=1, windows=(-1,), extras=False)
    _block_case(w, 0, B, T)


@pytest.mark.parametrize("l", [0, 1])
def test_block_fp8_mlp_with_extras(l):
    w = workload("d26").with_(n_layer=2, windows=(-1, -1), vocab=512)
    _block_extras_case(w, l, 1, 130)


def test_block_fp8_mlp_fp32_model():
    # fp8 products in an fp32 model: the quantiser sees float32 activations
    # that match the oracle's to ~1e-6, so only a few codes can differ and the
    # bars (twice the oracle's spread under a 1e-6 move of its quantiser
    # inputs) are far tighter than in bf16
    w = workload("tiny").with_(mlp_fp8=True)
    _block_case(w, 0, 2, 37)



def test_stack_d26_all_features():
    # the d26 block as specified: residual mixing, value embeddings on odd
    # layers, smear, backout and the fp8 MLP; 4 layers, vocabulary cut to 512
    _stack_case(workload("d26").with_(n_layer=4, B=1, T=128, vocab=512, windows=(-1,) * 4))
