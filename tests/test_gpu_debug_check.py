"""The GDB_CHECK_FINITE debug check of the block and head entry points.

With the variable set (to anything but "0"), an entry point whose output holds
a NaN or an infinity returns GDB_ENONFINITE and names that output; unset or
"0", the same call succeeds and the values simply propagate.  The non-finite
values come from the inputs (a NaN in one token's activations, an infinite
upstream gradient, a NaN in one row of the head's input), which the kernels
carry through ordinary arithmetic; finite inputs pass with the check on."""
import numpy as np
import pytest
import torch

from gpt_decoder_block_amd import _lib as L
from gpt_decoder_block_amd import ops
from gpu_util import DEV, TDT, dev, empty, rounded
from seeded_inputs import draw_ids, draw_layer, draw_upstream, workload

pytestmark = pytest.mark.gpu


def _wl(dt):
    w = workload("tiny")
    # the bf16 attention path needs head_dim 128
    return w if dt == "f32" else w.with_(dtype="bf16", C=256, head_dim=128, mlp_hidden=1024)


def _expect(fn, name, monkeypatch):
    """fn() succeeds with the check off and fails naming `name` with it on."""
    monkeypatch.delenv("GDB_CHECK_FINITE", raising=False)
    fn()
    monkeypatch.setenv("GDB_CHECK_FINITE", "0")
    fn()
    monkeypatch.setenv("GDB_CHECK_FINITE", "1")
    with pytest.raises(L.GdbError) as ei:
        fn()
    assert ei.value.status == L.GDB_ENONFINITE, ei.value
    assert ei.value.msg.startswith(name + " "), ei.value.msg


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_block_outputs_checked(dt, monkeypatch):
    w = _wl(dt)
    B, T, C = w.B, w.T, w.C
    N = B * T
    print(f"debug check block dt={dt} C={C}", flush=True)
    p = {k: rounded(v, dt) for k, v in draw_layer(w, 0).items()}
    cfg = ops.make_cfg(B, T, C, w.n_head, w.n_kv_head, w.head_dim, w.mlp_hidden, w.windows[0], TDT[dt], w.eps)
    sv, wf, wb = ops.block_sizes(cfg)
    saved = torch.empty(sv, dtype=torch.uint8, device=DEV)
    wsf = torch.empty(wf, dtype=torch.uint8, device=DEV)
    wsb = torch.empty(wb, dtype=torch.uint8, device=DEV)
    W = [dev(p[k], dt) for k in ("w_qkv", "w_o", "w_fc", "w_proj")]
    dW = [empty(t.shape, torch.float32) for t in W]
    rope = ops.rope_table(T, w.head_dim, w.rope_base, DEV)
    x = rounded(draw_upstream(w, 100, (N, C), 1.0), dt)
    dy = rounded(draw_upstream(w, 200, (N, C), 1.0), dt)
    out, dx = empty((N, C), dt), empty((N, C), dt)

    # finite inputs pass with the check on
    monkeypatch.setenv("GDB_CHECK_FINITE", "1")
    ops.block_fwd(cfg, W, rope, dev(x, dt), out, saved, wsf)
    ops.block_bwd(cfg, W, rope, saved, dev(dy, dt), dx, dW, wsb)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(dx).all()

    # a NaN in one token's input reaches x_out
    xb = x.copy()
    xb[T // 2, 3] = np.nan
    xg = dev(xb, dt)
    _expect(lambda: ops.block_fwd(cfg, W, rope, xg, out, saved, wsf), "x_out", monkeypatch)

    # an infinite upstream gradient reaches dx_in (the first output checked)
    monkeypatch.delenv("GDB_CHECK_FINITE", raising=False)
    ops.block_fwd(cfg, W, rope, dev(x, dt), out, saved, wsf)
    dyb = dy.copy()
    dyb[1, 0] = np.inf
    dyg = dev(dyb, dt)
    _expect(lambda: ops.block_bwd(cfg, W, rope, saved, dyg, dx, dW, wsb), "dx_in", monkeypatch)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_head_outputs_checked(dt, monkeypatch):
    w = _wl(dt)
    N, C, V = w.B * w.T, w.C, w.vocab
    print(f"debug check head dt={dt} N={N} C={C} V={V}", flush=True)
    x = rounded(draw_upstream(w, 300, (N, C), 1.0), dt)
    wl = rounded(draw_upstream(w, 301, (V, C), 0.05), dt)
    tgt = torch.from_numpy(draw_ids(w)[:, 1:].reshape(-1).astype(np.int32)).to(DEV)
    ws = torch.empty(ops.lm_head_ce_sizes(N, C, V, TDT[dt]), dtype=torch.uint8, device=DEV)
    loss = empty((1,), torch.float32)
    dx = empty((N, C), dt)
    dwl = empty((V, C), torch.float32)
    wg = dev(wl, dt)
    monkeypatch.setenv("GDB_CHECK_FINITE", "1")
    ops.lm_head_ce_fwd_bwd(dev(x, dt), wg, tgt, loss, dx, dwl, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(loss).all()
    xb = x.copy()
    xb[7, :] = np.nan
    xg = dev(xb, dt)
    _expect(lambda: ops.lm_head_ce_fwd_bwd(xg, wg, tgt, loss, dx, dwl, ws), "loss", monkeypatch)
