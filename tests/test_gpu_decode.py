"""Parity of the decode attention kernel (one new query per sequence against a
key/value cache) with the CPU oracle, through the C ABI: ragged lengths,
windows (including 0 and a window edge inside a chunk), GQA groups, one and
several KV splits, both cache layouts, and the d24 decode shape in full."""
import numpy as np
import pytest
import torch

import oracle as O
from gpt_decoder_block_amd import ops
from gpu_util import DEV, TOL, assert_close, dev, empty, host, rounded

pytestmark = pytest.mark.gpu


def _run_cache(dt, B, Tmax, H, Hkv, D, window, lens, seed=0, lse=True):
    """Dedicated cache [B, Tmax, Hkv, D]; returns (o, lse) from the GPU and the oracle's."""
    g = np.random.default_rng(seed)
    q = rounded(g.standard_normal((B, H, D)), dt)
    k = rounded(g.standard_normal((B, Tmax, Hkv, D)), dt)
    v = rounded(g.standard_normal((B, Tmax, Hkv, D)), dt)
    qg, kg, vg = dev(q, dt), dev(k, dt), dev(v, dt)
    max_len = int(max(lens))
    lg = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o = empty((B, H * D), dt, fill=float("nan"))
    ls = empty((B, H), torch.float32, fill=float("nan")) if lse else None
    nb = ops.attention_decode_ws_bytes(B, H, Hkv, D, max_len, window)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV) if nb else None
    print(f"decode cache dt={dt} B={B} Tmax={Tmax} H={H}/{Hkv} D={D} window={window} lens={list(lens)[:8]} "
          f"ws={nb}", flush=True)
    ops.attention_decode(B, H, Hkv, D, window, qg, H * D, kg, vg, Hkv * D, Tmax * Hkv * D, lg, max_len, o, H * D,
                         ls, ws)
    torch.cuda.synchronize()
    o_ref, lse_ref = O.attention_decode(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                                        np.asarray(lens), window)
    return o, ls, o_ref.reshape(B, H * D), lse_ref


def _check(dt, o, ls, o_ref, lse_ref):
    assert_close(o, o_ref, dt, "o")
    if ls is not None:
        lg = host(ls)
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lg), fin)
        assert np.max(np.abs(lg[fin] - lse_ref[fin])) <= 1e-5 * max(1.0, np.max(np.abs(lse_ref[fin])))


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("f32", 128), ("f32", 64), ("bf16", 64)])
@pytest.mark.parametrize("H,Hkv", [(12, 12), (6, 2), (8, 1), (4, 4)])
@pytest.mark.parametrize("window", [-1, 0, 40])
def test_decode_ragged(dt, D, H, Hkv, window):
    # lengths 1 .. Tmax, several not multiples of any tile or chunk size
    lens = [1, 77, 300, 129, 64]
    o, ls, o_ref, lse_ref = _run_cache(dt, len(lens), 300, H, Hkv, D, window, lens, seed=H * 7 + Hkv + D)
    _check(dt, o, ls, o_ref, lse_ref)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_decode_one_split_and_many(dt):
    # short sequences (one chunk: the workgroup writes the output itself), then
    # a single long sequence cut into many splits
    o, ls, o_ref, lse_ref = _run_cache(dt, 3, 64, 12, 12, 128, -1, [64, 33, 5], seed=1)
    _check(dt, o, ls, o_ref, lse_ref)
    o, ls, o_ref, lse_ref = _run_cache(dt, 1, 4000, 6, 2, 128, -1, [3999], seed=2)
    _check(dt, o, ls, o_ref, lse_ref)
    o, ls, o_ref, lse_ref = _run_cache(dt, 1, 4000, 6, 2, 128, 1500, [4000], seed=3)
    _check(dt, o, ls, o_ref, lse_ref)


def test_decode_without_lse_and_empty_sequence():
    # lse may be omitted; a length of 0 gives zeros (lse -inf)
    o, _, o_ref, _ = _run_cache("bf16", 3, 200, 6, 2, 128, -1, [200, 17, 90], seed=4, lse=False)
    _check("bf16", o, None, o_ref, None)
    o, ls, o_ref, lse_ref = _run_cache("bf16", 3, 200, 6, 2, 128, 30, [0, 17, 200], seed=5)
    assert np.all(host(o)[0] == 0) and np.all(np.isneginf(host(ls)[0]))
    _check("bf16", o, ls, o_ref, lse_ref)


@pytest.mark.parametrize("window", [-1, 10])
def test_decode_packed_prefill_rows(window):
    # K and V read straight from the packed QKV rows a prefill wrote
    # ([B*T, (H + 2Hkv)*D]: q heads, k heads, v heads), the new query separate
    dt, B, T, H, Hkv, D = "bf16", 2, 150, 6, 2, 128
    W3 = (H + 2 * Hkv) * D
    g = np.random.default_rng(11)
    qkv = rounded(g.standard_normal((B * T, W3)), dt)
    q = rounded(g.standard_normal((B, H, D)), dt)
    lens = [150, 61]
    qkvg, qg = dev(qkv, dt), dev(q, dt)
    flat = qkvg.view(-1)
    o = empty((B, H * D), dt)
    ls = empty((B, H), torch.float32)
    nb = ops.attention_decode_ws_bytes(B, H, Hkv, D, T, window)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV)
    print(f"decode packed window={window} ws={nb}", flush=True)
    ops.attention_decode(B, H, Hkv, D, window, qg, H * D, flat[H * D:], flat[(H + Hkv) * D:], W3, T * W3,
                         torch.tensor(lens, dtype=torch.int32, device=DEV), T, o, H * D, ls, ws)
    torch.cuda.synchronize()
    rows = qkv.astype(np.float64).reshape(B, T, H + 2 * Hkv, D)
    o_ref, lse_ref = O.attention_decode(q.astype(np.float64), rows[:, :, H:H + Hkv], rows[:, :, H + Hkv:],
                                        np.asarray(lens), window)
    _check(dt, o, ls, o_ref.reshape(B, H * D), lse_ref)


@pytest.mark.parametrize("window,ragged", [(-1, False), (1024, False), (-1, True)])
def test_decode_d24_full_size(window, ragged):
    # the d24 decode shape (16 sequences, 12 heads of 128, 2048 cached
    # positions) compared in full; the ragged case spreads lengths over 1..2048
    lens = (np.linspace(1, 2048, 16).astype(int).tolist() if ragged else [2048] * 16)
    o, ls, o_ref, lse_ref = _run_cache("bf16", 16, 2048, 12, 12, 128, window, lens, seed=24)
    _check("bf16", o, ls, o_ref, lse_ref)
