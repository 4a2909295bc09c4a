"""The allocation-free decode entry point (gdb_attention_decode_noalloc),
through the C ABI: its outputs against gdb_attention_decode's (the same
kernels, with a caller workspace) on two calls in a row, the second with a
smaller input, both with several KV splits so the fixed scratch is used."""
import ctypes

import numpy as np
import pytest
import torch

from gpt_decoder_block_amd import _lib as L
from gpt_decoder_block_amd import ops
from gpu_util import DEV, TOL, assert_close, dev, empty, host, rounded

pytestmark = pytest.mark.gpu


def _inputs(dt, B, Tmax, H, Hkv, D, lens, seed):
    g = np.random.default_rng(seed)
    q = dev(rounded(g.standard_normal((B, H * D)), dt), dt)
    k = dev(rounded(g.standard_normal((B, Tmax, Hkv, D)), dt), dt)
    v = dev(rounded(g.standard_normal((B, Tmax, Hkv, D)), dt), dt)
    return q, k, v, torch.tensor(lens, dtype=torch.int32, device=DEV)


def _pair(dt, B, Tmax, H, Hkv, D, window, lens, seed):
    q, k, v, lg = _inputs(dt, B, Tmax, H, Hkv, D, lens, seed)
    max_len = int(max(lens))
    nb = ops.attention_decode_ws_bytes(B, H, Hkv, D, max_len, window)
    assert nb > 0, "the case must split the keys (use the scratch)"
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    o_ref, l_ref = empty((B, H * D), dt, fill=float("nan")), empty((B, H), torch.float32, fill=float("nan"))
    o, ls = empty((B, H * D), dt, fill=float("nan")), empty((B, H), torch.float32, fill=float("nan"))
    print(f"decode noalloc dt={dt} B={B} Tmax={Tmax} H={H}/{Hkv} D={D} window={window} split bytes={nb}", flush=True)
    ops.attention_decode(B, H, Hkv, D, window, q, H * D, k, v, Hkv * D, Tmax * Hkv * D, lg, max_len, o_ref, H * D,
                         l_ref, ws)
    ops.attention_decode_noalloc(B, H, Hkv, D, window, q, H * D, k, v, Hkv * D, Tmax * Hkv * D, lg, max_len, o,
                                 H * D, ls)
    torch.cuda.synchronize()
    return o, ls, o_ref, l_ref


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_decode_noalloc_matches_workspace_entry(dt):
    # first call: 6 sequences up to 5000 keys, GQA 4:1, 32 splits of the longest
    first = _pair(dt, 6, 5000, 8, 2, 128, -1, [5000, 1, 4097, 2048, 0, 3333], seed=1)
    # second call, smaller: fewer sequences, shorter cache, a window; the
    # scratch still holds the first call's partials, which must not leak in
    second = _pair(dt, 2, 900, 4, 4, 64, 300, [900, 257], seed=2)
    for o, ls, o_ref, l_ref in (first, second):
        assert_close(o, host(o_ref), dt, "o")
        a, b = host(ls), host(l_ref)
        assert np.array_equal(np.isfinite(a), np.isfinite(b))
        fin = np.isfinite(b)
        assert np.max(np.abs(a[fin] - b[fin]), initial=0.0) <= 1e-5 * max(1.0, np.max(np.abs(b[fin]), initial=0.0))
        # the same kernels on the same inputs: the same bits
        assert torch.equal(o, o_ref) and torch.equal(ls, l_ref)


def test_decode_noalloc_validates_like_the_workspace_entry():
    lib = L.lib()
    buf = ctypes.create_string_buffer(4096)
    al = (ctypes.addressof(buf) + 255) & ~255
    # H not a multiple of Hkv, and a misaligned lse: rejected before any launch
    assert lib.gdb_attention_decode_noalloc(2, 6, 4, 128, -1, 1, al, 768, al, al, 512, 1 << 20, al, 64, al, 768,
                                            None, None) == L.GDB_EINVAL
    assert lib.gdb_attention_decode_noalloc(2, 8, 2, 128, -1, 1, al, 1024, al, al, 256, 1 << 20, al, 64, al, 1024,
                                            al + 4, None) == L.GDB_EINVAL
    assert "lse" in lib.gdb_last_error().decode()
