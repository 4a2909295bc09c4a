"""The C-ABI library on a CPU-only host: it loads, exports every function that
include/gdb.h declares, and rejects bad arguments with a message before any
device work (no compute call is made here)."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdb.h")


@pytest.fixture(scope="module")
def L():
    from gpt_decoder_block_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from gpt_decoder_block_amd import build
        build.build()
    return _lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdb_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("gdb_block_fwd", "gdb_block_bwd", "gdb_lm_head_ce_fwd_bwd", "gdb_embed_fwd", "gdb_embed_bwd",
                 "gdb_smear_fwd", "gdb_smear_bwd", "gdb_backout_fwd", "gdb_backout_bwd"):
        assert must in names


def test_library_exports_every_declared_symbol(L):
    lib = L.lib()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    # and the Python binding covers exactly the declared functions
    assert sorted(L.SIGNATURES) == declared_functions()


def test_abi_version(L):
    # header, library and binding agree
    hdr = open(HEADER).read()
    m = re.search(r"#define GDB_ABI_VERSION (\d+)", hdr)
    assert m and int(m.group(1)) == L.lib().gdb_abi_version() == L.ABI_VERSION


def test_status_codes(L):
    # every gdb_status value the header declares has the same value in the binding
    hdr = open(HEADER).read()
    body = re.search(r"typedef enum \{(.*?)\} gdb_status;", hdr, re.S).group(1)
    codes = dict((n, int(v)) for n, v in re.findall(r"(GDB_[A-Z]+) = (-?\d+)", body))
    assert set(codes) == {"GDB_OK", "GDB_EINVAL", "GDB_EUNSUPPORTED", "GDB_EHIP", "GDB_EWORKSPACE", "GDB_ENONFINITE"}
    for n, v in codes.items():
        assert getattr(L, n) == v, n


def _cfg(L, **kw):
    base = dict(B=2, T=64, C=256, n_head=2, n_kv_head=1, head_dim=128, mlp_hidden=1024, window=-1, dtype=1,
                mlp_fp8=0, accumulate_wgrad=0, deterministic=0, eps=1e-6)
    base.update(kw)
    return L.BlockCfg(**base)


def _sizes(L, cfg):
    s, f, b = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    st = L.lib().gdb_block_sizes(ctypes.byref(cfg), ctypes.byref(s), ctypes.byref(f), ctypes.byref(b))
    return st, s.value, f.value, b.value


def test_block_sizes_valid_and_monotone(L):
    st, s1, f1, b1 = _sizes(L, _cfg(L))
    assert st == L.GDB_OK and s1 > 0 and f1 > 0 and b1 > 0
    st, s2, f2, b2 = _sizes(L, _cfg(L, B=4))
    assert st == L.GDB_OK and s2 > s1 and f2 > f1 and b2 > b1
    # saved activations: xn1, q^k^v, o, xn2, h = relu(u)^2 in bf16 plus fp32 statistics
    N, C, W3, F = 128, 256, 4 * 128, 1024
    assert s1 >= N * (C + W3 + C + C + F) * 2


@pytest.mark.parametrize("kw,code,msg", [
    (dict(n_kv_head=3), -1, "multiple of n_kv_head"),
    (dict(head_dim=96, C=192), -2, "head_dim"),
    (dict(head_dim=64, C=128), -2, "bf16 attention needs head_dim 128"),
    (dict(C=384), -2, "must equal C"),
    (dict(B=0), -1, "positive"),
    (dict(window=-2), -1, "window"),
    (dict(dtype=7), -1, "dtype"),
    (dict(mlp_fp8=1, mlp_hidden=1032), -1, "multiples of 16"),
    (dict(mlp_hidden=1020), -1, "multiples of 8"),
    (dict(eps=0.0), -1, "eps"),
    (dict(deterministic=2), -1, "deterministic"),
])
def test_block_cfg_validation(L, kw, code, msg):
    st, *_ = _sizes(L, _cfg(L, **kw))
    assert st == code
    assert msg in L.lib().gdb_last_error().decode()


def test_deterministic_backward_reserves_sort_scratch(L):
    # the fixed-order path sorts the token ids in the backward workspace
    st, s0, f0, b0 = _sizes(L, _cfg(L))
    st1, s1, f1, b1 = _sizes(L, _cfg(L, deterministic=1))
    assert st == st1 == L.GDB_OK and (s1, f1) == (s0, f0) and b1 > b0
    n = ctypes.c_size_t()
    assert L.lib().gdb_embed_bwd_ws_bytes(4096, 1, ctypes.byref(n)) == L.GDB_OK and n.value >= 4 * 4096 * 4
    assert L.lib().gdb_embed_bwd_ws_bytes(4096, 0, ctypes.byref(n)) == L.GDB_OK and n.value == 0


def test_stage_entry_points_validate(L):
    lib = L.lib()
    buf = ctypes.create_string_buffer(4096)
    al = (ctypes.addressof(buf) + 255) & ~255
    # mixing: lam misaligned, bad sizes
    assert lib.gdb_mix_fwd(4, 12, 1, al, al, al + 2, al, None) == L.GDB_EINVAL
    assert lib.gdb_mix_fwd(4, 12, 1, al, al, al, al, None) == L.GDB_EINVAL
    assert "multiple of 8" in lib.gdb_last_error().decode()
    # value embedding: unsupported head size, gate width, voff past the row
    assert lib.gdb_ve_fwd(4, 2, 96, 1, al, 512, 256, al, 128, al, al, 10, al, 32, al, None) == L.GDB_EUNSUPPORTED
    assert lib.gdb_ve_fwd(4, 2, 128, 1, al, 512, 256, al, 128, al, al, 10, al, 65, al, None) == L.GDB_EINVAL
    assert lib.gdb_ve_fwd(4, 2, 128, 1, al, 512, 384, al, 128, al, al, 10, al, 32, al, None) == L.GDB_EINVAL
    n = ctypes.c_size_t()
    assert lib.gdb_ve_bwd_ws_bytes(100, 2, 32, 1, ctypes.byref(n)) == L.GDB_OK and n.value > 0
    # NorMuon: beta2 out of range, workspace too small
    coeffs = (ctypes.c_float * 3)(1.5, -0.5, 0.0)
    assert lib.gdb_normuon_step(1, 16, 16, 1, al, None, al, al, al, 0.1, 0.9, 1, 0.0, 1.0, 1.0, coeffs, 1, 1.0,
                                1e-7, al, 1 << 30, None) == L.GDB_EINVAL
    assert "beta2" in lib.gdb_last_error().decode()
    assert lib.gdb_normuon_ws_bytes(2, 16, 24, 1, ctypes.byref(n)) == L.GDB_OK
    need = n.value
    assert lib.gdb_normuon_step(2, 16, 24, 1, al, None, al, al, al, 0.1, 0.9, 1, 0.0, 1.0, 0.95, coeffs, 1, 1.0,
                                1e-7, al, need - 1, None) == L.GDB_EWORKSPACE


def test_block_fwd_rejects_null_and_misaligned_pointers(L):
    lib = L.lib()
    cfg = _cfg(L)
    buf = ctypes.create_string_buffer(4096)
    base = ctypes.addressof(buf)
    al = (base + 255) & ~255
    w = L.BlockWeights(al, al, al, al)
    st = lib.gdb_block_fwd(ctypes.byref(cfg), ctypes.byref(w), None, None, al, al + 512, al, al, None)
    assert st == L.GDB_EINVAL and "rope_tab is NULL" in lib.gdb_last_error().decode()
    st = lib.gdb_block_fwd(ctypes.byref(cfg), ctypes.byref(w), None, al, al + 2, al + 512, al, al, None)
    assert st == L.GDB_EINVAL and "x_in is not 16-byte aligned" in lib.gdb_last_error().decode()
    st = lib.gdb_block_fwd(ctypes.byref(cfg), ctypes.byref(w), None, al, al, al, al, al, None)
    assert st == L.GDB_EINVAL and "alias" in lib.gdb_last_error().decode()
    st = lib.gdb_block_fwd(ctypes.byref(cfg), None, None, al, al, al + 512, al, al, None)
    assert st == L.GDB_EINVAL
    dw = L.BlockWgrads(al, 0, al, al)
    st = lib.gdb_block_bwd(ctypes.byref(cfg), ctypes.byref(w), None, al, al, al, al, ctypes.byref(dw), None, al,
                           None)
    assert st == L.GDB_EINVAL and "dw_o is NULL" in lib.gdb_last_error().decode()


def test_block_extras_validation(L):
    lib = L.lib()
    cfg = _cfg(L)
    buf = ctypes.create_string_buffer(4096)
    al = (ctypes.addressof(buf) + 255) & ~255
    w = L.BlockWeights(al, al, al, al)
    dw = L.BlockWgrads(al, al, al, al)

    def fwd(ex):
        return lib.gdb_block_fwd(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(ex), al, al, al + 512, al, al,
                                 None)

    assert fwd(L.BlockExtras(lambdas=al)) == L.GDB_EINVAL
    assert "ex->x0 is NULL" in lib.gdb_last_error().decode()
    assert fwd(L.BlockExtras(lambdas=al + 2, x0=al)) == L.GDB_EINVAL
    assert fwd(L.BlockExtras(ve=al, ve_gate=al, ids=al, ve_vocab=100, ve_gate_channels=65)) == L.GDB_EINVAL
    assert "ve_gate_channels" in lib.gdb_last_error().decode()
    assert fwd(L.BlockExtras(ve=al, ve_gate=al, ids=None, ve_vocab=100, ve_gate_channels=32)) == L.GDB_EINVAL
    assert fwd(L.BlockExtras(ve=al, ve_gate=al, ids=al, ve_vocab=0, ve_gate_channels=32)) == L.GDB_EINVAL
    # backward: mixing needs x_in and the gradients
    ex = L.BlockExtras(lambdas=al, x0=al)
    st = lib.gdb_block_bwd(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(ex), al, al, al, al, ctypes.byref(dw),
                           None, al, None)
    assert st == L.GDB_EINVAL and "ex->x_in is NULL" in lib.gdb_last_error().decode()
    ex = L.BlockExtras(lambdas=al, x0=al, x_in=al)
    st = lib.gdb_block_bwd(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(ex), al, al, al, al, ctypes.byref(dw),
                           None, al, None)
    assert st == L.GDB_EINVAL and "without extras gradients" in lib.gdb_last_error().decode()
    dex = L.BlockExtrasGrads(dlambdas=al, dx0=None)
    st = lib.gdb_block_bwd(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(ex), al, al, al, al, ctypes.byref(dw),
                           ctypes.byref(dex), al, None)
    assert st == L.GDB_EINVAL and "dx0 is NULL" in lib.gdb_last_error().decode()


def test_smear_backout_validation(L):
    lib = L.lib()
    al = 1 << 20   # never dereferenced: validation fails first
    assert lib.gdb_smear_fwd(2, 16, 128, 64, 1, al, al, al, al + 4096, al, None) == L.GDB_EINVAL
    assert "ng must be" in lib.gdb_last_error().decode()
    assert lib.gdb_smear_fwd(2, 16, 128, 24, 1, al, al, al, al, al, None) == L.GDB_EINVAL
    assert "alias" in lib.gdb_last_error().decode()
    assert lib.gdb_smear_fwd(2, 16, 12, 8, 1, al, al, al, al + 4096, al, None) == L.GDB_EINVAL
    assert lib.gdb_smear_fwd(0, 16, 128, 24, 1, None, None, None, None, None, None) == L.GDB_OK
    assert lib.gdb_smear_bwd(2, 16, 128, 24, 1, al, al, al, al, al, None, al, al, al, 0, None, None) == L.GDB_EINVAL
    assert "ws is NULL" in lib.gdb_last_error().decode()
    assert lib.gdb_smear_bwd(2, 16, 128, 24, 1, al, al, al, al, al, None, al, al, al, 0, al, None) == L.GDB_EINVAL
    assert "de must not alias" in lib.gdb_last_error().decode()
    assert lib.gdb_backout_fwd(8, 128, 1, al, al + 4096, al, al + 4096, None) == L.GDB_EINVAL
    assert lib.gdb_backout_fwd(0, 128, 1, None, None, None, None, None) == L.GDB_OK
    assert lib.gdb_backout_bwd(8, 128, 1, al, al + 4096, None, al + 8192, al, 0, al, None) == L.GDB_EINVAL
    assert "lam is NULL" in lib.gdb_last_error().decode()
    assert lib.gdb_backout_bwd(8, 128, 1, al, al + 4096, al, al, al, 0, al, None) == L.GDB_EINVAL


def test_gemm_and_attention_validation(L):
    lib = L.lib()
    al = 1 << 20   # never dereferenced: validation fails first
    st = lib.gdb_gemm(1, 64, 60, 64, al, 1, 64, al, 1, 64, 0, al, 60, None, 0, None, 0, None, None)
    assert st == L.GDB_EINVAL and "multiples of 8" in lib.gdb_last_error().decode()
    st = lib.gdb_gemm(1, 64, 64, 64, al, 1, 32, al, 1, 64, 0, al, 64, None, 0, None, 0, None, None)
    assert st == L.GDB_EINVAL and "leading dimension" in lib.gdb_last_error().decode()
    st = lib.gdb_gemm(1, 64, 64, 64, al, 1, 64, al, 1, 64, 9, al, 64, None, 0, None, 0, None, None)
    assert st == L.GDB_EINVAL and "epilogue" in lib.gdb_last_error().decode()
    st = lib.gdb_gemm(1, 64, 64, 64, al, 1, 64, al, 1, 64, 1, al, 64, None, 64, None, 0, None, None)
    assert st == L.GDB_EINVAL and "R is NULL" in lib.gdb_last_error().decode()
    st = lib.gdb_attention_fwd(1, 64, 3, 2, 128, -1, 0, 1, al, 896, al, 384, al, None)
    assert st == L.GDB_EINVAL and "multiple of Hkv" in lib.gdb_last_error().decode()
    st = lib.gdb_attention_fwd(1, 64, 2, 1, 64, -1, 0, 1, al, 256, al, 128, al, None)
    assert st == L.GDB_EUNSUPPORTED
    # bf16 kernels address a sequence's rows with 32-bit byte offsets
    st = lib.gdb_attention_fwd(1, 4096, 2, 1, 128, -1, 0, 1, al, 262144, al, 256, al, None)
    assert st == L.GDB_EUNSUPPORTED and "2 GiB" in lib.gdb_last_error().decode()
    st = lib.gdb_attention_bwd(1, 4096, 2, 1, 128, -1, 1, al, 512, al, 256, al, al, 262144, al, 512, al, None)
    assert st == L.GDB_EUNSUPPORTED and "dO rows" in lib.gdb_last_error().decode()
    st = lib.gdb_lm_head_ce_fwd_bwd(8, 128, 100, 1, 1e-6, al, al, al, al, None, al, al, 0, al, None)
    assert st == L.GDB_EINVAL and "multiples of 8" in lib.gdb_last_error().decode()
    st = lib.gdb_lm_head_ce_fwd_bwd(8, 128, 128, 1, 1e-6, al, al, al, al, al + 2, al, al, 0, al, None)
    assert st == L.GDB_EINVAL and "row_loss" in lib.gdb_last_error().decode()
    st = lib.gdb_lm_head_ce_fwd_bwd(8, 128, 100, 1, 1e-6, al, al, al, al, None, al, al, 0, al, None)
    assert st == L.GDB_EINVAL and "multiples of 8" in lib.gdb_last_error().decode()
    st = lib.gdb_embed_fwd(8, 12, 100, 1, al, al, al, None)
    assert st == L.GDB_EINVAL


def test_rope_table_host(L):
    T, D, base = 37, 64, 10000.0
    out = np.zeros((T, D // 2, 2), dtype=np.float32)
    st = L.lib().gdb_rope_table_host(T, D, base, out.ctypes.data_as(ctypes.c_void_p))
    assert st == L.GDB_OK
    t = np.arange(T)[:, None]
    j = np.arange(D // 2)[None, :]
    th = t * base ** (-2.0 * j / D)
    np.testing.assert_array_equal(out[..., 0], np.cos(th).astype(np.float32))
    np.testing.assert_array_equal(out[..., 1], np.sin(th).astype(np.float32))
    assert L.lib().gdb_rope_table_host(T, 63, base, out.ctypes.data_as(ctypes.c_void_p)) == L.GDB_EINVAL


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from gpt_decoder_block_amd import _lib
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        _lib.lib()


def test_fp8_sizes_and_validation(L):
    lib = L.lib()
    st, s0, f0, b0 = _sizes(L, _cfg(L))
    st8, s1, f1, b1 = _sizes(L, _cfg(L, mlp_fp8=1))
    assert st == st8 == L.GDB_OK
    # the fp8 path keeps transposed codes of xn2, h and both weights for the backward
    N, C, F = 128, 256, 1024
    assert s1 - s0 >= N * (C + F) + 2 * C * F and f1 > f0 and b1 > b0
    al = 1 << 20   # never dereferenced: validation fails first
    assert lib.gdb_fp8_quantize(64, 24, 1, al, al, al, None, 0, None) == L.GDB_EINVAL
    assert "multiple of 16" in lib.gdb_last_error().decode()
    assert lib.gdb_fp8_quantize(64, 32, 1, al, al, None, al, 60, None) == L.GDB_EINVAL
    assert "Rp" in lib.gdb_last_error().decode()
    assert lib.gdb_fp8_quantize(64, 32, 1, al, al, None, None, 64, None) == L.GDB_EINVAL
    assert lib.gdb_fp8_quantize(64, 32, 1, al, None, al, None, 0, None) == L.GDB_EINVAL
    assert lib.gdb_gemm_fp8(1, 64, 64, 40, al, 40, al, al, 40, al, 0, al, 64, None, 0, None, 0, None,
                            None) == L.GDB_EINVAL
    assert "multiples of 16" in lib.gdb_last_error().decode()
    assert lib.gdb_gemm_fp8(1, 64, 64, 64, al, 64, None, al, 64, al, 0, al, 64, None, 0, None, 0, None,
                            None) == L.GDB_EINVAL
    assert "amax" in lib.gdb_last_error().decode()
    assert lib.gdb_gemm_fp8(1, 64, 64, 64, al, 64, al, al, 64, al, 3, al, 64, None, 64, None, 0, None,
                            None) == L.GDB_EINVAL
    assert "R is NULL" in lib.gdb_last_error().decode()
    assert lib.gdb_gemm_fp8(5, 64, 64, 64, al, 64, al, al, 64, al, 0, al, 64, None, 0, None, 0, None,
                            None) == L.GDB_EINVAL
    ws = ctypes.c_size_t()
    assert lib.gdb_gemm_fp8_ws_bytes(1536, 6144, 32768, 4, ctypes.byref(ws)) == L.GDB_OK


def test_attention_decode_validation(L):
    # every rejection happens before a launch (no GPU here)
    lib = L.lib()
    buf = ctypes.create_string_buffer(4096)
    al = (ctypes.addressof(buf) + 255) & ~255
    nb = ctypes.c_size_t()

    def call(B=2, H=12, Hkv=12, D=128, window=-1, dtype=1, ldq=1536, ldk=1536, bstride=2048 * 1536, lens=al,
             max_len=2048, ldo=1536, lse=None, ws=al, ws_bytes=1 << 30, q=al):
        return lib.gdb_attention_decode(B, H, Hkv, D, window, dtype, q, ldq, al, al, ldk, bstride, lens, max_len,
                                        al, ldo, lse, ws, ws_bytes, None)

    assert lib.gdb_attention_decode_ws_bytes(2, 12, 12, 128, 2048, -1, ctypes.byref(nb)) == L.GDB_OK
    assert nb.value > 0   # 2048 positions split over several workgroups
    assert lib.gdb_attention_decode_ws_bytes(2, 12, 12, 128, 64, -1, ctypes.byref(nb)) == L.GDB_OK
    assert nb.value == 0  # one chunk: no partials
    assert call(H=12, Hkv=5) == L.GDB_EINVAL
    assert call(H=10, Hkv=2) == L.GDB_EUNSUPPORTED and "H / Hkv = 5" in lib.gdb_last_error().decode()
    assert call(D=96) == L.GDB_EUNSUPPORTED
    assert call(max_len=0) == L.GDB_EINVAL
    assert call(window=-2) == L.GDB_EINVAL
    assert call(dtype=7) == L.GDB_EINVAL
    assert call(ldk=1000) == L.GDB_EINVAL and "leading dimension" in lib.gdb_last_error().decode()
    assert call(bstride=2047 * 1536) == L.GDB_EINVAL and "bstride" in lib.gdb_last_error().decode()
    assert call(lens=None) == L.GDB_EINVAL and "lens is NULL" in lib.gdb_last_error().decode()
    assert call(q=al + 8) == L.GDB_EINVAL and "aligned" in lib.gdb_last_error().decode()
    assert call(lse=al + 4) == L.GDB_EINVAL
    assert call(ws=None) == L.GDB_EINVAL
    assert call(ws_bytes=16) == L.GDB_EWORKSPACE


def test_optimizer_validation(L):
    lib = L.lib()
    buf = ctypes.create_string_buffer(4096)
    al = (ctypes.addressof(buf) + 255) & ~255
    nb = ctypes.c_size_t()
    co = (ctypes.c_float * 6)(8.156, -22.483, 15.879, 4.043, -2.809, 0.5)
    assert lib.gdb_newton_schulz_ws_bytes(1, 1536, 6144, 1, ctypes.byref(nb)) == L.GDB_OK and nb.value > 0
    big = nb.value
    assert lib.gdb_newton_schulz_ws_bytes(24, 1536, 6144, 1, ctypes.byref(nb)) == L.GDB_OK and nb.value > big

    def ns(m=64, n=32, dtype=1, G=al, X=al + 256, coeffs=co, steps=2, ns_=1.0, eps=1e-7, ws=al, wsb=big, count=1):
        return lib.gdb_newton_schulz(count, m, n, dtype, G, X, coeffs, steps, ctypes.c_float(ns_),
                                     ctypes.c_float(eps), ws, wsb, None)

    assert ns(m=60) == L.GDB_EINVAL and "multiples of 8" in lib.gdb_last_error().decode()
    assert ns(count=0) == L.GDB_EINVAL and "count" in lib.gdb_last_error().decode()
    assert ns(dtype=5) == L.GDB_EINVAL
    assert ns(steps=65) == L.GDB_EINVAL
    assert ns(coeffs=None) == L.GDB_EINVAL
    assert ns(coeffs=(ctypes.c_float * 6)(1, float("nan"), 0, 1, 1, 1)) == L.GDB_EINVAL
    assert ns(ns_=0.0) == L.GDB_EINVAL
    assert ns(X=al) == L.GDB_EINVAL and "alias" in lib.gdb_last_error().decode()
    assert ns(wsb=16) == L.GDB_EWORKSPACE
    assert ns(G=al + 4) == L.GDB_EINVAL
    # AdamW
    f = ctypes.c_float
    assert lib.gdb_adamw_step(12, al, None, al, al, al, 1, f(1e-3), f(0.9), f(0.95), f(1e-8), f(0.0), None) \
        == L.GDB_EINVAL
    assert lib.gdb_adamw_step(16, al, None, al, al, al, 0, f(1e-3), f(0.9), f(0.95), f(1e-8), f(0.0), None) \
        == L.GDB_EINVAL
    assert lib.gdb_adamw_step(16, al, None, al, al, al, 1, f(1e-3), f(1.0), f(0.95), f(1e-8), f(0.0), None) \
        == L.GDB_EINVAL
    assert lib.gdb_adamw_step(16, al, al + 2, al, al, al, 1, f(1e-3), f(0.9), f(0.95), f(1e-8), f(0.0), None) \
        == L.GDB_EINVAL
    # Muon
    assert lib.gdb_muon_ws_bytes(1, 64, 32, 1, ctypes.byref(nb)) == L.GDB_OK
    st = lib.gdb_muon_step(1, 64, 32, 1, al, None, al, None, f(0.02), f(0.95), 1, f(0.0), f(1.0), co, 2, f(1.0),
                           f(1e-7), al, nb.value, None)
    assert st == L.GDB_EINVAL and "buf is NULL" in lib.gdb_last_error().decode()
    st = lib.gdb_muon_step(1, 64, 32, 1, al, None, al, al, f(float("inf")), f(0.95), 1, f(0.0), f(1.0), co, 2, f(1.0),
                           f(1e-7), al, nb.value, None)
    assert st == L.GDB_EINVAL
