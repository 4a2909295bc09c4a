"""Python names of the C-ABI entry points (include/gdb.h), taking torch tensors.

Marshalling only: each function checks that tensors are contiguous device
tensors of the expected dtype, passes raw pointers and the current HIP stream,
and raises GdbError with the library's message on a non-zero status.  PyTorch
provides device memory and streams; it computes nothing here.
"""
from __future__ import annotations

import ctypes
from typing import Sequence, Tuple

import torch

from . import _lib as L

_DT = {torch.float32: L.GDB_F32, torch.bfloat16: L.GDB_BF16}


def dtype_code(dt: torch.dtype) -> int:
    if dt not in _DT:
        raise ValueError(f"unsupported dtype {dt}")
    return _DT[dt]


def _p(t: torch.Tensor) -> ctypes.c_void_p:
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor) -> ctypes.c_void_p:
    if t.device.type != "cuda":
        raise ValueError("tensors must live on the GPU (device 'cuda')")
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def make_cfg(B: int, T: int, C: int, n_head: int, n_kv_head: int, head_dim: int, mlp_hidden: int,
             window: int, dtype: torch.dtype, eps: float = 1e-6, accumulate_wgrad: bool = False,
             mlp_fp8: bool = False, deterministic: bool = False) -> L.BlockCfg:
    return L.BlockCfg(B, T, C, n_head, n_kv_head, head_dim, mlp_hidden, window, dtype_code(dtype), int(mlp_fp8),
                      int(accumulate_wgrad), int(deterministic), eps)


def block_sizes(cfg: L.BlockCfg) -> Tuple[int, int, int]:
    s, f, b = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    L.call("gdb_block_sizes", ctypes.byref(cfg), ctypes.byref(s), ctypes.byref(f), ctypes.byref(b))
    return s.value, f.value, b.value


def rope_table(T: int, head_dim: int, base: float, device) -> torch.Tensor:
    """[T, head_dim/2, 2] fp32 (cos, sin), filled on the host by the library."""
    host = torch.empty((T, head_dim // 2, 2), dtype=torch.float32)
    L.call("gdb_rope_table_host", T, head_dim, base, ctypes.c_void_p(host.data_ptr()))
    return host.to(device)


def embed_fwd(ids: torch.Tensor, wte: torch.Tensor, x0: torch.Tensor) -> None:
    V, C = wte.shape
    L.call("gdb_embed_fwd", ids.numel(), C, V, dtype_code(wte.dtype), _p(ids), _p(wte), _p(x0), _stream(wte))


def embed_bwd_ws_bytes(N: int, deterministic: bool) -> int:
    n = ctypes.c_size_t()
    L.call("gdb_embed_bwd_ws_bytes", N, int(deterministic), ctypes.byref(n))
    return n.value


def embed_bwd(ids: torch.Tensor, dx0: torch.Tensor, dwte: torch.Tensor, accumulate: bool = False,
              ws: torch.Tensor = None) -> None:
    """ws given: the deterministic (fixed-order) path, ws of embed_bwd_ws_bytes(N, True) bytes."""
    V, C = dwte.shape
    L.call("gdb_embed_bwd", ids.numel(), C, V, dtype_code(dx0.dtype), _p(ids), _p(dx0), _p(dwte),
           int(accumulate), int(ws is not None), None if ws is None else _p(ws), _stream(dwte))


def _weights(w: Sequence[torch.Tensor]) -> L.BlockWeights:
    return L.BlockWeights(*[t.data_ptr() for t in w])


def block_extras(lambdas: torch.Tensor = None, x0: torch.Tensor = None, x_in: torch.Tensor = None,
                 ids: torch.Tensor = None, ve: torch.Tensor = None, ve_gate: torch.Tensor = None) -> L.BlockExtras:
    """Extras of one block (residual mixing when `lambdas` is given, value
    embedding when `ve` is given).  The tensors must outlive the calls."""
    ex = L.BlockExtras()
    if lambdas is not None:
        if lambdas.dtype != torch.float32 or lambdas.numel() != 2:
            raise ValueError("lambdas must be a float32 tensor of 2 elements")
        ex.lambdas, ex.x0 = _p(lambdas).value, _p(x0).value
        if x_in is not None:
            ex.x_in = _p(x_in).value
    if ve is not None:
        if ids.dtype != torch.int32:
            raise ValueError("ids must be int32")
        ex.ids, ex.ve, ex.ve_gate = _p(ids).value, _p(ve).value, _p(ve_gate).value
        ex.ve_vocab, ex.ve_gate_channels = ve.shape[0], ve_gate.shape[1]
    return ex


def block_extras_grads(dlambdas: torch.Tensor = None, dx0: torch.Tensor = None, dve: torch.Tensor = None,
                       dve_gate: torch.Tensor = None, accumulate_dx0: bool = False) -> L.BlockExtrasGrads:
    g = L.BlockExtrasGrads()
    for name, t in (("dlambdas", dlambdas), ("dx0", dx0), ("dve", dve), ("dve_gate", dve_gate)):
        if t is not None:
            if t.dtype != torch.float32:
                raise ValueError(f"{name} must be float32")
            setattr(g, name, _p(t).value)
    g.accumulate_dx0 = int(accumulate_dx0)
    return g


def block_fwd(cfg: L.BlockCfg, w: Sequence[torch.Tensor], rope: torch.Tensor, x_in: torch.Tensor,
              x_out: torch.Tensor, saved: torch.Tensor, ws: torch.Tensor, ex: L.BlockExtras = None) -> None:
    for t in w:
        _p(t)
    L.call("gdb_block_fwd", ctypes.byref(cfg), ctypes.byref(_weights(w)), None if ex is None else ctypes.byref(ex),
           _p(rope), _p(x_in), _p(x_out), _p(saved), _p(ws), _stream(x_in))


def block_bwd(cfg: L.BlockCfg, w: Sequence[torch.Tensor], rope: torch.Tensor, saved: torch.Tensor,
              dx_out: torch.Tensor, dx_in: torch.Tensor, dw: Sequence[torch.Tensor], ws: torch.Tensor,
              ex: L.BlockExtras = None, dex: L.BlockExtrasGrads = None) -> None:
    for t in list(w) + list(dw):
        _p(t)
    wg = L.BlockWgrads(*[t.data_ptr() for t in dw])
    L.call("gdb_block_bwd", ctypes.byref(cfg), ctypes.byref(_weights(w)), None if ex is None else ctypes.byref(ex),
           _p(rope), _p(saved), _p(dx_out), _p(dx_in), ctypes.byref(wg), None if dex is None else ctypes.byref(dex),
           _p(ws), _stream(dx_out))


def smear_fwd(B: int, T: int, e: torch.Tensor, w: torch.Tensor, lam: torch.Tensor, x: torch.Tensor,
              s_save: torch.Tensor) -> None:
    C = e.shape[-1]
    L.call("gdb_smear_fwd", B, T, C, w.numel(), dtype_code(e.dtype), _p(e), _p(w), _p(lam), _p(x), _p(s_save),
           _stream(e))


def smear_bwd(B: int, T: int, e: torch.Tensor, w: torch.Tensor, lam: torch.Tensor, s_save: torch.Tensor,
              dx: torch.Tensor, dxa, de: torch.Tensor, dlam: torch.Tensor, dw: torch.Tensor, ws: torch.Tensor,
              accumulate: bool = False) -> None:
    C = e.shape[-1]
    L.call("gdb_smear_bwd", B, T, C, w.numel(), dtype_code(e.dtype), _p(e), _p(w), _p(lam), _p(s_save), _p(dx),
           None if dxa is None else _p(dxa), _p(de), _p(dlam), _p(dw), int(accumulate), _p(ws), _stream(e))


def backout_fwd(x: torch.Tensor, x_bo: torch.Tensor, lam: torch.Tensor, y: torch.Tensor) -> None:
    C = x.shape[-1]
    L.call("gdb_backout_fwd", x.numel() // C, C, dtype_code(x.dtype), _p(x), _p(x_bo), _p(lam), _p(y), _stream(x))


def backout_bwd(dy: torch.Tensor, x_bo: torch.Tensor, lam: torch.Tensor, dx_bo: torch.Tensor, dlam: torch.Tensor,
                ws: torch.Tensor, accumulate: bool = False) -> None:
    C = dy.shape[-1]
    L.call("gdb_backout_bwd", dy.numel() // C, C, dtype_code(dy.dtype), _p(dy), _p(x_bo), _p(lam), _p(dx_bo),
           _p(dlam), int(accumulate), _p(ws), _stream(dy))


def lm_head_ce_sizes(N: int, C: int, V: int, dtype: torch.dtype) -> int:
    s = ctypes.c_size_t()
    L.call("gdb_lm_head_ce_sizes", N, C, V, dtype_code(dtype), ctypes.byref(s))
    return s.value


def lm_head_ce_fwd_bwd(x: torch.Tensor, w_lm: torch.Tensor, targets: torch.Tensor, loss: torch.Tensor,
                       dx: torch.Tensor, dw_lm: torch.Tensor, ws: torch.Tensor, eps: float = 1e-6,
                       accumulate: bool = False, row_loss: torch.Tensor = None) -> None:
    N, C = x.shape[-2] if x.dim() == 2 else x.numel() // x.shape[-1], x.shape[-1]
    V = w_lm.shape[0]
    L.call("gdb_lm_head_ce_fwd_bwd", N, C, V, dtype_code(x.dtype), eps, _p(x), _p(w_lm), _p(targets), _p(loss),
           _opt(row_loss), _p(dx), _p(dw_lm), int(accumulate), _p(ws), _stream(x))


# ------------------------------------------------------------ building blocks
def _opt(t):
    return None if t is None else _p(t)


def stream_copy(src: torch.Tensor, dst: torch.Tensor) -> None:
    """dst = src (same byte size, a multiple of 16): the bandwidth reference copy."""
    nb = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nb:
        raise ValueError("src and dst must have the same size in bytes")
    L.call("gdb_stream_copy", nb, _p(src), _p(dst), _stream(src))


def rmsnorm_fwd(x: torch.Tensor, xn: torch.Tensor, r: torch.Tensor, eps: float = 1e-6) -> None:
    C = x.shape[-1]
    L.call("gdb_rmsnorm_fwd", x.numel() // C, C, dtype_code(x.dtype), eps, _p(x), _p(xn), _p(r), _stream(x))


def rmsnorm_bwd(dxn: torch.Tensor, xn: torch.Tensor, r: torch.Tensor, dres, dx: torch.Tensor) -> None:
    C = dxn.shape[-1]
    L.call("gdb_rmsnorm_bwd", dxn.numel() // C, C, dtype_code(dxn.dtype), _p(dxn), _p(xn), _p(r), _opt(dres),
           _p(dx), _stream(dxn))


EPI_STORE, EPI_RESID, EPI_RELU2, EPI_DRELU2, EPI_F32, EPI_SQR, EPI_DSQR = 0, 1, 2, 3, 4, 6, 7


def gemm_ws_bytes(dtype: torch.dtype, M: int, N: int, K: int, epi: int) -> int:
    s = ctypes.c_size_t()
    L.call("gdb_gemm_ws_bytes", dtype_code(dtype), M, N, K, epi, ctypes.byref(s))
    return s.value


def gemm(M: int, N: int, K: int, A: torch.Tensor, a_kmajor: bool, lda: int, B: torch.Tensor, b_kmajor: bool,
         ldb: int, epi: int, C: torch.Tensor, ldc: int, R=None, ldr: int = 0, C2=None, accumulate: bool = False,
         ws=None) -> None:
    L.call("gdb_gemm", dtype_code(A.dtype), M, N, K, _p(A), int(a_kmajor), lda, _p(B), int(b_kmajor), ldb, epi,
           _p(C), ldc, _opt(R), ldr, _opt(C2), int(accumulate), _opt(ws), _stream(A))


def fp8_quantize(x: torch.Tensor, amax: torch.Tensor, xq=None, xqt=None, Rp: int = 0) -> None:
    """x [R, Cc] -> e4m3 codes (uint8) row-major in xq and/or transposed [Cc, Rp] in xqt; amax fp32 [1]."""
    R, Cc = x.shape
    L.call("gdb_fp8_quantize", R, Cc, dtype_code(x.dtype), _p(x), _p(amax), _opt(xq), _opt(xqt), Rp, _stream(x))


def gemm_fp8_ws_bytes(M: int, N: int, K: int, epi: int) -> int:
    s = ctypes.c_size_t()
    L.call("gdb_gemm_fp8_ws_bytes", M, N, K, epi, ctypes.byref(s))
    return s.value


def gemm_fp8(M: int, N: int, K: int, A: torch.Tensor, lda: int, amax_a: torch.Tensor, B: torch.Tensor, ldb: int,
             amax_b: torch.Tensor, epi: int, C: torch.Tensor, ldc: int, R=None, ldr: int = 0, C2=None,
             accumulate: bool = False, ws=None) -> None:
    out_dt = L.GDB_BF16 if epi == EPI_F32 else dtype_code(C.dtype)
    L.call("gdb_gemm_fp8", out_dt, M, N, K, _p(A), lda, _p(amax_a), _p(B), ldb, _p(amax_b), epi, _p(C), ldc,
           _opt(R), ldr, _opt(C2), int(accumulate), _opt(ws), _stream(A))


def qk_norm_rope_fwd(B: int, T: int, H: int, Hkv: int, D: int, qkv: torch.Tensor, out: torch.Tensor,
                     rinv: torch.Tensor, rope: torch.Tensor, eps: float = 1e-6) -> None:
    L.call("gdb_qk_norm_rope_fwd", B, T, H, Hkv, D, dtype_code(qkv.dtype), eps, _p(qkv), _p(out), _p(rinv),
           _p(rope), _stream(qkv))


def qk_norm_rope_bwd(B: int, T: int, H: int, Hkv: int, D: int, d: torch.Tensor, qkvh: torch.Tensor,
                     rinv: torch.Tensor, rope: torch.Tensor) -> None:
    L.call("gdb_qk_norm_rope_bwd", B, T, H, Hkv, D, dtype_code(d.dtype), _p(d), _p(qkvh), _p(rinv), _p(rope),
           _stream(d))


def attention_fwd(B: int, T: int, H: int, Hkv: int, D: int, window: int, qkv: torch.Tensor, ld: int,
                  o: torch.Tensor, ldo: int, lse: torch.Tensor, qk_normed: bool = False) -> None:
    L.call("gdb_attention_fwd", B, T, H, Hkv, D, window, int(qk_normed), dtype_code(qkv.dtype), _p(qkv), ld, _p(o),
           ldo, _p(lse), _stream(qkv))


def attention_bwd(B: int, T: int, H: int, Hkv: int, D: int, window: int, qkv: torch.Tensor, ld: int,
                  o: torch.Tensor, ldo: int, lse: torch.Tensor, dout: torch.Tensor, lddo: int,
                  dqkv: torch.Tensor, lddq: int, delta: torch.Tensor) -> None:
    L.call("gdb_attention_bwd", B, T, H, Hkv, D, window, dtype_code(qkv.dtype), _p(qkv), ld, _p(o), ldo, _p(lse),
           _p(dout), lddo, _p(dqkv), lddq, _p(delta), _stream(qkv))


def attention_decode_ws_bytes(B: int, H: int, Hkv: int, D: int, max_len: int, window: int) -> int:
    s = ctypes.c_size_t()
    L.call("gdb_attention_decode_ws_bytes", B, H, Hkv, D, max_len, window, ctypes.byref(s))
    return s.value


def attention_decode(B: int, H: int, Hkv: int, D: int, window: int, q: torch.Tensor, ldq: int, k: torch.Tensor,
                     v: torch.Tensor, ldk: int, bstride: int, lens: torch.Tensor, max_len: int, o: torch.Tensor,
                     ldo: int, lse=None, ws=None) -> None:
    """One new query per sequence against its K/V cache (lens: device int32 [B])."""
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    L.call("gdb_attention_decode", B, H, Hkv, D, window, dtype_code(q.dtype), _p(q), ldq, _p(k), _p(v), ldk,
           bstride, _p(lens), max_len, _p(o), ldo, _opt(lse), _opt(ws), nbytes, _stream(q))


def attention_decode_noalloc(B: int, H: int, Hkv: int, D: int, window: int, q: torch.Tensor, ldq: int,
                             k: torch.Tensor, v: torch.Tensor, ldk: int, bstride: int, lens: torch.Tensor,
                             max_len: int, o: torch.Tensor, ldo: int, lse=None) -> None:
    """attention_decode with the library's fixed split scratch (no workspace argument)."""
    L.call("gdb_attention_decode_noalloc", B, H, Hkv, D, window, dtype_code(q.dtype), _p(q), ldq, _p(k), _p(v), ldk,
           bstride, _p(lens), max_len, _p(o), ldo, _opt(lse), _stream(q))


def _coeffs(coeffs):
    flat = [float(x) for t in coeffs for x in t]
    return (ctypes.c_float * max(len(flat), 1))(*flat), len(flat) // 3


def _stack(t: torch.Tensor):
    """(count, m, n) of a [m, n] matrix or a [count, m, n] stack."""
    return (1,) + tuple(t.shape) if t.dim() == 2 else tuple(t.shape)


def newton_schulz_ws_bytes(m: int, n: int, dtype: torch.dtype, count: int = 1) -> int:
    s = ctypes.c_size_t()
    L.call("gdb_newton_schulz_ws_bytes", count, m, n, dtype_code(dtype), ctypes.byref(s))
    return s.value


def newton_schulz(G: torch.Tensor, X: torch.Tensor, coeffs, norm_scale: float = 1.0, eps: float = 1e-7,
                  ws=None) -> None:
    """X (dtype of X) = the Newton-Schulz map of each float32 matrix of G
    ([m, n] or a stack [count, m, n])."""
    count, m, n = _stack(G)
    arr, steps = _coeffs(coeffs)
    L.call("gdb_newton_schulz", count, m, n, dtype_code(X.dtype), _p(G), _p(X), arr, steps, norm_scale, eps, _p(ws),
           ws.numel() * ws.element_size(), _stream(G))


def muon_ws_bytes(m: int, n: int, dtype: torch.dtype, count: int = 1) -> int:
    s = ctypes.c_size_t()
    L.call("gdb_muon_ws_bytes", count, m, n, dtype_code(dtype), ctypes.byref(s))
    return s.value


def muon_step(p: torch.Tensor, g: torch.Tensor, buf: torch.Tensor, lr: float, momentum: float, nesterov: bool,
              wd: float, scale: float, coeffs, dtype: torch.dtype, ws: torch.Tensor, p_bf16=None,
              norm_scale: float = 1.0, eps: float = 1e-7) -> None:
    """One Muon step on a matrix [m, n] or a stack [count, m, n] (float32)."""
    count, m, n = _stack(p)
    arr, steps = _coeffs(coeffs)
    L.call("gdb_muon_step", count, m, n, dtype_code(dtype), _p(p), _opt(p_bf16), _p(g), _p(buf), lr, momentum,
           int(nesterov), wd, scale, arr, steps, norm_scale, eps, _p(ws), ws.numel() * ws.element_size(),
           _stream(p))


def adamw_step(p: torch.Tensor, g: torch.Tensor, m: torch.Tensor, v: torch.Tensor, t: int, lr: float,
               beta1: float, beta2: float, eps: float, wd: float, p_bf16=None) -> None:
    L.call("gdb_adamw_step", p.numel(), _p(p), _opt(p_bf16), _p(g), _p(m), _p(v), t, lr, beta1, beta2, eps, wd,
           _stream(p))


def cross_entropy(z: torch.Tensor, targets: torch.Tensor, row_loss: torch.Tensor, loss: torch.Tensor) -> None:
    N, V = z.shape
    if targets.numel() != N or row_loss.numel() != N or loss.numel() < 1:
        raise ValueError(f"cross_entropy: {N} rows of logits need {N} targets and {N} row losses "
                         f"(got {targets.numel()} and {row_loss.numel()})")
    L.call("gdb_cross_entropy", N, V, dtype_code(z.dtype), _p(z), _p(targets), _p(row_loss), _p(loss),
           _stream(z))


def mix_fwd(x: torch.Tensor, x0: torch.Tensor, lam: torch.Tensor, y: torch.Tensor) -> None:
    N, C = x.shape
    L.call("gdb_mix_fwd", N, C, dtype_code(x.dtype), _p(x), _p(x0), _p(lam), _p(y), _stream(x))


def mix_bwd(dy: torch.Tensor, x: torch.Tensor, x0: torch.Tensor, lam: torch.Tensor, dx: torch.Tensor,
            dx0: torch.Tensor, dlam: torch.Tensor, ws: torch.Tensor, accumulate_dx0: bool = False,
            accumulate: bool = False) -> None:
    N, C = dy.shape
    L.call("gdb_mix_bwd", N, C, dtype_code(dy.dtype), _p(dy), _p(x), _p(x0), _p(lam), _p(dx), _p(dx0),
           int(accumulate_dx0), _p(dlam), int(accumulate), _p(ws), _stream(dy))


def ve_fwd(Hkv: int, D: int, qkv: torch.Tensor, voff: int, xn: torch.Tensor, ids: torch.Tensor, ve: torch.Tensor,
           wg: torch.Tensor, s_save: torch.Tensor) -> None:
    N, ldq = qkv.shape
    L.call("gdb_ve_fwd", N, Hkv, D, dtype_code(qkv.dtype), _p(qkv), ldq, voff, _p(xn), xn.shape[1], _p(ids),
           _p(ve), ve.shape[0], _p(wg), wg.shape[1], _p(s_save), _stream(qkv))


def ve_bwd_ws_bytes(N: int, Hkv: int, nc: int, deterministic: bool) -> int:
    n = ctypes.c_size_t()
    L.call("gdb_ve_bwd_ws_bytes", N, Hkv, nc, int(deterministic), ctypes.byref(n))
    return n.value


def ve_bwd(Hkv: int, D: int, dqkv: torch.Tensor, voff: int, ids: torch.Tensor, ve: torch.Tensor,
           s_save: torch.Tensor, xn: torch.Tensor, dxn: torch.Tensor, wg: torch.Tensor, dve: torch.Tensor,
           dwg: torch.Tensor, ws: torch.Tensor, accumulate: bool = False, deterministic: bool = False) -> None:
    N, ldq = dqkv.shape
    L.call("gdb_ve_bwd", N, Hkv, D, dtype_code(dqkv.dtype), _p(dqkv), ldq, voff, _p(ids), _p(ve), ve.shape[0],
           _p(s_save), _p(xn), _p(dxn), xn.shape[1], _p(wg), wg.shape[1], _p(dve), _p(dwg), int(accumulate),
           int(deterministic), _p(ws), _stream(dqkv))


def normuon_ws_bytes(m: int, n: int, dtype: torch.dtype, count: int = 1) -> int:
    b = ctypes.c_size_t()
    L.call("gdb_normuon_ws_bytes", count, m, n, dtype_code(dtype), ctypes.byref(b))
    return b.value


def normuon_step(p: torch.Tensor, g: torch.Tensor, buf: torch.Tensor, v: torch.Tensor, lr: float, momentum: float,
                 nesterov: bool, wd: float, scale: float, beta2: float, coeffs, dtype: torch.dtype,
                 ws: torch.Tensor, p_bf16: torch.Tensor = None, norm_scale: float = 1.0, eps: float = 1e-7) -> None:
    """p, g, buf float32 [count, m, n] (or [m, n]); v float32 [count, m] (or [m]): the per-neuron state."""
    count, m, n = _stack(p)
    c, steps = _coeffs(coeffs)
    L.call("gdb_normuon_step", count, m, n, dtype_code(dtype), _p(p), None if p_bf16 is None else _p(p_bf16), _p(g),
           _p(buf), _p(v), lr, momentum, int(nesterov), wd, scale, beta2, c, steps, norm_scale, eps, _p(ws),
           ws.numel(), _stream(p))
