"""ctypes binding of libgdb.so (the C ABI declared in include/gdb.h).

Argument marshalling only: torch tensors are turned into device pointers and
the current HIP stream; every step of the computation runs in the library's
HIP kernels.  Loading fails loudly if the library has not been built; there is
no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
# GDB_LIB selects another build of the same library (for example the
# host-sanitizer build made by `python -m gpt_decoder_block_amd.build --sanitize`)
LIB_PATH = os.environ.get("GDB_LIB") or os.path.join(HERE, "libgdb.so")

# the GDB_ABI_VERSION this binding's structures and signatures follow
ABI_VERSION = 7

GDB_OK, GDB_EINVAL, GDB_EUNSUPPORTED, GDB_EHIP, GDB_EWORKSPACE, GDB_ENONFINITE = 0, -1, -2, -3, -4, -5
GDB_F32, GDB_BF16 = 0, 1

c_void_p, c_int32, c_float, c_size_t = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
c_int64 = ctypes.c_int64


class BlockCfg(ctypes.Structure):
    _fields_ = [("B", c_int32), ("T", c_int32), ("C", c_int32),
                ("n_head", c_int32), ("n_kv_head", c_int32), ("head_dim", c_int32),
                ("mlp_hidden", c_int32), ("window", c_int32), ("dtype", c_int32),
                ("mlp_fp8", c_int32), ("accumulate_wgrad", c_int32), ("deterministic", c_int32),
                ("eps", c_float)]


class BlockWeights(ctypes.Structure):
    _fields_ = [("w_qkv", c_void_p), ("w_o", c_void_p), ("w_fc", c_void_p), ("w_proj", c_void_p)]


class BlockWgrads(ctypes.Structure):
    _fields_ = [("dw_qkv", c_void_p), ("dw_o", c_void_p), ("dw_fc", c_void_p), ("dw_proj", c_void_p)]


class BlockExtras(ctypes.Structure):
    _fields_ = [("lambdas", c_void_p), ("x0", c_void_p), ("x_in", c_void_p), ("ids", c_void_p),
                ("ve", c_void_p), ("ve_gate", c_void_p), ("ve_vocab", c_int32), ("ve_gate_channels", c_int32)]


class BlockExtrasGrads(ctypes.Structure):
    _fields_ = [("dlambdas", c_void_p), ("dx0", c_void_p), ("dve", c_void_p), ("dve_gate", c_void_p),
                ("accumulate_dx0", c_int32)]


GDB_EXTRAS_WS_BYTES = 1 << 20


class GdbError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status
        self.msg = msg


_lib: Optional[ctypes.CDLL] = None

# name -> (restype, argtypes), in the order of include/gdb.h
SIGNATURES = {
    "gdb_abi_version": (c_int32, []),
    "gdb_last_error": (ctypes.c_char_p, []),
    "gdb_block_sizes": (c_int32, [ctypes.POINTER(BlockCfg), ctypes.POINTER(c_size_t),
                                  ctypes.POINTER(c_size_t), ctypes.POINTER(c_size_t)]),
    "gdb_rope_table_host": (c_int32, [c_int32, c_int32, ctypes.c_double, c_void_p]),
    "gdb_embed_fwd": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
    "gdb_embed_bwd_ws_bytes": (c_int32, [c_int32, c_int32, ctypes.POINTER(c_size_t)]),
    "gdb_embed_bwd": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_int32,
                                c_int32, c_void_p, c_void_p]),
    "gdb_block_fwd": (c_int32, [ctypes.POINTER(BlockCfg), ctypes.POINTER(BlockWeights),
                                ctypes.POINTER(BlockExtras), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                c_void_p]),
    "gdb_block_bwd": (c_int32, [ctypes.POINTER(BlockCfg), ctypes.POINTER(BlockWeights),
                                ctypes.POINTER(BlockExtras), c_void_p, c_void_p, c_void_p, c_void_p,
                                ctypes.POINTER(BlockWgrads), ctypes.POINTER(BlockExtrasGrads), c_void_p,
                                c_void_p]),
    "gdb_lm_head_ce_sizes": (c_int32, [c_int32, c_int32, c_int32, c_int32, ctypes.POINTER(c_size_t)]),
    "gdb_lm_head_ce_fwd_bwd": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_float, c_void_p, c_void_p,
                                         c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p,
                                         c_void_p]),
    "gdb_smear_fwd": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                c_void_p, c_void_p, c_void_p]),
    "gdb_smear_bwd": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p,
                                c_void_p]),
    "gdb_backout_fwd": (c_int32, [c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "gdb_backout_bwd": (c_int32, [c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_int32, c_void_p, c_void_p]),
    "gdb_mix_fwd": (c_int32, [c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "gdb_mix_bwd": (c_int32, [c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                              c_int32, c_void_p, c_int32, c_void_p, c_void_p]),
    "gdb_ve_fwd": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_void_p, c_int32, c_int32, c_void_p, c_int32,
                             c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_void_p]),
    "gdb_ve_bwd_ws_bytes": (c_int32, [c_int32, c_int32, c_int32, c_int32, ctypes.POINTER(c_size_t)]),
    "gdb_ve_bwd": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                             c_int32, c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_void_p,
                             c_int32, c_int32, c_void_p, c_void_p]),
    "gdb_stream_copy": (c_int32, [c_size_t, c_void_p, c_void_p, c_void_p]),
    "gdb_rmsnorm_fwd": (c_int32, [c_int32, c_int32, c_int32, c_float, c_void_p, c_void_p, c_void_p, c_void_p]),
    "gdb_rmsnorm_bwd": (c_int32, [c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_void_p]),
    "gdb_gemm_ws_bytes": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_int32, ctypes.POINTER(c_size_t)]),
    "gdb_gemm": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_void_p, c_int32, c_int32, c_void_p, c_int32,
                           c_int32, c_int32, c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_int32, c_void_p,
                           c_void_p]),
    "gdb_fp8_quantize": (c_int32, [c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                   c_void_p]),
    "gdb_gemm_fp8_ws_bytes": (c_int32, [c_int32, c_int32, c_int32, c_int32, ctypes.POINTER(c_size_t)]),
    "gdb_gemm_fp8": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_void_p, c_int32, c_void_p, c_void_p, c_int32,
                               c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_int32, c_void_p,
                               c_void_p]),
    "gdb_qk_norm_rope_fwd": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_float, c_void_p,
                                       c_void_p, c_void_p, c_void_p, c_void_p]),
    "gdb_qk_norm_rope_bwd": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p,
                                       c_void_p, c_void_p, c_void_p]),
    "gdb_attention_fwd": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                    c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_void_p]),
    "gdb_attention_bwd": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p,
                                    c_int32, c_void_p, c_int32, c_void_p, c_void_p, c_int32, c_void_p, c_int32,
                                    c_void_p, c_void_p]),
    "gdb_cross_entropy": (c_int32, [c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_void_p]),
    "gdb_newton_schulz_ws_bytes": (c_int32, [c_int32, c_int32, c_int32, c_int32, ctypes.POINTER(c_size_t)]),
    "gdb_newton_schulz": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_int32,
                                    c_float, c_float, c_void_p, c_size_t, c_void_p]),
    "gdb_muon_ws_bytes": (c_int32, [c_int32, c_int32, c_int32, c_int32, ctypes.POINTER(c_size_t)]),
    "gdb_muon_step": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_float,
                                c_float, c_int32, c_float, c_float, c_void_p, c_int32, c_float, c_float, c_void_p,
                                c_size_t, c_void_p]),
    "gdb_normuon_ws_bytes": (c_int32, [c_int32, c_int32, c_int32, c_int32, ctypes.POINTER(c_size_t)]),
    "gdb_normuon_step": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_void_p, c_float, c_float, c_int32, c_float, c_float, c_float, c_void_p, c_int32,
                                   c_float, c_float, c_void_p, c_size_t, c_void_p]),
    "gdb_adamw_step": (c_int32, [c_int64, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_float, c_float,
                                 c_float, c_float, c_float, c_void_p]),
    "gdb_attention_decode_ws_bytes": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                                ctypes.POINTER(c_size_t)]),
    "gdb_attention_decode": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p, c_int32,
                                       c_void_p, c_void_p, c_int32, c_int64, c_void_p, c_int32, c_void_p, c_int32,
                                       c_void_p, c_void_p, c_size_t, c_void_p]),
    "gdb_attention_decode_noalloc": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p,
                                               c_int32, c_void_p, c_void_p, c_int32, c_int64, c_void_p, c_int32,
                                               c_void_p, c_int32, c_void_p, c_void_p]),
}


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m gpt_decoder_block_amd.build` "
                               "(the HIP library is required; there is no CPU fallback)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        if l.gdb_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {l.gdb_abi_version()}, the binding expects "
                               f"{ABI_VERSION}: rebuild it")
        _lib = l
    return _lib


def check(fn: str, status: int) -> None:
    if status != GDB_OK:
        raise GdbError(fn, status, lib().gdb_last_error().decode())


def call(fn: str, *args) -> None:
    check(fn, getattr(lib(), fn)(*args))
