"""Helpers of the GPU parity tests (imported by test_gpu_*.py only)."""
import contextlib

import numpy as np
import torch

from seeded_inputs import to_dtype

# max relative error bars: ||gpu - oracle||_inf / ||oracle||_inf per tensor
TOL = {"f32": 1e-4, "bf16": 2e-2}
TDT = {"f32": torch.float32, "bf16": torch.bfloat16}
DEV = "cuda:0"


def rounded(a, dt: str) -> np.ndarray:
    """float32 values representable in dt (what both sides consume)."""
    return to_dtype(np.asarray(a, dtype=np.float32), dt)


def dev(a, dt: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(rounded(a, dt))).to(TDT[dt]).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(gpu, ref) -> float:
    g = host(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), "non-finite values in GPU output"
    den = float(np.max(np.abs(r))) if r.size else 0.0
    return float(np.max(np.abs(g - r))) / den if den > 0 else float(np.max(np.abs(g)))


def assert_close(gpu, ref, dt: str, what: str = "", tol: float = None):
    e = rel_err(gpu, ref)
    bar = TOL[dt] if tol is None else tol
    assert e <= bar, f"{what}: max rel err {e:.3e} > {bar:.1e}"
    return e


def sum_close(gpu, ref, sum_abs, dt: str, what: str = "", tol: float = None):
    """A gradient that is a sum over tokens with cancellation (the value
    embedding gate's): the plain relative bar, or in bf16 the forward error
    bound of each element's sum, |gpu - ref| <= TOL * sum|terms| with the
    oracle's sum of the terms' magnitudes.  Returns the smaller normalised error."""
    e = rel_err(gpu, ref)
    bar = TOL[dt] if tol is None else tol
    if e <= bar:
        return e
    g = host(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, dtype=np.float64)
    eb = float(np.max(np.abs(g - np.asarray(ref)) / np.maximum(np.asarray(sum_abs, dtype=np.float64), 1e-300)))
    assert dt == "bf16" and eb <= TOL[dt], f"{what}: max rel err {e:.3e} > {bar:.1e} and err/sum|terms| {eb:.3e}"
    return eb


def empty(shape, dt, fill=None):
    t = torch.empty(shape, dtype=TDT[dt] if isinstance(dt, str) else dt, device=DEV)
    if fill is not None:
        t.fill_(fill)
    return t


def fp8_bars(pairs: dict, dt: str) -> dict:
    """Bars for tensors computed through fp8 products (the largest model's MLP).
    A code is a discrete decision: where the quantiser inputs of the two sides
    differ by a rounding, some codes differ by one e4m3 step, so the results
    differ by far more than that rounding.  Both sides are fp8 evaluations of
    the same exact quantity, and each lies within the method's own
    quantisation distance q of the exact value, so (triangle inequality, the
    GPU's quantisation moving its result about as far as the oracle's does)
    |gpu - oracle| <= 2q.  q is measured on the oracle alone: its fp8 result
    against its result with the quantiser off.  pairs: name -> (oracle output
    with fp8, oracle output without); bar = max(dtype bar, 2q)."""
    bars = {}
    for k, (ref, exact) in pairs.items():
        ref = np.asarray(ref, dtype=np.float64)
        den = float(np.max(np.abs(ref))) or 1.0
        q = float(np.max(np.abs(np.asarray(exact, dtype=np.float64) - ref))) / den
        bars[k] = max(TOL[dt], 2.0 * q)
    return bars
