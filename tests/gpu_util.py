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
    """Bars for outputs computed through fp8 products.  A code is a discrete
    decision, so two correct implementations whose quantiser inputs differ by
    one rounding differ by far more than that rounding: each tensor's bar is
    twice the oracle's own spread under such a difference (never below the
    dtype's plain bar).  pairs: name -> (oracle output, list of the oracle's
    outputs with its quantiser inputs changed as `fp8_alternative` describes);
    the spread is the largest over that list."""
    bars = {}
    for k, (ref, alts) in pairs.items():
        ref = np.asarray(ref, dtype=np.float64)
        den = float(np.max(np.abs(ref))) or 1.0
        spread = max(float(np.max(np.abs(np.asarray(a) - ref))) for a in alts) / den
        bars[k] = max(TOL[dt], 2.0 * spread)
    return bars


def fp8_alternatives(dt: str):
    """The changes of the oracle's quantiser inputs that `fp8_bars` samples:
    one for bf16 (a different rounding), three random ones for f32."""
    return [0] if dt == "bf16" else [0, 1, 2]


@contextlib.contextmanager
def fp8_alternative(dt: str, seed: int = 0):
    """The oracle with its quantiser inputs moved by about the rounding error
    the GPU pipeline carries into them.  bf16: the quantised tensors are not
    rounded to bfloat16 (float32 inputs instead).  f32: each input is scaled
    by 1 +- 4e-6 (random signs), the size of the float32 pipeline's own
    deviation from the oracle (an fp32 GEMM accumulating K ~ 10^3 terms is off
    by ~sqrt(K) * 2^-24 of its terms' magnitude, several 1e-6 of a small
    output).  Yields the dtype to give the oracle's cfg."""
    if dt == "bf16":
        yield "f32"
        return
    from oracle import reference as R
    orig = R.fp8_quant_dequant
    rng = np.random.default_rng(seed)

    def moved(x, storage=None):
        x = np.asarray(x, dtype=np.float64)
        return orig(x * (1.0 + 4e-6 * rng.choice([-1.0, 1.0], size=x.shape)), storage)

    R.fp8_quant_dequant = moved
    try:
        yield dt
    finally:
        R.fp8_quant_dequant = orig
