"""Helpers of the GPU parity tests (imported by test_gpu_*.py only)."""
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


def empty(shape, dt, fill=None):
    t = torch.empty(shape, dtype=TDT[dt] if isinstance(dt, str) else dt, device=DEV)
    if fill is not None:
        t.fill_(fill)
    return t
