"""The fp8 quantiser takes x / s as RN(q0 + e*y) with y = RN(1/s),
q0 = RN(x*y) and e = x - q0*s (exact, one FMA): Markstein's theorem says this
is the correctly rounded quotient for a normal s.  Checked here in float32 on
the host for every bf16 x over scales across the exponent range and for
random fp32 x; float64 emulates each FMA exactly, and every case the float64
emulation cannot decide (a result on a float32 midpoint) or where it
disagrees is settled with exact rationals.  Subnormal quotients are left out:
their e4m3 code is 0 whichever way they round."""
from fractions import Fraction

import numpy as np


def _rn32(fr: Fraction) -> np.float32:
    g = np.float32(float(fr))
    cands = [np.nextafter(g, np.float32(-np.inf)), g, np.nextafter(g, np.float32(np.inf))]
    return min(cands, key=lambda c: (abs(Fraction(float(c)) - fr), int(np.float32(c).view(np.uint32)) & 1))


def _midpoint(x64: np.ndarray) -> np.ndarray:
    f = x64.astype(np.float32)
    lo = np.where(f.astype(np.float64) <= x64, f, np.nextafter(f, np.float32(-np.inf)))
    hi = np.nextafter(lo, np.float32(np.inf))
    return (lo.astype(np.float64) + hi.astype(np.float64)) / 2 == x64


def _check(v: np.ndarray, s: np.float32) -> int:
    y = np.float32(1) / s
    q0 = (v * y).astype(np.float32)
    e = (v.astype(np.float64) - q0.astype(np.float64) * np.float64(s)).astype(np.float32)
    t = e.astype(np.float64) * np.float64(y) + q0.astype(np.float64)
    got = t.astype(np.float32)
    x64 = v.astype(np.float64) / np.float64(s)
    want = x64.astype(np.float32)
    look = ((got != want) | _midpoint(x64) | _midpoint(t)) & (np.abs(want) >= 2.0 ** -126) & np.isfinite(want)
    bad = 0
    for i in np.nonzero(look)[0]:
        exact = Fraction(float(v[i])) / Fraction(float(s))
        rem = Fraction(float(v[i])) - Fraction(float(q0[i])) * Fraction(float(s))
        if _rn32(rem * Fraction(float(y)) + Fraction(float(q0[i]))) != _rn32(exact):
            bad += 1
    return bad


def test_reciprocal_quotient_is_correctly_rounded():
    rng = np.random.default_rng(0)
    bf16 = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    bf16 = bf16[np.isfinite(bf16)]
    scales = [np.float32(rng.uniform(1, 2) * 2.0 ** e) for e in range(-110, 100, 7)]
    scales += [np.float32(a) / np.float32(448) for a in (448.0, 1.0, 24576.0, 2.0 ** -100, 3.0, 0.1)]
    bad = 0
    with np.errstate(all="ignore"):
        for s in scales:
            bad += _check(bf16, s)
        for k in range(4):
            s = np.float32(rng.uniform(1, 2) * 2.0 ** int(rng.integers(-60, 40)))
            v = (rng.standard_normal(500_000) * 2.0 ** int(rng.integers(-40, 40))).astype(np.float32)
            bad += _check(v, s)
    assert bad == 0
