"""Write tests/golden/depth_bars.json: the parity bounds of the full-depth
stack tests, computed from the oracle alone before any GPU comparison.

A bf16 model stores its residual streams (x between blocks, dx between blocks)
as bf16 values (explicit dtypes, "Comment Entraîner Votre Propre ChatGPT Pour
50€ ?", section "3. Gestion de la précision"), and the rounding of those
streams compounds over 24-26 blocks.  For every checked tensor t this script
measures q_t = ||oracle(bf16 streams) - oracle(exact)||_inf / ||oracle(exact)||_inf
on the tests' seeded inputs.  An evaluation with bf16 streams lies about q_t
from the exact result and the GPU's also carries each block's own rounding
(the dtype bar b = 2e-2), so the tests hold |gpu - oracle| / |oracle| to
b + 2 q_t.

Run from the repository root:  python tests/golden/make_depth_bars.py
(calls only oracle/ and the seeded input generators; about 10 minutes on
8 cores with OMP_NUM_THREADS=4, two oracle runs at a time).
"""
import json
import os
import sys
from concurrent.futures import ProcessPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

TOL_BF16 = 2e-2
# the full-depth workloads of tests/test_gpu_block.py (name -> overrides)
CASES = {
    "d24_full_depth": ("d24", dict(B=1, T=256, windows=(-1, 128) * 12)),
    "d26_full_depth_extras": ("d26", dict(B=1, T=128, vocab=512, windows=(-1,) * 26, mlp_fp8=False)),
}


def case_workload(name):
    from seeded_inputs import workload
    base, over = CASES[name]
    return workload(base).with_(**over)


def describe(w) -> dict:
    return {"workload": w.name, "n_layer": w.n_layer, "B": w.B, "T": w.T, "C": w.C, "vocab": w.vocab,
            "windows": list(w.windows), "extras": bool(w.extras), "mlp_fp8": bool(w.mlp_fp8), "dtype": w.dtype}


def flat_grads(w, loss, g) -> dict:
    """The tensors the stack test compares, by the test's keys."""
    out = {"loss": loss, "wte": g["wte"], "w_lm": g["w_lm"]}
    for l, gl in enumerate(g["layers"]):
        for k, v in gl.items():
            if k not in ("sum_abs", "resid_lambda", "x0_lambda"):
                out[f"{l}.{k}"] = v
    if w.extras:
        out["smear_gate"] = g["smear_gate"]
    return out


def run(args):
    name, stream = args
    import numpy as np
    import oracle.reference as O
    from seeded_inputs import draw_all, to_dtype
    w = case_workload(name)
    d = draw_all(w)
    rd = lambda v: to_dtype(np.asarray(v, dtype=np.float32), w.dtype)
    glob = {k: rd(v) for k, v in d["globals"].items()}
    layers = [{k: rd(v) for k, v in p.items()} for p in d["layers"]]
    loss, g, _ = O.stack_forward_backward(w, d["ids"], glob, layers, stream_dtype=stream)
    return name, stream, {k: np.asarray(v, dtype=np.float64) for k, v in flat_grads(w, loss, g).items()}


def main():
    import numpy as np
    jobs = [(n, s) for n in CASES for s in (None, "bf16")]
    with ProcessPoolExecutor(max_workers=2) as ex:  # two full-depth oracles fit in 64 GiB
        res = {(n, s): r for n, s, r in ex.map(run, jobs)}
    out = {"tol": TOL_BF16, "rule": "bar = tol + 2 q, q = ||oracle(bf16 streams) - oracle||_inf / ||oracle||_inf",
           "cases": {}}
    for n in CASES:
        ex_, st = res[(n, None)], res[(n, "bf16")]
        q = {}
        for k, v in ex_.items():
            den = float(np.max(np.abs(v))) or 1.0
            q[k] = float(np.max(np.abs(st[k] - v))) / den
        out["cases"][n] = {"config": describe(case_workload(n)), "q": q,
                           "bars": {k: TOL_BF16 + 2.0 * v for k, v in q.items()}}
        worst = sorted(q.items(), key=lambda kv: -kv[1])[:3]
        print(n, "largest q:", [(k, round(v, 5)) for k, v in worst], flush=True)
    with open(os.path.join(HERE, "depth_bars.json"), "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
