#!/usr/bin/env python3
"""Training-step throughput of the decoder stack on one MI355X.

One step = embed_fwd -> L x block_fwd -> lm_head_ce_fwd_bwd -> L x block_bwd
-> embed_bwd on seeded synthetic inputs already resident in HBM (the optimizer
step is not part of the path).  Prints ONE JSON line with tokens/s, TFLOP/s
and the fraction of the bf16 MFMA peak, a roofline entry for the dominant
kernel (timed on its own with HIP events on the stream it is launched on),
per-kernel figures, and the CPU oracle timed on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--workload d24] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "train tokens/s on 1 MI355X, d24 stack fwd+bwd; % of bf16 MFMA peak"
PEAK_BF16 = 2.5e15       # dense bf16 MFMA, FLOP/s
PEAK_FP8 = 5.0e15        # dense fp8 MFMA, FLOP/s
PEAK_HBM = 8.0e12        # HBM3E, bytes/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="d24")
    ap.add_argument("--batch", type=int, default=None, help="override B (default: the workload's)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--kernel-reps", type=int, default=10)
    ap.add_argument("--counter-run", action="store_true",
                    help="only launch each hot kernel class 3 times at the workload's shapes, then a 1 GiB device "
                         "copy 3 times, for hardware-counter collection (rocprofv3 --pmc)")
    ap.add_argument("--counter-summary", nargs="+", metavar="DIR",
                    help="summarise the rocprofv3 counter CSV files under these directories (no GPU needed)")
    return ap.parse_args()


def counter_run(w):
    """Launch sequence for rocprofv3 --pmc passes: each hot kernel class of
    the step at the workload's shapes, 3 launches each, then a plain copy of
    known size (its FETCH_SIZE / WRITE_SIZE readings calibrate the counters
    to bytes).  Prints the launch list as JSON."""
    import torch
    from gpt_decoder_block_amd import ops
    dev, dt = "cuda:0", torch.bfloat16 if w.dtype == "bf16" else torch.float32
    N, C, F, V = w.B * w.T, w.C, w.mlp_hidden, w.vocab
    H, Hkv, D = w.n_head, w.n_kv_head, w.head_dim
    W3 = (H + 2 * Hkv) * D
    g = torch.Generator(device=dev).manual_seed(1)
    rnd = lambda *shape, sc=1.0: (torch.randn(*shape, generator=g, device=dev) * sc).to(dt)
    launched = []
    # GEMMs: MLP up-projection with relu^2 (stores h), and the MLP down-projection's weight gradient
    A, B = rnd(N, C), rnd(F, C, sc=0.02)
    Hh = torch.empty(N, F, dtype=dt, device=dev)
    for _ in range(3):
        ops.gemm(N, F, C, A, True, C, B, True, C, ops.EPI_SQR, Hh, F)
    launched.append({"kernel": "gemm mlp_up relu2", "shape": [N, F, C], "flops": 2.0 * N * F * C})
    dW = torch.empty(C, F, dtype=torch.float32, device=dev)
    ws = torch.empty(max(ops.gemm_ws_bytes(dt, C, F, N, ops.EPI_F32), 16), dtype=torch.uint8, device=dev)
    for _ in range(3):
        ops.gemm(C, F, N, A, False, C, Hh, False, F, ops.EPI_F32, dW, F, ws=ws)
    launched.append({"kernel": "gemm wgrad mlp_down", "shape": [C, F, N], "flops": 2.0 * N * F * C})
    del Hh, dW, ws, B
    # attention forward / backward at the workload's windows
    from gpt_decoder_block_amd.workmodel import attn_pairs
    qkv = rnd(N, W3)
    qk = qkv[:, :(H + Hkv) * D].float().view(N, H + Hkv, D)
    qkv[:, :(H + Hkv) * D] = (qk * torch.rsqrt(qk.pow(2).mean(-1, keepdim=True))).view(N, -1).to(dt)
    del qk
    o, do = torch.empty(N, H * D, dtype=dt, device=dev), rnd(N, H * D)
    lse, delta = (torch.empty(w.B, H, w.T, dtype=torch.float32, device=dev) for _ in range(2))
    dqkv = torch.empty(N, W3, dtype=dt, device=dev)
    for win in sorted(set(w.windows)):
        pairs = attn_pairs(w.T, win) * w.B * H
        for _ in range(3):
            ops.attention_fwd(w.B, w.T, H, Hkv, D, win, qkv, W3, o, H * D, lse, qk_normed=True)
        for _ in range(3):
            ops.attention_bwd(w.B, w.T, H, Hkv, D, win, qkv, W3, o, H * D, lse, do, H * D, dqkv, W3, delta)
        launched.append({"kernel": f"attention window {win}", "pairs": pairs, "fwd_flops": 4.0 * D * pairs,
                         "bwd_flops": 8.0 * D * pairs})
    del qkv, o, do, dqkv
    # bandwidth kernels: RMSNorm forward / backward, cross-entropy over the vocabulary
    x, xn = rnd(N, C), torch.empty(N, C, dtype=dt, device=dev)
    r = torch.empty(N, dtype=torch.float32, device=dev)
    for _ in range(3):
        ops.rmsnorm_fwd(x, xn, r, w.eps)
    dres, dx = rnd(N, C), torch.empty(N, C, dtype=dt, device=dev)
    for _ in range(3):
        ops.rmsnorm_bwd(x, xn, r, dres, dx)
    launched.append({"kernel": "rmsnorm", "fwd_bytes": 2.0 * N * C * s_el(dt) + 4 * N,
                     "bwd_bytes": 4.0 * N * C * s_el(dt) + 4 * N})
    del x, xn, dres, dx
    z = rnd(N, V)
    tg = torch.randint(0, V, (N,), device=dev, dtype=torch.int32)
    rl, ls = torch.empty(N, dtype=torch.float32, device=dev), torch.empty(1, dtype=torch.float32, device=dev)
    for _ in range(3):
        ops.cross_entropy(z, tg, rl, ls)
    launched.append({"kernel": "cross entropy", "bytes": N * V * 2.0 * s_el(dt) + 8 * N})
    del z
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)   # 1 GiB
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    launched.append({"kernel": "copy", "bytes_each_way": src.numel() * 4})
    print(json.dumps({"counter_run": True, "workload": w.name, "launched": launched}))


def _short(name: str) -> str:
    """Readable kernel symbol: demangled (c++filt, when the tracer kept the
    mangled name), without namespaces' anonymous parts and the argument list."""
    if name.startswith("_Z"):
        import subprocess
        try:
            # GNU c++filt does not know the DF16b code of __bf16; spell it as a vendor type
            dm = name.replace("DF16b", "u6__bf16")
            name = subprocess.run(["c++filt", dm], capture_output=True, text=True, timeout=10).stdout.strip() or name
        except (OSError, subprocess.SubprocessError):
            pass
    name = name.replace("void ", "").replace("(anonymous namespace)::", "")
    depth = 0
    for i, ch in enumerate(name):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            return name[:i]
    return name


def counter_summary(dirs):
    """Per-kernel averages of every counter found in the rocprofv3 CSV files
    under `dirs` (one directory per --pmc pass), plus the derived figures:
    MFMA busy (% of the SIMDs' cycles), VALU busy, the effective clock
    (GUI-active cycles of the busiest XCD / duration), HBM bytes from
    FETCH_SIZE / WRITE_SIZE calibrated on the 1 GiB copy.  Markdown on stdout."""
    import csv
    import glob
    from collections import defaultdict
    vals = defaultdict(lambda: defaultdict(list))   # kernel -> counter -> per-dispatch values
    durs = defaultdict(dict)                         # kernel -> dispatch -> ns
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            per = defaultdict(lambda: defaultdict(float))
            with open(f) as fh:
                for row in csv.DictReader(fh):
                    k = _short(row["Kernel_Name"])
                    key = (k, f, row["Dispatch_Id"])
                    per[key][row["Counter_Name"]] += float(row["Counter_Value"])
                    if row.get("End_Timestamp") and row.get("Start_Timestamp"):
                        durs[k][(f, row["Dispatch_Id"])] = float(row["End_Timestamp"]) - float(row["Start_Timestamp"])
            for (k, _, _), cs in per.items():
                for c, v in cs.items():
                    vals[k][c].append(v)
    avg = {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in vals.items()}
    copy = next((k for k in avg if "copyBuffer" in k), None)
    fmt = lambda v, p=1: "" if v is None else f"{v:.{p}f}"
    gib = float(1 << 30)
    rf = avg[copy]["FETCH_SIZE"] * 1024 / gib if copy and "FETCH_SIZE" in avg[copy] else None
    wf = avg[copy]["WRITE_SIZE"] * 1024 / gib if copy and "WRITE_SIZE" in avg[copy] else None
    cols = ["kernel", "dispatches", "avg us", "MfmaUtil %", "VALUBusy %", "clock MHz", "VALU/MFMA", "LDS/MFMA",
            "LDS wait %", "LDS conflict %", "HBM read MB", "HBM write MB", "HBM GB/s"]
    print("| " + " | ".join(cols) + " |")
    print("|" + "---|" * len(cols))
    for k in sorted(avg, key=lambda k: -sum(durs[k].values()) / max(1, len(durs[k]))):
        a = avg[k]
        n = max(len(v) for v in vals[k].values())
        us = sum(durs[k].values()) / max(1, len(durs[k])) / 1e3
        clk = a["GRBM_GUI_ACTIVE"] / 8 / (us * 1e-6) / 1e6 if "GRBM_GUI_ACTIVE" in a and us > 0 else None
        ratio = lambda x, y: (a[x] / a[y]) if x in a and y in a and a[y] > 0 else None
        rd = a["FETCH_SIZE"] * 1024 / rf / 1e6 if rf and "FETCH_SIZE" in a else None
        wr = a["WRITE_SIZE"] * 1024 / wf / 1e6 if wf and "WRITE_SIZE" in a else None
        bw = ((rd or 0) + (wr or 0)) * 1e6 / (us * 1e-6) / 1e9 if (rd or wr) and us > 0 else None
        # share of the waves' cycles spent waiting on LDS; bank-conflict cycles per LDS-active cycle
        lw = ratio("SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES")
        lc = ratio("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE")
        print(f"| `{k[:90]}` | {n} | {us:.1f} | {fmt(a.get('MfmaUtil'))} | {fmt(a.get('VALUBusy'))} | {fmt(clk, 0)} | "
              f"{fmt(ratio('SQ_INSTS_VALU', 'SQ_INSTS_MFMA'), 2)} | {fmt(ratio('SQ_INSTS_LDS', 'SQ_INSTS_MFMA'), 2)} | "
              f"{fmt(None if lw is None else 100 * lw)} | {fmt(None if lc is None else 100 * lc)} | "
              f"{fmt(rd)} | {fmt(wr)} | {fmt(bw, 0)} |")
    print(f"\ncalibration on the 1 GiB copy: read factor {fmt(rf, 4) if rf else 'n/a'}, write factor "
          f"{fmt(wf, 4) if wf else 'n/a'} (counter KiB x 1024 / bytes moved)")


def s_el(dt) -> int:
    import torch
    return 2 if dt == torch.bfloat16 else 4


def ev_time(fn, reps, torch):
    """Average duration (s) of fn() over reps launches, HIP events on the current stream."""
    s = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    a.record(s)
    for _ in range(reps):
        fn()
    b.record(s)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / 1e3 / reps


def cold_time(fn, reps, torch, flush):
    """Average duration (s) of fn() launched right after overwriting a flush
    buffer larger than the 256 MB Infinity Cache, so its operands come from
    HBM (only the launch is timed)."""
    s = torch.cuda.current_stream()
    tot = 0.0
    for _ in range(reps):
        flush.fill_(1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        fn()
        b.record(s)
        torch.cuda.synchronize()
        tot += a.elapsed_time(b) / 1e3
    return tot / reps


def kernel_figures(w, st, reps, torch, ops):
    """Each hot kernel class timed alone at the workload's shapes."""
    dev, dt = st.device, st.dt
    N, C, F, V = st.N, w.C, w.mlp_hidden, w.vocab
    H, Hkv, D = w.n_head, w.n_kv_head, w.head_dim
    W3 = (H + 2 * Hkv) * D
    g = torch.Generator(device=dev).manual_seed(1)
    rnd = lambda *shape: torch.randn(*shape, generator=g, device=dev, dtype=torch.float32).to(dt)
    out = {}
    # MLP up-projection with fused ReLU^2 (the largest block GEMM; the block
    # stores h = relu(u)^2 only), on a real normalised residual stream (middle
    # layer) and that layer's W_fc
    lm = w.n_layer // 2
    A = torch.empty(N, C, dtype=dt, device=dev)
    ops.rmsnorm_fwd(st.xs[lm], A, torch.empty(N, dtype=torch.float32, device=dev), w.eps)
    B = st.layers[lm][2]
    Hh = torch.empty(N, F, dtype=dt, device=dev)
    t = ev_time(lambda: ops.gemm(N, F, C, A, True, C, B, True, C, ops.EPI_SQR, Hh, F), reps, torch)
    fl = 2.0 * N * F * C
    out["gemm_mlp_up_sqr"] = {"shape": [N, F, C], "ms": t * 1e3, "tflops": fl / t / 1e12,
                                "frac_bf16_peak": fl / t / PEAK_BF16, "flops": fl}
    if w.mlp_fp8:
        # the same product on e4m3 codes (as the fp8 block runs it), and the
        # quantiser of the activation (amax pass + codes row-major and transposed)
        Np = (N + 15) // 16 * 16
        am = torch.empty(2, dtype=torch.float32, device=dev)
        Aq, AqT = torch.empty(N, C, dtype=torch.uint8, device=dev), torch.empty(C, Np, dtype=torch.uint8, device=dev)
        Bq = torch.empty(F, C, dtype=torch.uint8, device=dev)
        ops.fp8_quantize(B, am[1:], Bq)
        tq = ev_time(lambda: ops.fp8_quantize(A, am[:1], Aq, AqT, Np), reps, torch)
        by = N * C * (2.0 * s_el(dt) + 2.0)   # amax read + quantiser read, two code writes
        out["fp8_quantize_act"] = {"shape": [N, C], "ms": tq * 1e3, "GBps": by / tq / 1e9,
                                   "frac_hbm_peak": by / tq / PEAK_HBM}
        t8 = ev_time(lambda: ops.gemm_fp8(N, F, C, Aq, C, am[:1], Bq, C, am[1:], ops.EPI_SQR, Hh, F),
                     reps, torch)
        out["gemm_fp8_mlp_up_sqr"] = {"shape": [N, F, C], "ms": t8 * 1e3, "tflops": fl / t8 / 1e12,
                                        "frac_fp8_peak": fl / t8 / PEAK_FP8, "flops": fl}
        del Aq, AqT, Bq
    # weight gradients (token contraction, fp32 out, split over K with a
    # fixed-order reduction): every shape one step launches, with its count
    # per step; both operands token-major as in the block
    Q, KV = H * D, Hkv * D
    W3 = Q + 2 * KV
    wshapes = [("mlp_down", C, F, w.n_layer), ("mlp_up", F, C, w.n_layer), ("attn_out", C, Q, w.n_layer),
               ("qkv", W3, C, w.n_layer), ("lm_head", V, C, 1)]
    if not w.mlp_fp8:
        src = torch.empty(N, max(F, V, W3), dtype=dt, device=dev).normal_()
        tot_t = tot_f = 0.0
        per = {}
        for name, M_, N_, cnt in wshapes:
            dW = torch.empty(M_, N_, dtype=torch.float32, device=dev)
            ws = torch.empty(max(ops.gemm_ws_bytes(dt, M_, N_, N, ops.EPI_F32), 16), dtype=torch.uint8, device=dev)
            a_op, b_op = src[:, :M_].contiguous(), src[:, :N_].contiguous()
            t = ev_time(lambda: ops.gemm(M_, N_, N, a_op, False, M_, b_op, False, N_, ops.EPI_F32, dW, N_, ws=ws),
                        reps, torch)
            f_ = 2.0 * M_ * N_ * N
            per[name] = {"shape": [M_, N_, N], "per_step": cnt, "ms": t * 1e3, "tflops": f_ / t / 1e12,
                         "frac_bf16_peak": f_ / t / PEAK_BF16}
            tot_t += cnt * t
            tot_f += cnt * f_
            del dW, ws, a_op, b_op
        del src
        out["gemm_wgrad"] = {"shapes": per, "step_ms": tot_t * 1e3, "tflops": tot_f / tot_t / 1e12,
                             "frac_bf16_peak": tot_f / tot_t / PEAK_BF16,
                             "launches_per_step": sum(c for *_, c in wshapes),
                             "avg_launch_ms": tot_t / sum(c for *_, c in wshapes) * 1e3,
                             "avg_flops_per_launch": tot_f / sum(c for *_, c in wshapes)}
    del Hh
    # attention forward / backward, full causal and windowed
    from gpt_decoder_block_amd.workmodel import attn_pairs
    qkv = rnd(N, W3)
    qk = qkv[:, :(H + Hkv) * D].float().view(N, H + Hkv, D)   # unit-RMS q, k heads (QK-norm output)
    qkv[:, :(H + Hkv) * D] = (qk * torch.rsqrt(qk.pow(2).mean(-1, keepdim=True))).view(N, -1).to(dt)
    del qk
    o = torch.empty(N, H * D, dtype=dt, device=dev)
    lse = torch.empty(w.B, H, w.T, dtype=torch.float32, device=dev)
    do = rnd(N, H * D)
    dqkv = torch.empty(N, W3, dtype=dt, device=dev)
    delta = torch.empty(w.B, H, w.T, dtype=torch.float32, device=dev)
    for win in sorted(set(w.windows)):
        pairs = attn_pairs(w.T, win) * w.B * H
        f_fwd, f_bwd = 4.0 * D * pairs, 8.0 * D * pairs
        tf = ev_time(lambda: ops.attention_fwd(w.B, w.T, H, Hkv, D, win, qkv, W3, o, H * D, lse, qk_normed=True),
                     reps, torch)
        tb = ev_time(lambda: ops.attention_bwd(w.B, w.T, H, Hkv, D, win, qkv, W3, o, H * D, lse, do, H * D,
                                               dqkv, W3, delta), reps, torch)
        key = "full" if win < 0 else f"window{win}"
        out[f"attn_fwd_{key}"] = {"ms": tf * 1e3, "tflops": f_fwd / tf / 1e12, "frac_bf16_peak": f_fwd / tf / PEAK_BF16}
        out[f"attn_bwd_{key}"] = {"ms": tb * 1e3, "tflops": f_bwd / tb / 1e12, "frac_bf16_peak": f_bwd / tb / PEAK_BF16}
    del qkv, o, do, dqkv
    # RMSNorm forward (bandwidth): read x, write xn, write r
    x, xn, r = rnd(N, C), torch.empty(N, C, dtype=dt, device=dev), torch.empty(N, dtype=torch.float32, device=dev)
    s = 2 if dt == torch.bfloat16 else 4
    t = ev_time(lambda: ops.rmsnorm_fwd(x, xn, r, w.eps), reps, torch)
    by = 2.0 * N * C * s + 4 * N
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
    tc = cold_time(lambda: ops.rmsnorm_fwd(x, xn, r, w.eps), 5, torch, flush)
    out["rmsnorm_fwd"] = {"ms": t * 1e3, "GBps": by / t / 1e9, "frac_hbm_peak": by / t / PEAK_HBM,
                          "cold_ms": tc * 1e3, "cold_frac_hbm_peak": by / tc / PEAK_HBM}
    dres = rnd(N, C)
    dx = torch.empty(N, C, dtype=dt, device=dev)
    t = ev_time(lambda: ops.rmsnorm_bwd(x, xn, r, dres, dx), reps, torch)
    by = 4.0 * N * C * s + 4 * N
    tc = cold_time(lambda: ops.rmsnorm_bwd(x, xn, r, dres, dx), 5, torch, flush)
    out["rmsnorm_bwd"] = {"ms": t * 1e3, "GBps": by / t / 1e9, "frac_hbm_peak": by / t / PEAK_HBM,
                          "cold_ms": tc * 1e3, "cold_frac_hbm_peak": by / tc / PEAK_HBM}
    del x, xn, dres, dx
    # the box's read+write reference: the library's streaming copy of 1 GiB,
    # warm (back to back) and cold (after the flush buffer is written)
    csrc, cdst = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0), torch.empty(1 << 28, device=dev)
    t = ev_time(lambda: ops.stream_copy(csrc, cdst), reps, torch)
    tc = cold_time(lambda: ops.stream_copy(csrc, cdst), 5, torch, flush)
    out["stream_copy_1gib"] = {"GBps": 2.0 * (1 << 30) / t / 1e9, "frac_hbm_peak": 2.0 * (1 << 30) / t / PEAK_HBM,
                               "cold_GBps": 2.0 * (1 << 30) / tc / 1e9,
                               "cold_frac_hbm_peak": 2.0 * (1 << 30) / tc / PEAK_HBM}
    del csrc, cdst
    # cross-entropy over the vocabulary (bandwidth): one read + one write of the logits
    z0 = rnd(N, V)
    z = torch.empty_like(z0)
    tg = torch.randint(0, V, (N,), device=dev, dtype=torch.int32)
    rl, ls = torch.empty(N, dtype=torch.float32, device=dev), torch.empty(1, dtype=torch.float32, device=dev)
    # restore the logits before each launch outside the timed launches: time copy+ce, subtract copy
    tc = ev_time(lambda: z.copy_(z0), reps, torch)
    tce = ev_time(lambda: (z.copy_(z0), ops.cross_entropy(z, tg, rl, ls)), reps, torch) - tc
    by = N * V * 2.0 * s + 8 * N
    out["cross_entropy"] = {"ms": tce * 1e3, "GBps": by / tce / 1e9, "frac_hbm_peak": by / tce / PEAK_HBM}
    del flush
    del z0, z
    # embedding-gradient scatter (B0) and value-embedding table gradient (E2),
    # with uniform ids and with Zipf(1.0) ids (many tokens on a few rows: a
    # stand-in for natural text's contention), float32 atomics and the
    # deterministic path (tokens sorted by id, each row summed in token order).
    # B0's bytes: dx0 read once plus a float32 read-modify-write per token row;
    # the overwrite's zero fill of the table is inside the timed call.
    from seeded_inputs import draw_ids_zipf
    ids_by = {"uniform": tg,
              "zipf1": torch.from_numpy(draw_ids_zipf(w).reshape(-1)[:N].astype(np.int32)).to(dev)}
    dx0 = rnd(N, C)
    dwte = torch.empty(V, C, dtype=torch.float32, device=dev)
    wse = torch.empty(max(ops.embed_bwd_ws_bytes(N, True), 16), dtype=torch.uint8, device=dev)
    by = N * C * s + 8.0 * N * C
    emb = {"shape": [N, C, V], "bytes": by}
    for kind, ids in ids_by.items():
        for det in (False, True):
            t = ev_time(lambda: ops.embed_bwd(ids, dx0, dwte, ws=wse if det else None), reps, torch)
            emb[f"{kind}_{'deterministic' if det else 'atomic'}"] = {
                "ms": t * 1e3, "GBps": by / t / 1e9, "frac_hbm_peak": by / t / PEAK_HBM}
    out["embed_bwd"] = emb
    del dwte, wse
    nc, voff = w.ve_gate_channels, (H + Hkv) * D
    dq_ve, ve_t = rnd(N, W3), rnd(V, Hkv * D)
    s_save = torch.randn(N, Hkv, generator=g, device=dev, dtype=torch.float32)
    xn_ve, dxn_ve, wg = rnd(N, C), rnd(N, C), rnd(Hkv, nc)
    dve = torch.empty(V, Hkv * D, dtype=torch.float32, device=dev)
    dwg = torch.empty(Hkv, nc, dtype=torch.float32, device=dev)
    vef = {"shape": [N, Hkv, D, V, nc]}
    for det in (False, True):
        wsv = torch.empty(max(ops.ve_bwd_ws_bytes(N, Hkv, nc, det), 16), dtype=torch.uint8, device=dev)
        for kind, ids in ids_by.items():
            t = ev_time(lambda: ops.ve_bwd(Hkv, D, dq_ve, voff, ids, ve_t, s_save, xn_ve, dxn_ve, wg, dve, dwg, wsv,
                                           deterministic=det), reps, torch)
            vef[f"{kind}_{'deterministic' if det else 'atomic'}"] = {"ms": t * 1e3}
        del wsv
    out["value_embed_bwd"] = vef
    del dq_ve, ve_t, s_save, xn_ve, dxn_ve, wg, dve, dwg, dx0, ids_by
    # decode attention (inference step, bandwidth): the workload's B sequences
    # with T cached positions, one new query each; every visible K and V row
    # read once (a window keeps only the last window+1 rows)
    lens = torch.full((w.B,), w.T, dtype=torch.int32, device=dev)
    kc, vc = rnd(w.B, w.T, Hkv, D), rnd(w.B, w.T, Hkv, D)
    qd, od = rnd(w.B, H * D), torch.empty(w.B, H * D, dtype=dt, device=dev)
    lsd = torch.empty(w.B, H, dtype=torch.float32, device=dev)
    for win in sorted(set(w.windows)):
        nb = ops.attention_decode_ws_bytes(w.B, H, Hkv, D, w.T, win)
        wsd = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
        t = ev_time(lambda: ops.attention_decode(w.B, H, Hkv, D, win, qd, H * D, kc, vc, Hkv * D, w.T * Hkv * D,
                                                 lens, w.T, od, H * D, lsd, wsd), reps, torch)
        nvis = w.T if win < 0 else min(w.T, win + 1)
        by = 2.0 * w.B * nvis * Hkv * D * s + 2.0 * w.B * H * D * s
        key = "full" if win < 0 else f"window{win}"
        out[f"attn_decode_{key}"] = {"shape": [w.B, w.T, H, Hkv, D], "ms": t * 1e3, "GBps": by / t / 1e9,
                                     "frac_hbm_peak": by / t / PEAK_HBM}
    del kc, vc
    # optimizer step (after the backward): Muon on the stack of every layer's
    # MLP up-projection matrix (momentum, 5 Newton-Schulz iterations as
    # batched MFMA GEMMs, update), AdamW over the embedding and lm_head tables
    coeffs = [(8.156, -22.483, 15.879), (4.043, -2.809, 0.5)] + [(1.5, -0.5, 0.0)] * 3
    nl = w.n_layer
    pm = torch.zeros(nl, F, C, dtype=torch.float32, device=dev)
    gm, bm = rnd(nl, F, C).float(), torch.zeros(nl, F, C, dtype=torch.float32, device=dev)
    wsm = torch.empty(ops.muon_ws_bytes(F, C, dt, nl), dtype=torch.uint8, device=dev)
    t = ev_time(lambda: ops.muon_step(pm, gm, bm, 0.02, 0.95, True, 0.0, 1.0, coeffs, dt, wsm), max(2, reps // 5),
                torch)
    s_, L_ = min(F, C), max(F, C)
    fl = nl * len(coeffs) * (4.0 * s_ * s_ * L_ + 2.0 * s_ ** 3)
    out["muon_step_w_fc_stack"] = {"shape": [nl, F, C], "ns_steps": len(coeffs), "ms": t * 1e3,
                                   "tflops": fl / t / 1e12, "frac_bf16_peak": fl / t / PEAK_BF16}
    del pm, gm, bm, wsm
    na = 2 * V * C
    pa, ga = torch.zeros(na, dtype=torch.float32, device=dev), rnd(na).float()
    ma, va = torch.zeros(na, dtype=torch.float32, device=dev), torch.zeros(na, dtype=torch.float32, device=dev)
    plo = torch.empty(na, dtype=torch.bfloat16, device=dev)
    t = ev_time(lambda: ops.adamw_step(pa, ga, ma, va, 1, 1e-3, 0.8, 0.95, 1e-8, 0.0, p_bf16=plo), reps, torch)
    by = na * (7 * 4.0 + 2)
    out["adamw_wte_lm_head"] = {"params": na, "ms": t * 1e3, "GBps": by / t / 1e9, "frac_hbm_peak": by / t / PEAK_HBM}
    del pa, ga, ma, va, plo
    torch.cuda.empty_cache()
    return out


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_mlp_up_d24_hbm_traffic.txt")
GEMM_SOURCES = [os.path.join(ROOT, "gpt_decoder_block_amd", "csrc", f) for f in ("gemm.hip", "common.h", "kernels.h")]


def gemm_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the roofline kernel from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, each calibrated on a copy of known
    size), or None when the GEMM sources changed since it was taken."""
    try:
        kv = dict(l.split(":", 1) for l in open(TRAFFIC_FILE) if ":" in l and not l.startswith("#"))
        kv = {k.strip(): v.strip() for k, v in kv.items()}
        if kv.get("source_sha256_16") != gemm_source_hash():
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(w):
    """The fp64 oracle on the host cores: one block forward+backward per layer
    kind at B=1, T=w.T, plus the head at N=T tokens; scaled to the whole stack."""
    import oracle as O
    from seeded_inputs import draw_globals, draw_ids, draw_layer, draw_upstream, to_dtype
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    T = w.T
    cos, sin = O.rope_tables(T, w.head_dim, w.rope_base)
    times = {}
    t_start = time.perf_counter()
    # layer kinds: window, and (with the extras) whether the block has a value embedding
    kind = lambda l: (w.windows[l], bool(w.extras and l % 2 == 1))
    ids = draw_ids(w.with_(B=1))[:, :T]
    for l in range(w.n_layer):
        if kind(l) in times:
            continue
        p = {k: np.asarray(to_dtype(v, w.dtype), dtype=np.float64) for k, v in draw_layer(w, l).items()}
        x = draw_upstream(w, 100, (1, T, w.C), 1.0).astype(np.float64)
        x0 = draw_upstream(w, 150, (1, T, w.C), 1.0).astype(np.float64) if w.extras else None
        dy = draw_upstream(w, 200, (1, T, w.C), 1.0).astype(np.float64)
        t0 = time.perf_counter()
        out, c = O.block_forward(x, p, w, l, cos, sin, x0=x0, ids=ids)
        O.block_backward(dy, c, p, w, l, cos, sin, ids=ids)
        times[kind(l)] = time.perf_counter() - t0
    g = draw_globals(w)
    x = draw_upstream(w, 300, (T, w.C), 1.0).astype(np.float64)
    y = np.random.default_rng(0).integers(0, w.vocab, size=T)
    t0 = time.perf_counter()
    O.lm_head_ce(x, to_dtype(g["w_lm"], w.dtype).astype(np.float64), y, w.eps)
    O.embed_backward(x, y, w.vocab)
    t_head = time.perf_counter() - t0
    total = sum(times[kind(l)] for l in range(w.n_layer)) + t_head
    return {"value": T / total, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"one block fwd+bwd per layer kind ({len(times)} kinds) at B=1, T={T} and the "
                      f"head+embedding at {T} tokens, fp64 numpy; per-step time = sum over the {w.n_layer} "
                      f"layers of their kind's time + head; measured {time.perf_counter() - t_start:.1f} s",
            "host_cpu_count": os.cpu_count()}


class ClockSampler:
    """GPU core clock during the timed steps: `amd-smi metric -c` sampled in a
    thread (the mean over the compute dies' current clocks per sample)."""

    def __init__(self):
        import threading
        self.samples, self._stop = [], threading.Event()
        self._t = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        import re
        import subprocess
        while not self._stop.is_set():
            try:
                r = subprocess.run(["amd-smi", "metric", "-c"], capture_output=True, text=True, timeout=5)
                blk = r.stdout.split("CLOCK:", 1)[-1]
                mhz = [int(m) for m in re.findall(r"GFX_\d+:\s*CLK:\s*(\d+)\s*MHz", blk)]
                if mhz:
                    self.samples.append(sum(mhz) / len(mhz))
            except (OSError, subprocess.SubprocessError, ValueError):
                return
            self._stop.wait(0.2)

    def __enter__(self):
        self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._t.join(timeout=10)

    def summary(self):
        if not self.samples:
            return None
        v = sorted(self.samples)
        return {"samples": len(v), "median_mhz": v[len(v) // 2], "min_mhz": v[0], "max_mhz": v[-1],
                "source": "amd-smi metric -c, mean over the compute dies, sampled during the timed steps"}


def env_info(torch):
    """Device and runtime the figures were taken on."""
    pr = torch.cuda.get_device_properties(0)
    cpu = ""
    try:
        cpu = next((l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name")), "")
    except OSError:
        pass
    return {"device": pr.name, "arch": getattr(pr, "gcnArchName", ""), "compute_units": pr.multi_processor_count,
            "hbm_gib": round(pr.total_memory / 2 ** 30, 1), "hip": torch.version.hip, "torch": torch.__version__,
            "host_cpu": cpu, "host_cpu_count": os.cpu_count()}


def main():
    args = parse()
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; --gpus must be 1 "
                                   "(the multi-GPU data-parallel design is described, not built)"}))
        sys.exit(2)
    import torch
    from gpt_decoder_block_amd import ops
    from gpt_decoder_block_amd.stack import DecoderStack
    from gpt_decoder_block_amd.workmodel import flops_per_token, flops_per_token_pages, step_flops
    from seeded_inputs import draw_globals, draw_ids, draw_layer, to_dtype, workload

    w = workload(args.workload)
    if args.batch:
        w = w.with_(B=args.batch)
    if args.counter_run:
        counter_run(w)
        return
    dev = "cuda:0"
    st = DecoderStack(n_layer=w.n_layer, B=w.B, T=w.T, C=w.C, n_head=w.n_head, n_kv_head=w.n_kv_head,
                      head_dim=w.head_dim, mlp_hidden=w.mlp_hidden, vocab=w.vocab, windows=w.windows,
                      dtype=w.dtype, eps=w.eps, rope_base=w.rope_base, device=dev, extras=w.extras,
                      ve_gate_channels=w.ve_gate_channels, smear_channels=w.smear_channels, mlp_fp8=w.mlp_fp8)
    print(f"[bench] {w.name}: L={w.n_layer} B={w.B} T={w.T} C={w.C} H={w.n_head}/{w.n_kv_head} "
          f"dtype={w.dtype} extras={w.extras} fp8={w.mlp_fp8}; drawing weights", file=sys.stderr, flush=True)
    rd = lambda v: np.asarray(to_dtype(v, w.dtype)) if np.ndim(v) else np.float32(v)
    st.load({k: rd(v) for k, v in draw_globals(w).items()},
            [{k: rd(v) for k, v in draw_layer(w, l).items()} for l in range(w.n_layer)])
    st.set_ids(draw_ids(w))
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        st.step()
    torch.cuda.synchronize()
    loss0 = float(st.loss.item())
    print("[bench] kernel figures", file=sys.stderr, flush=True)
    kern = kernel_figures(w, st, args.kernel_reps, torch, ops)
    for _ in range(2):   # back to the step's steady state
        st.step()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    with ClockSampler() as clk:
        e0.record(s)
        evs[0].record(s)
        for i in range(args.steps):
            st.step()
            evs[i + 1].record(s)
        e1.record(s)
        torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / args.steps
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    print(f"[bench] {args.steps} steps: {ms:.2f} ms/step (wall {wall / args.steps * 1e3:.2f}), loss {loss0:.4f}",
          file=sys.stderr, flush=True)
    tokens = w.B * w.T
    fpt = flops_per_token(w.n_layer, w.C, w.n_head, w.n_kv_head, w.head_dim, w.mlp_hidden, w.vocab, w.T, w.windows)
    fpt_pages = flops_per_token_pages(w.n_layer, w.C, w.n_head, w.n_kv_head, w.head_dim, w.mlp_hidden, w.vocab,
                                      w.T, w.windows)
    tps = tokens / (ms / 1e3)
    tflops = fpt * tps / 1e12
    if w.mlp_fp8:
        dom, peak = kern["gemm_fp8_mlp_up_sqr"], PEAK_FP8
        kname = "gemm_bf16_k<K-major, K-major, relu^2 epilogue, fp8> (MLP up-projection on e4m3 codes, stores h)"
        traffic = None
    else:
        dom, peak = kern["gemm_mlp_up_sqr"], PEAK_BF16
        kname = "gemm_bf16_k<K-major, K-major, relu^2 epilogue> (MLP up-projection, stores h = relu(u)^2)"
        traffic = measured_traffic()
    roof = {"kernel": kname, "bound": "mfma", "achieved": dom["tflops"], "peak": peak / 1e12, "unit": "TFLOP/s",
            "frac": dom["tflops"] / (peak / 1e12), "traffic": traffic,
            "algorithmic_per_launch": f"2*M*N*K = {dom['flops']:.4g} FLOP (M={dom['shape'][0]} tokens, "
                                      f"N={dom['shape'][1]}, K={dom['shape'][2]})",
            "avg_launch_ms": dom["ms"]}
    res = {"metric": METRIC, "value": tps, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": w.dtype + ("; MLP products fp8 e4m3" if w.mlp_fp8 else ""),
           "data": "synthetic",
           "config": {"workload": f"{w.name}: {w.n_layer} blocks, C={w.C}, heads {w.n_head}/{w.n_kv_head}x"
                                  f"{w.head_dim}, MLP {w.mlp_hidden}, vocab {w.vocab}"
                                  + (", residual mixing, value embeddings, smear, backout" if w.extras else "")
                                  + (", fp8 MLP products" if w.mlp_fp8 else ""),
                      "global_batch": w.B, "seq_len": w.T, "windows": sorted(set(w.windows)),
                      "parallelism": "single GPU"},
           "tflops": tflops, "pct_bf16_peak": 100.0 * tflops * 1e12 / PEAK_BF16,
           "flops_per_token": fpt, "flops_per_token_pages_convention": fpt_pages,
           "tflops_pages_convention": fpt_pages * tps / 1e12,
           "loss_after_warmup": loss0,
           "ms_per_step_median": per_step[len(per_step) // 2], "ms_per_step_min": per_step[0],
           "ms_per_step_max": per_step[-1],
           "env": env_info(torch), "gpu_clock_during_timed_steps": clk.summary(),
           "roofline": roof, "kernels": kern}
    if "gemm_wgrad" in kern:
        wg = kern["gemm_wgrad"]
        res["roofline_weight_gradients"] = {
            "kernel": "gemm_bf16_k<M-major, N-major, fp32 split-K epilogue> + splitk_reduce_k (every weight "
                      "gradient of the step: the largest kernel by time)",
            "bound": "mfma", "achieved": wg["tflops"], "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
            "frac": wg["frac_bf16_peak"], "avg_launch_ms": wg["avg_launch_ms"],
            "algorithmic_per_launch": f"2*M*N*K averaged over the step's {wg['launches_per_step']} launches = "
                                      f"{wg['avg_flops_per_launch']:.4g} FLOP (K = {w.B * w.T} tokens)"}
    if w.mlp_fp8:
        # mixed roofline: the MLP's six products per layer on the fp8 peak, the rest on bf16
        f_fp8 = 6.0 * 2 * w.C * w.mlp_hidden * w.n_layer * tokens
        f_all = fpt * tokens
        t_ideal = (f_all - f_fp8) / PEAK_BF16 + f_fp8 / PEAK_FP8
        res["mixed_roofline"] = {"fp8_flops_per_step": f_fp8, "bf16_flops_per_step": f_all - f_fp8,
                                 "ideal_ms": t_ideal * 1e3, "frac": t_ideal / (ms / 1e3)}
    if not args.no_cpu:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
