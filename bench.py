"""Benchmark of the Kronecker-factored layer's forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps 100] [--warmup 10] [--cpu-seconds 10]

One step is one kron_linear_fwd + one kron_linear_bwd call (x, S, A, B, dy resident in
HBM; outputs and workspace preallocated) on the 1024 x 1024 layer with m = n = 32
(p = q = 32), r = 4, half of S zeroed, 20,000 rows.  Prints one JSON line.

Algorithmic work per row (counted once, whatever the kernels execute):
  forward  2*r*n*(p*m + nnz)                 flops, 4*(in + out) bytes
  backward 2*r*n*(nnz + 2*p*m + p*q)         flops, 4*(2*in + out) bytes
with nnz the number of nonzero entries of S.
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

PEAK_FP32_TFLOPS = 157.3     # MI355X dense fp32 (matrix cores), published
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, published
METRIC = "kron_linear fwd+bwd rows/s and % of HBM/fp32 roofline, 1024² m=32 r=4"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def work_per_row(p, q, m, n, r, nnz):
    ff = 2 * r * n * (p * m + nnz)
    fb = 2 * r * n * (nnz + 2 * p * m + p * q)
    bf = 4 * (p * m + q * n)
    bb = 4 * (2 * p * m + q * n)
    return ff, fb, bf, bb


def cpu_baseline(inp, seconds: float):
    """The oracle (as it stands) on the same workload, repeated for about `seconds`."""
    from oracle import kron as OK
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    N = inp.x.shape[0]
    rows, t0 = 0, time.perf_counter()
    calls = 0
    while True:
        OK.forward(inp.x, inp.S, inp.A, inp.B, inp.bias)
        OK.backward(inp.x, inp.S, inp.A, inp.B, inp.dy, want_dx=True)
        rows += N
        calls += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": rows / dt, "unit": "rows/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{calls} x (fwd+bwd over all {N} rows of the same workload), fp64 numpy/OpenBLAS, "
                      f"{dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the Kronecker layer's hot path runs on one GPU's share "
              f"of rows); --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import kronecker_factored_structured_amd as K
    from workloads import headline_layer

    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    dev = torch.device("cuda:0")
    inp = headline_layer()
    sh = inp.shape
    N, p, q, m, n, r = sh.N, sh.p, sh.q, sh.m, sh.n, sh.r
    nnz = int(np.count_nonzero(inp.S))
    t = lambda a: torch.from_numpy(a).to(dev).contiguous()
    x, S, A, B, bias, dy = t(inp.x), t(inp.S), t(inp.A), t(inp.B), t(inp.bias), t(inp.dy)
    y = torch.empty(N, q * n, device=dev)
    outs = dict(dx=torch.empty_like(x), dS=torch.empty_like(S), dA=torch.empty_like(A),
                dB=torch.empty_like(B), dbias=torch.empty_like(bias))
    shape = K.layer_shape(N, S, A, B)
    ws = torch.empty(K.kron_linear_bwd_workspace_bytes(shape), dtype=torch.uint8, device=dev)

    def fwd():
        K.kron_linear_fwd(x, S, A, B, bias, out=y)

    def bwd():
        K.kron_linear_bwd(x, S, A, B, dy, workspace=ws, outs=outs)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()

    # Whole-step timing.
    log(f"[bench] timing {args.steps} steps")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        fwd()
        bwd()
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - w0) * 1e3 / args.steps
    ms_step = e0.elapsed_time(e1) / args.steps

    # Per-call timing with events on the stream the kernels run on.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for a, b, c in ev:
        a.record()
        fwd()
        b.record()
        bwd()
        c.record()
    torch.cuda.synchronize()
    t_fwd = float(np.mean([a.elapsed_time(b) for a, b, _ in ev])) * 1e-3
    t_bwd = float(np.mean([b.elapsed_time(c) for _, b, c in ev])) * 1e-3

    ff, fb, bf, bb = work_per_row(p, q, m, n, r, nnz)
    t_roof = max(N * (ff + fb) / (PEAK_FP32_TFLOPS * 1e12), N * (bf + bb) / (PEAK_HBM_GBS * 1e9))
    # Dominant launch: the backward call (its main kernel plus the fixed-order reduction).
    achieved = N * fb / t_bwd / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_FP32_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP32_TFLOPS, 4), "traffic": None,
                "kernel": "kron_linear_bwd", "t_us": round(t_bwd * 1e6, 2),
                "flop_per_row": fb, "rows": N}
    value = N / (ms_step * 1e-3)
    rec = {
        "metric": METRIC, "value": round(value, 1), "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "kron_linear fwd+bwd, 1024x1024 layer, m=n=32 (p=q=32), r=4, "
                               "S~U(0,1) with 512 of 1024 entries zeroed, 20000 rows",
                   "N": N, "p": p, "q": q, "m": m, "n": n, "r": r, "nnz_S": nnz, "parallelism": "none"},
        "roofline": roofline,
        "pass_roofline": {"bound": "fp32", "t_roof_us": round(t_roof * 1e6, 2),
                          "t_us": round(ms_step * 1e3, 2), "frac": round(t_roof / (ms_step * 1e-3), 4),
                          "effective_tflops": round(N * (ff + fb) / (ms_step * 1e-3) / 1e12, 3)},
        "t_fwd_us": round(t_fwd * 1e6, 2), "t_bwd_us": round(t_bwd * 1e6, 2),
        "wall_ms_per_step": round(wall_ms, 5),
    }
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (oracle) for ~{args.cpu_seconds} s")
        rec["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
