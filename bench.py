"""Benchmark of the Kronecker-factored layer on one MI355X.

    python bench.py [--gpus 1] [--steps 100] [--warmup 10] [--cpu-seconds 10]
    python bench.py --workload {headline,headline_bf16,tiny,mlp_step,gpt2_ffn,gpt2_ffn_bf16,ks,ks_bwd,chain,van_loan,sweep,small_blocks}
    python bench.py --calibrate-copy      (plain device copy of known size, for HBM counters)

Default workload (one JSON line): one step is one kron_linear_fwd + one kron_linear_bwd
call (x, S, A, B, dy resident in HBM; outputs and workspace preallocated) on the
1024 x 1024 layer with m = n = 32 (p = q = 32), r = 4, half of S zeroed, 20,000 rows.

Algorithmic work per row (counted once, whatever the kernels execute):
  forward  2*r*n*(p*m + nnz)                 flops, 4*(in + out) bytes
  backward 2*r*n*(nnz + 2*p*m + p*q)         flops, 4*(2*in + out) bytes
with nnz the number of nonzero entries of S (S-zero terms are not counted as work).
The roofline entry describes the backward call, the dominant launch: its main kernel
and the fixed-order reduction of the per-workgroup partial sums, timed together with
HIP events on the stream the kernels run on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP32_TFLOPS = 157.3     # MI355X dense fp32 matrix, published
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 matrix, published
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, published
METRIC = "kron_linear fwd+bwd rows/s and % of HBM/fp32 roofline, 1024² m=32 r=4"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_kron_linear_bwd_headline.json")
KERNEL_SOURCES = ("kron_mfma.hip", "kron_generic.hip", "kron_api.cpp", "kron_internal.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "kronecker_factored_structured_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per backward call from the committed counter summary, or None when the
    kernel sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_sha():
        return None
    return t.get("bytes_per_call")


def work_per_row(p, q, m, n, r, nnz):
    ff = 2 * r * n * (p * m + nnz)
    fb = 2 * r * n * (nnz + 2 * p * m + p * q)
    bf = 4 * (p * m + q * n)
    bb = 4 * (2 * p * m + q * n)
    return ff, fb, bf, bb


SETTLE_SECONDS = [1.0]


def timed(fn, steps, warmup):
    """Mean ms per call of fn (events on the current stream) and the host wall clock.

    Before the `warmup` untimed calls, fn runs untimed for SETTLE_SECONDS so that the
    GPU clock has left its idle state (the first ~0.1 s of work after idle runs about 10%
    slower); neither phase is part of the timed region."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < SETTLE_SECONDS[0]:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, (time.perf_counter() - w0) * 1e3 / steps


def cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(inp, seconds: float):
    """The oracle (as it stands) on the same workload, repeated for about `seconds`."""
    from oracle import kron as OK
    N = inp.x.shape[0]
    rows, calls, t0 = 0, 0, time.perf_counter()
    while True:
        OK.forward(inp.x, inp.S, inp.A, inp.B, inp.bias)
        OK.backward(inp.x, inp.S, inp.A, inp.B, inp.dy, want_dx=True)
        rows += N
        calls += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": rows / dt, "unit": "rows/s", "cores": int(cpu_threads()), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{calls} x (fwd+bwd over all {N} rows of the same workload), fp64 numpy/OpenBLAS, "
                      f"{dt:.1f} s"}


class Layer:
    """Device tensors and preallocated outputs of one Kronecker layer workload."""

    def __init__(self, inp, dev, sparse_rows=False, save_z=False):
        import torch
        import kronecker_factored_structured_amd as K
        self.K = K
        self.sparse_rows = sparse_rows
        t = lambda a: None if a is None else torch.from_numpy(a).to(dev).contiguous()
        self.x, self.S, self.A, self.B, self.bias, self.dy = (t(a) for a in (inp.x, inp.S, inp.A, inp.B,
                                                                           inp.bias, inp.dy))
        sh = inp.shape
        self.y = torch.empty(sh.N, sh.q * sh.n, device=dev)
        self.outs = dict(dx=torch.empty_like(self.x), dS=None if self.S is None else torch.empty_like(self.S),
                         dA=torch.empty_like(self.A), dB=torch.empty_like(self.B),
                         dbias=None if self.bias is None else torch.empty_like(self.bias))
        shape = K.layer_shape(sh.N, self.S, self.A, self.B)
        self.ws = torch.empty(K.kron_linear_bwd_workspace_bytes(shape), dtype=torch.uint8, device=dev)
        # save_z: the forward keeps Z_i = X B_i for the backward (None where the shape has no such path)
        self.zc = K.new_zcache(self.x, self.S, self.A, self.B) if save_z else None

    def fwd(self):
        self.K.kron_linear_fwd(self.x, self.S, self.A, self.B, self.bias, out=self.y, sparse_rows=self.sparse_rows,
                               zcache=self.zc)

    def bwd(self):
        self.K.kron_linear_bwd(self.x, self.S, self.A, self.B, self.dy, workspace=self.ws, outs=self.outs,
                               sparse_rows=self.sparse_rows, zcache=self.zc)


class LayerBf16:
    """bf16 tensors of one Kronecker layer workload (inputs rounded to bf16 once, on the host);
    y and dx bf16, factor gradients fp32."""

    def __init__(self, inp, dev):
        import torch
        import kronecker_factored_structured_amd as K
        from workloads import bf16_bits
        self.K = K

        def t(a):
            if a is None:
                return None
            bits = bf16_bits(np.ascontiguousarray(a, dtype=np.float32))
            return torch.from_numpy(bits.view(np.int16).copy()).to(dev).view(torch.bfloat16)

        self.x, self.S, self.A, self.B, self.bias, self.dy = (t(a) for a in (inp.x, inp.S, inp.A, inp.B,
                                                                           inp.bias, inp.dy))
        sh = inp.shape
        f32 = torch.float32
        self.y = torch.empty(sh.N, sh.q * sh.n, device=dev, dtype=torch.bfloat16)
        self.outs = dict(dx=torch.empty_like(self.x),
                         dS=None if self.S is None else torch.empty(self.S.shape, device=dev, dtype=f32),
                         dA=torch.empty(self.A.shape, device=dev, dtype=f32),
                         dB=torch.empty(self.B.shape, device=dev, dtype=f32),
                         dbias=None if self.bias is None else torch.empty(self.bias.shape, device=dev, dtype=f32))
        shape = K.layer_shape(sh.N, self.S, self.A, self.B)
        self.ws = torch.empty(K.kron_linear_bwd_bf16_workspace_bytes(shape), dtype=torch.uint8, device=dev)

    def fwd(self):
        self.K.kron_linear_fwd_bf16(self.x, self.S, self.A, self.B, self.bias, out=self.y)

    def bwd(self):
        self.K.kron_linear_bwd_bf16(self.x, self.S, self.A, self.B, self.dy, workspace=self.ws, outs=self.outs)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def measured_ceilings(dev):
    """Context for the roofline fractions, measured on this GPU outside the timed region:
    a 1 GiB device copy (read + write bytes per second) and a large fp32 GEMM through the
    vendor library (matrix-core throughput without the layer's structure)."""
    import torch
    ev = lambda: torch.cuda.Event(enable_timing=True)
    nb = 1 << 30
    a = torch.empty(nb // 4, device=dev)
    b = torch.empty_like(a)
    a.fill_(1.0)
    for _ in range(3):
        b.copy_(a)
    e0, e1 = ev(), ev()
    e0.record()
    for _ in range(10):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * nb * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    n = 8192
    allow = torch.backends.cuda.matmul.allow_tf32
    torch.backends.cuda.matmul.allow_tf32 = False
    A = torch.randn(n, n, device=dev)
    B = torch.randn(n, n, device=dev)
    C = torch.empty(n, n, device=dev)
    for _ in range(2):
        torch.mm(A, B, out=C)
    e0, e1 = ev(), ev()
    e0.record()
    for _ in range(5):
        torch.mm(A, B, out=C)
    e1.record()
    torch.cuda.synchronize()
    torch.backends.cuda.matmul.allow_tf32 = allow
    gemm_tflops = 2 * n ** 3 * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del A, B, C
    torch.cuda.empty_cache()
    return {"copy_gbs": round(copy_gbs, 1), "fp32_gemm_tflops": round(gemm_tflops, 2),
            "how": "1 GiB torch device copy x10 (read+write bytes); torch.mm fp32 8192^3 x5, TF32 off"}


def split_times(layer, steps, medians=False):
    """Mean seconds of the forward and of the backward call, from events around each call
    (and their medians, and the median of their sum, when asked)."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b, c in ev:
        a.record()
        layer.fwd()
        b.record()
        layer.bwd()
        c.record()
    torch.cuda.synchronize()
    f = np.array([a.elapsed_time(b) for a, b, _ in ev]) * 1e-3
    g = np.array([b.elapsed_time(c) for _, b, c in ev]) * 1e-3
    t_fwd, t_bwd = float(np.mean(f)), float(np.mean(g))
    if medians:
        return t_fwd, t_bwd, float(np.median(f)), float(np.median(g)), float(np.median(f + g))
    return t_fwd, t_bwd


def run_headline(args, dev):
    from workloads import headline_layer
    inp = headline_layer()
    sh = inp.shape
    N, p, q, m, n, r = sh.N, sh.p, sh.q, sh.m, sh.n, sh.r
    nnz = int(np.count_nonzero(inp.S))
    # the timed step saves Z_i = X B_i in the forward for the backward (kron_linear_fwd_save /
    # kron_linear_bwd_saved); the recomputing pair (kron_linear_fwd / kron_linear_bwd) is
    # timed beside it
    L = Layer(inp, dev, save_z=not args.recompute_z)
    log(f"[bench] headline ({'recomputed' if L.zc is None else 'saved'} Z): warmup {args.warmup}, "
        f"timing {args.steps} steps")
    ms_step, wall_ms = timed(lambda: (L.fwd(), L.bwd()), args.steps, args.warmup)
    t_fwd, t_bwd, med_fwd, med_bwd, med_step = split_times(L, args.steps, medians=True)
    other = None
    if L.zc is not None:
        L.zc = None
        log(f"[bench] headline, recomputed Z: timing {args.steps} steps")
        ms_r, _ = timed(lambda: (L.fwd(), L.bwd()), args.steps, args.warmup)
        tf_r, tb_r = split_times(L, args.steps)
        other = {"path": "kron_linear_fwd + kron_linear_bwd (Z recomputed in the backward)",
                 "ms_per_step": round(ms_r, 5), "t_fwd_us": round(tf_r * 1e6, 2), "t_bwd_us": round(tb_r * 1e6, 2)}
    ff, fb, bf, bb = work_per_row(p, q, m, n, r, nnz)
    t_roof = max(N * (ff + fb) / (PEAK_FP32_TFLOPS * 1e12), N * (bf + bb) / (PEAK_HBM_GBS * 1e9))
    achieved = N * fb / t_bwd / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_FP32_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP32_TFLOPS, 4),
                "traffic": measured_traffic(),
                "kernel": "kron_linear_bwd (main kernel + fixed-order partial-sum reduction)",
                "t_us": round(t_bwd * 1e6, 2), "flop_per_row": fb, "rows": N,
                "algorithmic_bytes": N * bb,
                "z_saved": other is not None,
                # the saved Z, written by the forward and read by the backward (not algorithmic)
                "zcache_bytes": N * r * p * n * 4 if other is not None else 0}
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
                          "effective_tflops": round(N * (ff + fb) / (ms_step * 1e-3) / 1e12, 3),
                          # context only: the flops the same pass would count with S dense
                          "dense_equivalent_tflops": round(N * sum(work_per_row(p, q, m, n, r, p * q)[:2]) /
                                                           (ms_step * 1e-3) / 1e12, 3)},
        "t_fwd_us": round(t_fwd * 1e6, 2), "t_bwd_us": round(t_bwd * 1e6, 2),
        "median_us": {"fwd": round(med_fwd * 1e6, 2), "bwd": round(med_bwd * 1e6, 2),
                      "fwd_bwd": round(med_step * 1e6, 2)},
        "wall_ms_per_step": round(wall_ms, 5),
        "recompute_path": other,
        "kernel_source_sha": kernel_source_sha(),
        "settle_seconds": args.settle_seconds,
    }
    if not args.no_ceilings:
        log("[bench] measured ceilings (copy, fp32 GEMM)")
        ceil = measured_ceilings(dev)
        ceil["bwd_frac_of_gemm"] = round(achieved / ceil["fp32_gemm_tflops"], 4)
        ceil["pass_frac_of_gemm"] = round(N * (ff + fb) / (ms_step * 1e-3) / 1e12 / ceil["fp32_gemm_tflops"], 4)
        rec["measured_ceilings"] = ceil
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (oracle) for ~{args.cpu_seconds} s")
        rec["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def layer_record(name, inp, L, args, extra=None):
    sh = inp.shape
    N, p, q, m, n, r = sh.N, sh.p, sh.q, sh.m, sh.n, sh.r
    nnz = p * q if inp.S is None else int(np.count_nonzero(inp.S))
    ms, _ = timed(lambda: (L.fwd(), L.bwd()), args.steps, args.warmup)
    t_fwd, t_bwd, med_fwd, med_bwd, med_step = split_times(L, args.steps, medians=True)
    ff, fb, bf, bb = work_per_row(p, q, m, n, r, nnz)
    if inp.S is None:   # dense factors: the cheaper association of each product counts
        ff = 2 * r * min(p * n * (m + q), q * m * (p + n))
        fb = 2 * ff
    t_roof = max(N * (ff + fb) / (PEAK_FP32_TFLOPS * 1e12), N * (bf + bb) / (PEAK_HBM_GBS * 1e9))
    rec = {"workload": name, "rows_per_s": round(N / (ms * 1e-3), 1), "us_per_fwd_bwd": round(ms * 1e3, 2),
           "t_fwd_us": round(t_fwd * 1e6, 2), "t_bwd_us": round(t_bwd * 1e6, 2),
           "effective_tflops": round(N * (ff + fb) / (ms * 1e-3) / 1e12, 3),
           "t_roof_us": round(t_roof * 1e6, 2), "roofline_frac": round(t_roof / (ms * 1e-3), 4),
           "bound": "fp32" if N * (ff + fb) / (PEAK_FP32_TFLOPS * 1e12) >= N * (bf + bb) / (PEAK_HBM_GBS * 1e9)
           else "hbm",
           "shape": {"N": N, "p": p, "q": q, "m": m, "n": n, "r": r}}
    if extra:
        rec.update(extra)
    print(json.dumps(rec), flush=True)


def bf16_layer_record(name, inp, L, args):
    """One bf16 layer's fwd+bwd line.  Algorithmic bytes halve with the element size while
    the flops stay, so these layers are bound by HBM or by the bf16 matrix rate, whichever
    is slower."""
    sh = inp.shape
    N, p, q, m, n, r = sh.N, sh.p, sh.q, sh.m, sh.n, sh.r
    nnz = p * q if inp.S is None else int(np.count_nonzero(inp.S))
    ms, _ = timed(lambda: (L.fwd(), L.bwd()), args.steps, args.warmup)
    t_fwd, t_bwd = split_times(L, args.steps)
    ff, fb, _, _ = work_per_row(p, q, m, n, r, nnz)
    if inp.S is None:   # dense factors: the cheaper association of each product counts
        ff = 2 * r * min(p * n * (m + q), q * m * (p + n))
        fb = 2 * ff
    bf, bb = 2 * (p * m + q * n), 2 * (2 * p * m + q * n)
    t_flop = N * (ff + fb) / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = N * (bf + bb) / (PEAK_HBM_GBS * 1e9)
    t_roof = max(t_flop, t_hbm)
    print(json.dumps({"workload": name,
                      "rows_per_s": round(N / (ms * 1e-3), 1), "us_per_fwd_bwd": round(ms * 1e3, 2),
                      "t_fwd_us": round(t_fwd * 1e6, 2), "t_bwd_us": round(t_bwd * 1e6, 2),
                      "achieved_gbs": round(N * (bf + bb) / (ms * 1e-3) / 1e9, 1),
                      "effective_tflops": round(N * (ff + fb) / (ms * 1e-3) / 1e12, 3),
                      "t_roof_us": round(t_roof * 1e6, 2), "roofline_frac": round(t_roof / (ms * 1e-3), 4),
                      "bound": "hbm" if t_hbm >= t_flop else "bf16",
                      "t_bf16_flops_us": round(t_flop * 1e6, 2), "t_hbm_us": round(t_hbm * 1e6, 2),
                      "shape": {"N": N, "p": p, "q": q, "m": m, "n": n, "r": r}}), flush=True)


def run_headline_bf16(args, dev):
    """The same layer and rows in bf16 (inputs, y, dx), fp32 accumulation and fp32 factor
    gradients."""
    from workloads import headline_layer
    inp = headline_layer()
    bf16_layer_record("headline_bf16: kron_linear fwd+bwd, 1024x1024, m=n=32, r=4, half of S zeroed, 20000 rows, "
                      "bf16 x/S/A/B/bias/dy/y/dx, fp32 dS/dA/dB/dbias", inp, LayerBf16(inp, dev), args)


def run_gpt2_bf16(args, dev):
    """The GPT-2 small FFN pair in bf16 (the side of 24 padded to 32 inside the tiles)."""
    from workloads import gpt2_ffn_layers
    for r in (1, 2, 4, 8):
        up, down = gpt2_ffn_layers(r)
        bf16_layer_record(f"gpt2 ffn bf16 768->3072 (A 32x64, B 24x48), r={r}, 8192 rows", up, LayerBf16(up, dev), args)
        bf16_layer_record(f"gpt2 ffn bf16 3072->768 (A 64x32, B 48x24), r={r}, 8192 rows", down,
                          LayerBf16(down, dev), args)


def run_tiny(args, dev):
    from workloads import tiny_layer
    inp = tiny_layer()
    layer_record("tiny: 64 rows, 64x64, m=8, r=2", inp, Layer(inp, dev), args)


def run_gpt2(args, dev):
    from workloads import gpt2_ffn_layers
    for r in (1, 2, 4, 8):
        up, down = gpt2_ffn_layers(r)
        layer_record(f"gpt2 ffn 768->3072 (A 32x64, B 24x48), r={r}, 8192 rows", up, Layer(up, dev), args)
        layer_record(f"gpt2 ffn 3072->768 (A 64x32, B 48x24), r={r}, 8192 rows", down, Layer(down, dev), args)


def run_small_blocks(args, dev):
    """The tutorial's 1024 x 1024 layer with small blocks (8x8, 4x4, 2x2; the settings its
    batch-20,000 results single out), half of S zeroed, 20,000 rows."""
    from workloads import kron_inputs
    for p, m, r in ((128, 8, 1), (128, 8, 2), (256, 4, 1), (256, 4, 2), (512, 2, 1)):
        inp = kron_inputs(80 + r, 20000, p, p, m, m, r, s_mode="uniform_zeroed", bias_mode="zeros")
        layer_record(f"small_blocks: 1024x1024 layer, {m}x{m} blocks (p=q={p}), r={r}, half of S zeroed, "
                     f"20000 rows", inp, Layer(inp, dev), args)


def run_sparse_s(args, dev):
    """The 1024 x 1024 layer (m = 32, r = 4, 20,000 rows) with whole rows of S zero (the
    structure an l1-pruned mask can leave), against S with the same share of zero entries
    at random positions, which leaves no row empty: the forward's row map runs only the
    16-row tiles that hold nonzero rows of C = S o A_i."""
    from workloads import kron_inputs
    for mode, frac in (("uniform_zeroed", 0.5), ("rows_zeroed", 0.0), ("rows_zeroed", 0.25), ("rows_zeroed", 0.5),
                       ("rows_zeroed", 0.75), ("rows_zeroed", 0.875), ("blocks_zeroed", 0.5), ("blocks_zeroed", 0.75)):
        inp = kron_inputs(90, 20000, 32, 32, 32, 32, 4, s_mode=mode, zero_frac=frac, bias_mode="zeros")
        rows_left = int(np.count_nonzero(inp.S.any(axis=1)))
        zero_blocks = [(tj, tk) for tj in range(2) for tk in range(2)
                       if not inp.S[16 * tj:16 * tj + 16, 16 * tk:16 * tk + 16].any()]
        what = (f"{frac:.0%} of S's entries zero at random" if mode == "uniform_zeroed"
                else f"{frac:.1%} of S's rows zero ({rows_left} of 32 rows left)" if mode == "rows_zeroed"
                else f"16x16 blocks {zero_blocks} of S zero")
        for hint in (False, True):
            layer_record(f"sparse_s: 1024x1024 layer, m=32, r=4, 20000 rows, {what}, "
                         f"{'KRON_SPARSE_ROWS' if hint else 'dense path'}", inp, Layer(inp, dev, sparse_rows=hint),
                         args, extra={"s_rows_nonzero": rows_left, "s_zero_blocks": zero_blocks, "sparse_rows": hint,
                                      "fwd_tiles_run": max(1, -(-rows_left // 16)) if hint else 2})


def run_mlp_step(args, dev):
    import torch
    import kronecker_factored_structured_amd as K
    from workloads import mlp_step_inputs
    inp = mlp_step_inputs()
    step = K.KronMLPStep(inp.layers, inp.head_w, inp.head_b, inp.lam, inp.lr, dev)
    x = torch.from_numpy(inp.x).to(dev)
    lab = torch.from_numpy(inp.labels).to(dev)
    ms, wall = timed(lambda: step.step(x, lab), args.steps, args.warmup)
    N = x.shape[0]
    # kron layers: layer 1 without dX, layer 2 with dX; head: 3 products of N x 1024 x 10
    p, m, r = 16, 64, 2
    ff = 2 * r * m * (p * m + p * p)
    fb2 = 2 * ff
    fb1 = fb2 - 2 * r * m * p * m
    head = 3 * 2 * 1024 * 10
    flops = N * (2 * ff + fb1 + fb2 + head)
    print(json.dumps({"workload": "mlp_step: MLP 1024-1024-1024-10, Kronecker hidden layers m=64 r=2, "
                                  "CE + 1e-4*sum|S|, fused Adam, 20000 rows",
                      "ms_per_step": round(ms, 4), "wall_ms_per_step": round(wall, 4),
                      "rows_per_s": round(N / (ms * 1e-3), 1),
                      "effective_tflops": round(flops / (ms * 1e-3) / 1e12, 3),
                      "t_roof_us": round(flops / (PEAK_FP32_TFLOPS * 1e12) * 1e6, 2)}), flush=True)


def run_ks(args, dev):
    import torch
    import kronecker_factored_structured_amd as K
    from workloads import vit_ks
    for dtype, out_dtype in (("f32", "f32"), ("bf16", "f32"), ("bf16", "bf16")):
        sets = []
        for s in range(3):   # rotate buffer sets so the working set exceeds the last-level cache
            inp = vit_ks(dtype, seed=5 + 10 * s)
            if dtype == "bf16":
                x = torch.from_numpy(inp.x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
                v = torch.from_numpy(inp.vals_bits.view(np.int16)).to(dev).view(torch.bfloat16)
            else:
                x = torch.from_numpy(inp.x).to(dev)
                v = torch.from_numpy(inp.vals).to(dev)
            y = torch.empty(x.shape[0], inp.a * inp.c * inp.d, device=dev,
                            dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16)
            sets.append((x, v, y))
        a, b, c, d = inp.a, inp.b, inp.c, inp.d
        it = [0]

        def call():
            x, v, y = sets[it[0] % len(sets)]
            it[0] += 1
            if out_dtype == "f32":
                K.ks_matmul(x, v, a, b, c, d, out=y)
            else:
                K.ks_matmul_out(x, v, a, b, c, d, out_dtype=torch.bfloat16, out=y)

        ms, _ = timed(call, args.steps, args.warmup)
        N = sets[0][0].shape[0]
        s_in = 4 if dtype == "f32" else 2
        s_out = 4 if out_dtype == "f32" else 2
        flops = N * 2 * a * b * c * d
        byts = N * (s_in * a * b * d + s_out * a * c * d) + s_in * a * b * c * d
        peak = PEAK_FP32_TFLOPS if dtype == "f32" else PEAK_BF16_TFLOPS   # the contraction's input dtype
        t_flop, t_hbm = flops / (peak * 1e12), byts / (PEAK_HBM_GBS * 1e9)
        t_roof = max(t_flop, t_hbm)
        print(json.dumps({"workload": f"ks_matmul (a,b,c,d)=(2,48,192,4), 25216 rows, {dtype} inputs, "
                                      f"{out_dtype} output",
                          "us_per_call": round(ms * 1e3, 2), "rows_per_s": round(N / (ms * 1e-3), 1),
                          "achieved_gbs": round(byts / (ms * 1e-3) / 1e9, 1),
                          "effective_tflops": round(flops / (ms * 1e-3) / 1e12, 3),
                          "t_roof_us": round(t_roof * 1e6, 2), "roofline_frac": round(t_roof / (ms * 1e-3), 4),
                          "bound": "hbm" if t_hbm >= t_flop else ("fp32" if dtype == "f32" else "bf16")}),
              flush=True)


def run_ks_bwd(args, dev):
    """ks_matmul_bwd at the ViT shape: dx = dy K^T and dvals in one call, fp32 and bf16
    inputs (fp32 outputs).  Algorithmic work: 2 products of 2*a*b*c*d flop per row; bytes
    read x and dy once and write dx once (s_in * (in + out) + 4 * in per row)."""
    import torch
    import kronecker_factored_structured_amd as K
    from workloads import vit_ks
    for dtype in ("f32", "bf16"):
        inp = vit_ks(dtype, seed=5)
        a, b, c, d = inp.a, inp.b, inp.c, inp.d
        N = inp.x.shape[0]
        g = torch.Generator(device=dev).manual_seed(3)
        dy = torch.randn(N, a * c * d, device=dev, generator=g)
        if dtype == "bf16":
            x = torch.from_numpy(inp.x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
            v = torch.from_numpy(inp.vals_bits.view(np.int16)).to(dev).view(torch.bfloat16)
            dy = dy.to(torch.bfloat16)
        else:
            x = torch.from_numpy(inp.x).to(dev)
            v = torch.from_numpy(inp.vals).to(dev)
        ws = torch.empty(K.ks_matmul_bwd_workspace_bytes(N, a, b, c, d, x.dtype), dtype=torch.uint8, device=dev)
        outs = dict(dx=torch.empty(N, a * b * d, device=dev), dvals=torch.empty(a, d, b, c, device=dev))
        ms, _ = timed(lambda: K.ks_matmul_bwd(x, v, dy, a, b, c, d, workspace=ws, outs=outs), args.steps, args.warmup)
        s_in = 4 if dtype == "f32" else 2
        flops = 2 * N * 2 * a * b * c * d
        byts = N * (s_in * (a * b * d + a * c * d) + 4 * a * b * d) + (s_in + 4) * a * b * c * d
        peak = PEAK_FP32_TFLOPS if dtype == "f32" else PEAK_BF16_TFLOPS
        t_flop, t_hbm = flops / (peak * 1e12), byts / (PEAK_HBM_GBS * 1e9)
        t_roof = max(t_flop, t_hbm)
        print(json.dumps({"workload": f"ks_matmul_bwd (a,b,c,d)=(2,48,192,4), 25216 rows, {dtype} inputs, dx and dvals",
                          "us_per_call": round(ms * 1e3, 2), "rows_per_s": round(N / (ms * 1e-3), 1),
                          "achieved_gbs": round(byts / (ms * 1e-3) / 1e9, 1),
                          "effective_tflops": round(flops / (ms * 1e-3) / 1e12, 3),
                          "t_roof_us": round(t_roof * 1e6, 2), "roofline_frac": round(t_roof / (ms * 1e-3), 4),
                          "bound": "hbm" if t_hbm >= t_flop else ("fp32" if dtype == "f32" else "bf16")}),
              flush=True)


def run_chain(args, dev):
    """Fused KS chains at 20,000 rows of 1024 values: the triple Kronecker product
    (8x8) (x) (16x16) (x) (8x8) as three factors, and a Monarch-style pair of 32x32-block
    factors.  Algorithmic work: sum over factors of 2*a*b*c*d flop per row; bytes: x read
    and y written once (4 * (in + out) per row)."""
    import torch
    import kronecker_factored_structured_amd as K
    rng = np.random.default_rng(70)
    A, B, C = (rng.standard_normal(s) / np.sqrt(s[0]) for s in ((8, 8), (16, 16), (8, 8)))
    # A (x) B (x) C = (A (x) I_128)(I_8 (x) B (x) I_8)(I_128 (x) C): each factor repeats its block
    kron3 = [(1, 8, 8, 128, np.broadcast_to(A, (1, 128, 8, 8))),
             (8, 16, 16, 8, np.broadcast_to(B, (8, 8, 16, 16))),
             (128, 8, 8, 1, np.broadcast_to(C, (128, 1, 8, 8)))]
    cases = {
        "triple Kronecker (8x8)(x)(16x16)(x)(8x8)": kron3,
        "Monarch pair, 32 blocks of 32x32 twice": [
            (32, 32, 32, 1, rng.standard_normal((32, 1, 32, 32)) / np.sqrt(32)),
            (1, 32, 32, 32, rng.standard_normal((1, 32, 32, 32)) / np.sqrt(32))],
    }
    N = 20000
    x = torch.from_numpy(rng.standard_normal((N, 1024)).astype(np.float32)).to(dev)
    y = torch.empty(N, 1024, device=dev)
    for name, fs in cases.items():
        tf = [(torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(dev), a, b, c, d) for (a, b, c, d, v) in fs]
        ms, _ = timed(lambda: K.ks_chain(x, tf, out=y), args.steps, args.warmup)
        flops = N * sum(2 * a * b * c * d for (a, b, c, d, _) in fs)
        byts = N * 4 * (1024 + 1024)
        t_flop, t_hbm = flops / (PEAK_FP32_TFLOPS * 1e12), byts / (PEAK_HBM_GBS * 1e9)
        t_roof = max(t_flop, t_hbm)
        print(json.dumps({"workload": f"ks_chain {name}, {N} rows, fp32", "us_per_call": round(ms * 1e3, 2),
                          "rows_per_s": round(N / (ms * 1e-3), 1), "achieved_gbs": round(byts / (ms * 1e-3) / 1e9, 1),
                          "effective_tflops": round(flops / (ms * 1e-3) / 1e12, 3), "t_roof_us": round(t_roof * 1e6, 2),
                          "roofline_frac": round(t_roof / (ms * 1e-3), 4),
                          "bound": "hbm" if t_hbm >= t_flop else "fp32"}), flush=True)


def run_van_loan(args, dev):
    """Van Loan rank-4 projection of a 1024 x 1024 W onto 32x32 (x) 32x32 factors: block
    subspace iteration of width 12, 8 power iterations.  Each iteration reads W twice
    (R Q and R^T Z); 2 * (iters + 1) reads of W's 4 MB are the algorithmic bytes."""
    import torch
    import kronecker_factored_structured_amd as K
    rng = np.random.default_rng(81)
    W = torch.from_numpy(rng.standard_normal((1024, 1024)).astype(np.float32)).to(dev)
    omega = torch.from_numpy(rng.standard_normal((1024, 12)).astype(np.float32)).to(dev)
    ws = torch.empty(int(K._lib.lib().kron_van_loan_workspace_bytes(32, 32, 32, 32, 12)), dtype=torch.uint8, device=dev)
    iters = 8
    ms, _ = timed(lambda: K.kron_van_loan(W, 32, 32, 32, 32, 4, omega, iters=iters, workspace=ws),
                  max(5, args.steps // 5), 2)
    byts = 2 * (iters + 1) * 4 * 1024 * 1024
    print(json.dumps({"workload": "van_loan: rank-4 projection of a 1024x1024 W, p=q=m=n=32, subspace 12, 8 iterations",
                      "us_per_call": round(ms * 1e3, 2), "achieved_gbs": round(byts / (ms * 1e-3) / 1e9, 1),
                      "t_roof_us": round(byts / (PEAK_HBM_GBS * 1e9) * 1e6, 2),
                      "roofline_frac": round(byts / (PEAK_HBM_GBS * 1e9) / (ms * 1e-3), 4), "bound": "hbm",
                      "limited_by": "latency: a dependent chain of 30 launches, the orthonormalisations and the "
                                    "Jacobi eigensolve on one compute unit each"}),
          flush=True)


def run_sweep(args, dev):
    """Batch-size sweep of the 1024 x 1024 layer (the tutorial's comparison): the Kronecker
    layer's fwd+bwd against a dense layer and a dense layer with the group-LASSO penalty
    on its m x n blocks (tutorial, "The baselines": the sum of the blocks' Frobenius norms,
    each norm sqrt(sum of squares + 1e-12)).  The dense sides are PyTorch matrix products
    (rocBLAS / hipBLASLt), timed as comparators only; nothing is dispatched to them."""
    import torch
    from workloads import kron_inputs
    steps = max(5, min(args.steps, 20))
    configs = [(32, 32, 32, 32, 4), (32, 32, 32, 32, 1), (16, 16, 64, 64, 2), (128, 128, 8, 8, 1),
               (128, 128, 8, 8, 2), (256, 256, 4, 4, 1), (256, 256, 4, 4, 2), (512, 512, 2, 2, 1)]
    lam = 1e-4
    for N in (256, 1024, 4096, 20000, 65536):
        rec = {"workload": f"sweep: 1024x1024 layer fwd+bwd, {N} rows", "N": N}
        for (p, q, m, n, r) in configs:
            inp = kron_inputs(70 + r, N, p, q, m, n, r, s_mode="uniform_zeroed", bias_mode="zeros")
            L = Layer(inp, dev)
            ms, _ = timed(lambda: (L.fwd(), L.bwd()), steps, 3)
            rec[f"kron p{p} m{m} r{r} us"] = round(ms * 1e3, 2)
            del L
        g = torch.Generator(device=dev).manual_seed(N)
        x = torch.randn(N, 1024, device=dev, generator=g)
        dy = torch.randn(N, 1024, device=dev, generator=g)
        W = torch.randn(1024, 1024, device=dev, generator=g) / 32.0
        bias = torch.zeros(1024, device=dev)
        y = torch.empty(N, 1024, device=dev)
        dx = torch.empty_like(x)
        dW = torch.empty_like(W)

        def dense():
            torch.addmm(bias, x, W, out=y)
            torch.mm(dy, W.t(), out=dx)
            torch.mm(x.t(), dy, out=dW)
            return dy.sum(0)

        def dense_lasso():
            db = dense()
            blocks = W.view(32, 32, 32, 32)   # in x out = (p, m) x (q, n) blocks of 32 x 32
            norms = (blocks.pow(2).sum(dim=(1, 3)) + 1e-12).sqrt()
            pen = lam * norms.sum()
            dW.view(32, 32, 32, 32).add_(blocks / norms[:, None, :, None], alpha=lam)
            return db, pen

        ms_d, _ = timed(dense, steps, 3)
        ms_l, _ = timed(dense_lasso, steps, 3)
        rec["dense us"] = round(ms_d * 1e3, 2)
        rec["dense+group-lasso us"] = round(ms_l * 1e3, 2)
        rec["kron r4 m32 speedup vs dense"] = round(ms_d / (rec["kron p32 m32 r4 us"] * 1e-3), 3)
        rec["kron r1 m8 speedup vs dense"] = round(ms_d / (rec["kron p128 m8 r1 us"] * 1e-3), 3)
        print(json.dumps(rec), flush=True)


def run_copy(args, dev):
    """Plain device-to-device copy of a known size (reference for the HBM counters)."""
    import torch
    nbytes = 1 << 30
    a = torch.empty(nbytes // 4, device=dev)
    b = torch.empty_like(a)
    a.fill_(1.0)
    for _ in range(args.steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read_per_copy": nbytes,
                      "bytes_written_per_copy": nbytes, "copies": args.steps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the copy and GEMM ceiling measurements")
    ap.add_argument("--workload", default="headline",
                    choices=("headline", "headline_bf16", "tiny", "mlp_step", "gpt2_ffn", "gpt2_ffn_bf16", "ks", "ks_bwd", "chain", "van_loan", "sweep", "small_blocks", "sparse_s"))
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--recompute-z", action="store_true",
                    help="headline: time the recomputing pair only (no saved Z)")
    ap.add_argument("--settle-seconds", type=float, default=1.0,
                    help="untimed running before the warmup steps, for the GPU clock to ramp up")
    args = ap.parse_args()
    SETTLE_SECONDS[0] = args.settle_seconds
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the Kronecker layer's hot path runs on one GPU's share "
              f"of rows); --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        raise SystemExit("no GPU visible")
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        return run_copy(args, dev)
    {"headline": run_headline, "headline_bf16": run_headline_bf16, "sparse_s": run_sparse_s, "tiny": run_tiny, "sweep": run_sweep, "small_blocks": run_small_blocks, "ks_bwd": run_ks_bwd, "chain": run_chain, "van_loan": run_van_loan, "mlp_step": run_mlp_step, "gpt2_ffn": run_gpt2, "gpt2_ffn_bf16": run_gpt2_bf16,
     "ks": run_ks}[args.workload](args, dev)


if __name__ == "__main__":
    main()
