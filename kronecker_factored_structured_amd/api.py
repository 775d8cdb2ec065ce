"""Python binding of libkron over torch device tensors (argument marshalling only).

Every computation runs in libkron's HIP kernels; torch supplies device memory and the
current stream.  The functions carry the C ABI's names.  Inputs must be contiguous
tensors on a GPU; anything else raises (there is no CPU fallback).
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from . import _lib
from ._lib import KRON_BF16, KRON_DX_RELU_MASK, KRON_F32, KRON_RELU_OUT, KronShape, check


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: Optional[torch.Tensor], name: str, dtype=torch.float32) -> None:
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (libkron has no CPU path)")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def layer_shape(x_rows: int, S, A: torch.Tensor, B: torch.Tensor, flags: int = 0) -> KronShape:
    r, p, q = A.shape
    rb, m, n = B.shape
    if rb != r:
        raise ValueError(f"A has rank {r} but B has rank {rb}")
    if S is not None and tuple(S.shape) != (p, q):
        raise ValueError(f"S must be {p}x{q}, got {tuple(S.shape)}")
    return KronShape(int(x_rows), p, q, m, n, r, flags)


def kron_linear_bwd_workspace_bytes(shape: KronShape) -> int:
    return int(_lib.lib().kron_linear_bwd_workspace_bytes(ctypes.byref(shape)))


def kron_linear_fwd(x: torch.Tensor, S: Optional[torch.Tensor], A: torch.Tensor, B: torch.Tensor,
                    bias: Optional[torch.Tensor] = None, relu: bool = False,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = x W + bias with W = sum_i kron(S o A_i, B_i) (optionally ReLU-ed)."""
    for t, nm in ((x, "x"), (S, "S"), (A, "A"), (B, "B"), (bias, "bias"), (out, "out")):
        _dev(t, nm)
    shape = layer_shape(x.shape[0], S, A, B, KRON_RELU_OUT if relu else 0)
    if x.dim() != 2 or x.shape[1] != shape.p * shape.m:
        raise ValueError(f"x must be N x {shape.p * shape.m}")
    y = out if out is not None else torch.empty(x.shape[0], shape.q * shape.n, device=x.device)
    check("kron_linear_fwd", _lib.lib().kron_linear_fwd(
        ctypes.byref(shape), _ptr(x), _ptr(S), _ptr(A), _ptr(B), _ptr(bias), _ptr(y), _stream(x.device)))
    return y


def kron_linear_bwd(x: torch.Tensor, S: Optional[torch.Tensor], A: torch.Tensor, B: torch.Tensor,
                    dy: torch.Tensor, want_dx: bool = True, want_dbias: bool = True,
                    relu_mask: bool = False, workspace: Optional[torch.Tensor] = None,
                    outs: Optional[dict] = None) -> dict:
    """Gradients of sum(dy * (x W + bias)): dict(dx, dS, dA, dB, dbias) (None where not asked)."""
    for t, nm in ((x, "x"), (S, "S"), (A, "A"), (B, "B"), (dy, "dy")):
        _dev(t, nm)
    shape = layer_shape(x.shape[0], S, A, B, KRON_DX_RELU_MASK if relu_mask else 0)
    dev = x.device
    o = dict(outs or {})
    dx = o.get("dx") if "dx" in o else (torch.empty_like(x) if want_dx else None)
    dS = o.get("dS") if "dS" in o else (torch.empty_like(S) if S is not None else None)
    dA = o.get("dA") if "dA" in o else torch.empty_like(A)
    dB = o.get("dB") if "dB" in o else torch.empty_like(B)
    dbias = o.get("dbias") if "dbias" in o else (
        torch.empty(shape.q * shape.n, device=dev) if want_dbias else None)
    need = kron_linear_bwd_workspace_bytes(shape)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    check("kron_linear_bwd", _lib.lib().kron_linear_bwd(
        ctypes.byref(shape), _ptr(x), _ptr(S), _ptr(A), _ptr(B), _ptr(dy), _ptr(dx), _ptr(dS), _ptr(dA),
        _ptr(dB), _ptr(dbias), _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(dev)))
    return dict(dx=dx, dS=dS, dA=dA, dB=dB, dbias=dbias)


def kron_linear_bwd_bf16_workspace_bytes(shape: KronShape) -> int:
    return int(_lib.lib().kron_linear_bwd_bf16_workspace_bytes(ctypes.byref(shape)))


def kron_linear_fwd_bf16(x: torch.Tensor, S: Optional[torch.Tensor], A: torch.Tensor, B: torch.Tensor,
                         bias: Optional[torch.Tensor] = None, relu: bool = False,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 layer: y = x W + bias (bf16 tensors, fp32 accumulation, bf16 y)."""
    bf = torch.bfloat16
    for t, nm in ((x, "x"), (S, "S"), (A, "A"), (B, "B"), (bias, "bias"), (out, "out")):
        _dev(t, nm, bf)
    shape = layer_shape(x.shape[0], S, A, B, KRON_RELU_OUT if relu else 0)
    if x.dim() != 2 or x.shape[1] != shape.p * shape.m:
        raise ValueError(f"x must be N x {shape.p * shape.m}")
    y = out if out is not None else torch.empty(x.shape[0], shape.q * shape.n, device=x.device, dtype=bf)
    check("kron_linear_fwd_bf16", _lib.lib().kron_linear_fwd_bf16(
        ctypes.byref(shape), _ptr(x), _ptr(S), _ptr(A), _ptr(B), _ptr(bias), _ptr(y), _stream(x.device)))
    return y


def kron_linear_bwd_bf16(x: torch.Tensor, S: Optional[torch.Tensor], A: torch.Tensor, B: torch.Tensor,
                         dy: torch.Tensor, want_dx: bool = True, want_dbias: bool = True,
                         relu_mask: bool = False, workspace: Optional[torch.Tensor] = None,
                         outs: Optional[dict] = None) -> dict:
    """bf16 layer backward: dx bf16; dS, dA, dB, dbias fp32 (None where not asked)."""
    bf = torch.bfloat16
    for t, nm in ((x, "x"), (S, "S"), (A, "A"), (B, "B"), (dy, "dy")):
        _dev(t, nm, bf)
    shape = layer_shape(x.shape[0], S, A, B, KRON_DX_RELU_MASK if relu_mask else 0)
    dev = x.device
    f32 = torch.float32
    o = dict(outs or {})
    dx = o.get("dx") if "dx" in o else (torch.empty_like(x) if want_dx else None)
    dS = o.get("dS") if "dS" in o else (torch.empty(S.shape, device=dev, dtype=f32) if S is not None else None)
    dA = o.get("dA") if "dA" in o else torch.empty(A.shape, device=dev, dtype=f32)
    dB = o.get("dB") if "dB" in o else torch.empty(B.shape, device=dev, dtype=f32)
    dbias = o.get("dbias") if "dbias" in o else (
        torch.empty(shape.q * shape.n, device=dev, dtype=f32) if want_dbias else None)
    _dev(dx, "dx", bf)
    for t, nm in ((dS, "dS"), (dA, "dA"), (dB, "dB"), (dbias, "dbias")):
        _dev(t, nm)
    need = kron_linear_bwd_bf16_workspace_bytes(shape)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    check("kron_linear_bwd_bf16", _lib.lib().kron_linear_bwd_bf16(
        ctypes.byref(shape), _ptr(x), _ptr(S), _ptr(A), _ptr(B), _ptr(dy), _ptr(dx), _ptr(dS), _ptr(dA),
        _ptr(dB), _ptr(dbias), _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(dev)))
    return dict(dx=dx, dS=dS, dA=dA, dB=dB, dbias=dbias)


def _ks_checks(x, vals, a, b, c, d):
    if x.dtype == torch.float32:
        dt = KRON_F32
    elif x.dtype == torch.bfloat16:
        dt = KRON_BF16
    else:
        raise ValueError(f"unsupported dtype {x.dtype}")
    _dev(x, "x", x.dtype)
    _dev(vals, "vals", x.dtype)
    if x.dim() != 2 or x.shape[1] != a * b * d:
        raise ValueError(f"x must be N x {a * b * d}")
    if vals.numel() != a * b * c * d:
        raise ValueError(f"vals must hold a*b*c*d = {a * b * c * d} values")
    return dt


def ks_matmul(x: torch.Tensor, vals: torch.Tensor, a: int, b: int, c: int, d: int,
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = X K for the Kronecker-sparse K with support I_a (x) 1_{b x c} (x) I_d; vals is
    a x d x b x c.  x and vals are float32 or bfloat16 (same dtype); y is float32."""
    dt = _ks_checks(x, vals, a, b, c, d)
    _dev(out, "out")
    y = out if out is not None else torch.empty(x.shape[0], a * c * d, device=x.device)
    check("ks_matmul", _lib.lib().ks_matmul(x.shape[0], a, b, c, d, dt, _ptr(x), _ptr(vals), _ptr(y),
                                            _stream(x.device)))
    return y


def ks_matmul_out(x: torch.Tensor, vals: torch.Tensor, a: int, b: int, c: int, d: int,
                  out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """ks_matmul with y stored as out_dtype (float32, or bfloat16 rounded to nearest even
    from the fp32 accumulation)."""
    dt = _ks_checks(x, vals, a, b, c, d)
    if out_dtype == torch.float32:
        odt = KRON_F32
    elif out_dtype == torch.bfloat16:
        odt = KRON_BF16
    else:
        raise ValueError(f"unsupported output dtype {out_dtype}")
    _dev(out, "out", out_dtype)
    y = out if out is not None else torch.empty(x.shape[0], a * c * d, device=x.device, dtype=out_dtype)
    check("ks_matmul_out", _lib.lib().ks_matmul_out(x.shape[0], a, b, c, d, dt, odt, _ptr(x), _ptr(vals),
                                                    _ptr(y), _stream(x.device)))
    return y


def ks_matmul_bwd_workspace_bytes(N: int, a: int, b: int, c: int, d: int, dtype: torch.dtype = torch.float32) -> int:
    dt = KRON_F32 if dtype == torch.float32 else KRON_BF16
    return int(_lib.lib().ks_matmul_bwd_workspace_bytes(N, a, b, c, d, dt))


def ks_matmul_bwd(x: torch.Tensor, vals: torch.Tensor, dy: torch.Tensor, a: int, b: int, c: int, d: int,
                  want_dx: bool = True, want_dvals: bool = True, workspace: Optional[torch.Tensor] = None,
                  outs: Optional[dict] = None) -> dict:
    """Gradients of ks_matmul: dx = dy K^T and dvals (fp32), from x, vals, dy of one dtype."""
    dt = _ks_checks(x, vals, a, b, c, d)
    _dev(dy, "dy", x.dtype)
    if dy.dim() != 2 or dy.shape != (x.shape[0], a * c * d):
        raise ValueError(f"dy must be N x {a * c * d}")
    o = dict(outs or {})
    dev = x.device
    dx = o.get("dx") if "dx" in o else (torch.empty(x.shape, device=dev) if want_dx else None)
    dv = o.get("dvals") if "dvals" in o else (torch.empty(a, d, b, c, device=dev) if want_dvals else None)
    _dev(dx, "dx")
    _dev(dv, "dvals")
    need = ks_matmul_bwd_workspace_bytes(x.shape[0], a, b, c, d, x.dtype)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    check("ks_matmul_bwd", _lib.lib().ks_matmul_bwd(
        x.shape[0], a, b, c, d, dt, _ptr(x), _ptr(vals), _ptr(dy), _ptr(dx), _ptr(dv), _ptr(workspace),
        ctypes.c_size_t(workspace.numel()), _stream(dev)))
    return dict(dx=dx, dvals=dv)


def ks_chain(x: torch.Tensor, factors: Sequence, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Fused y = x K_1 ... K_n; factors is a sequence of (vals, a, b, c, d) with vals
    a x d x b x c in x's dtype (float32 or bfloat16); y is float32."""
    if x.dtype == torch.float32:
        dt = KRON_F32
    elif x.dtype == torch.bfloat16:
        dt = KRON_BF16
    else:
        raise ValueError(f"unsupported dtype {x.dtype}")
    _dev(x, "x", x.dtype)
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    arr = (_lib.KsFactor * max(len(factors), 1))()
    for i, (v, a, b, c, d) in enumerate(factors):
        _dev(v, "vals", x.dtype)
        if v.numel() != a * b * c * d:
            raise ValueError(f"factor {i}: vals must hold a*b*c*d = {a * b * c * d} values")
        arr[i] = _lib.KsFactor(a, b, c, d, _ptr(v))
    if factors:
        v, a, b, c, d = factors[-1]
        width = a * c * d
    else:
        width = 0
    _dev(out, "out")
    y = out if out is not None else torch.empty(x.shape[0], width, device=x.device)
    check("ks_chain", _lib.lib().ks_chain(x.shape[0], len(factors), arr, dt, _ptr(x), _ptr(y), _stream(x.device)))
    return y


def kron_van_loan(W: torch.Tensor, p: int, q: int, m: int, n: int, r: int, omega: torch.Tensor,
                  iters: int = 8, workspace: Optional[torch.Tensor] = None) -> tuple:
    """Rank-r Van Loan factors (C [r,p,q], B [r,m,n], sigma [r]) of a dense W [p*m, q*n];
    omega [m*n, s] is the random starting block (its width s sets the subspace)."""
    _dev(W, "W")
    _dev(omega, "omega")
    if W.shape != (p * m, q * n):
        raise ValueError(f"W must be {p * m} x {q * n}")
    if omega.dim() != 2 or omega.shape[0] != m * n:
        raise ValueError(f"omega must be {m * n} x s")
    s = omega.shape[1]
    dev = W.device
    C = torch.empty(r, p, q, device=dev)
    B = torch.empty(r, m, n, device=dev)
    sigma = torch.empty(r, device=dev)
    need = int(_lib.lib().kron_van_loan_workspace_bytes(p, q, m, n, s))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    check("kron_van_loan", _lib.lib().kron_van_loan(p, q, m, n, r, s, iters, _ptr(W), _ptr(omega), _ptr(C), _ptr(B),
                                                    _ptr(sigma), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
                                                    _stream(dev)))
    return C, B, sigma


def kron_adam_l1_step(params: Sequence[torch.Tensor], grads: Sequence[torch.Tensor],
                      m: Sequence[torch.Tensor], v: Sequence[torch.Tensor], step: int, lr: float,
                      beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
                      l1: Optional[Sequence[float]] = None) -> None:
    """One fused Adam (+ l1 subgradient) update of every tensor, in place."""
    nt = len(params)
    if not (len(grads) == len(m) == len(v) == nt) or (l1 is not None and len(l1) != nt):
        raise ValueError("params, grads, m, v (and l1) must have the same length")
    for i in range(nt):
        for t, nm in ((params[i], "param"), (grads[i], "grad"), (m[i], "m"), (v[i], "v")):
            _dev(t, f"{nm}[{i}]")
            if t.numel() != params[i].numel():
                raise ValueError(f"tensor {i}: sizes differ")
    if nt == 0:
        return
    arr = ctypes.c_void_p * nt
    P = arr(*[t.data_ptr() for t in params])
    G = arr(*[t.data_ptr() for t in grads])
    M = arr(*[t.data_ptr() for t in m])
    V = arr(*[t.data_ptr() for t in v])
    n = (ctypes.c_int64 * nt)(*[t.numel() for t in params])
    L = (ctypes.c_float * nt)(*(l1 if l1 is not None else [0.0] * nt))
    check("kron_adam_l1_step", _lib.lib().kron_adam_l1_step(
        nt, P, G, M, V, n, L, int(step), float(lr), float(beta1), float(beta2), float(eps),
        _stream(params[0].device)))


def kron_head_ce(h: torch.Tensor, W: torch.Tensor, b: torch.Tensor, labels: torch.Tensor,
                 want_dh: bool = True, relu_mask: bool = False) -> dict:
    """Dense head + mean softmax cross-entropy, forward and backward in one call:
    dict(loss (1-element tensor), dh, dW, db)."""
    _dev(h, "h")
    _dev(W, "W")
    _dev(b, "b")
    _dev(labels, "labels", torch.int64)
    N, K = h.shape
    C = W.shape[1]
    dev = h.device
    loss = torch.empty(1, device=dev)
    dh = torch.empty_like(h) if want_dh else None
    dW = torch.empty_like(W)
    db = torch.empty_like(b)
    need = int(_lib.lib().kron_head_ce_workspace_bytes(N, K, C))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    check("kron_head_ce", _lib.lib().kron_head_ce(
        N, K, C, _ptr(h), _ptr(W), _ptr(b), _ptr(labels), _ptr(loss), _ptr(dh), _ptr(dW), _ptr(db),
        KRON_DX_RELU_MASK if relu_mask else 0, _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev)))
    return dict(loss=loss, dh=dh, dW=dW, db=db)
