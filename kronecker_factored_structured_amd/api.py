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
from ._lib import (KRON_ACCUMULATE, KRON_BF16, KRON_DX_RELU_MASK, KRON_F32, KRON_RELU_OUT, KRON_SPARSE_ROWS, KronShape,
                   check)


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


def _need(t: Optional[torch.Tensor], name: str, shape: tuple, dtype=torch.float32,
          device: Optional[torch.device] = None) -> None:
    """t (if given) must be a contiguous GPU tensor of exactly this shape and dtype (on
    `device` when one is given): libkron derives every extent from the sizes it is passed,
    so a tensor of another shape would be read or written past its end."""
    if t is None:
        return
    _dev(t, name, dtype)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def layer_shape(x_rows: int, S, A: torch.Tensor, B: torch.Tensor, flags: int = 0) -> KronShape:
    if A.dim() != 3 or B.dim() != 3:
        raise ValueError("A must be r x p x q and B r x m x n")
    r, p, q = A.shape
    rb, m, n = B.shape
    if rb != r:
        raise ValueError(f"A has rank {r} but B has rank {rb}")
    if S is not None and tuple(S.shape) != (p, q):
        raise ValueError(f"S must be {p}x{q}, got {tuple(S.shape)}")
    return KronShape(int(x_rows), p, q, m, n, r, flags)


def _layer_io_checks(x: torch.Tensor, shape: KronShape, S, A: torch.Tensor, B: torch.Tensor,
                     dy: Optional[torch.Tensor] = None) -> None:
    """x is N x p*m (and dy N x q*n), every tensor on x's device."""
    if x.dim() != 2 or x.shape[1] != shape.p * shape.m:
        raise ValueError(f"x must be N x {shape.p * shape.m}, got {tuple(x.shape)}")
    for t, nm in ((S, "S"), (A, "A"), (B, "B"), (dy, "dy")):
        if t is not None and t.device != x.device:
            raise ValueError(f"{nm} is on {t.device}, expected {x.device}")
    if dy is not None and tuple(dy.shape) != (x.shape[0], shape.q * shape.n):
        raise ValueError(f"dy must have shape {(x.shape[0], shape.q * shape.n)}, got {tuple(dy.shape)}")


def _grad_out_checks(o: dict, x: torch.Tensor, shape: KronShape, dx_dtype=torch.float32) -> None:
    """Caller-supplied gradient buffers: exact shapes, dx in dx_dtype, the rest fp32."""
    N, p, q, m, n, r = x.shape[0], shape.p, shape.q, shape.m, shape.n, shape.r
    _need(o.get("dx"), "dx", (N, p * m), dx_dtype, x.device)
    _need(o.get("dS"), "dS", (p, q), device=x.device)
    _need(o.get("dA"), "dA", (r, p, q), device=x.device)
    _need(o.get("dB"), "dB", (r, m, n), device=x.device)
    _need(o.get("dbias"), "dbias", (q * n,), device=x.device)


def _workspace(workspace: Optional[torch.Tensor], need: int, dev: torch.device) -> torch.Tensor:
    if workspace is not None:
        _dev(workspace, "workspace", torch.uint8)
        if workspace.device != dev:
            raise ValueError(f"workspace is on {workspace.device}, expected {dev}")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    return workspace


def kron_linear_bwd_workspace_bytes(shape: KronShape) -> int:
    return int(_lib.lib().kron_linear_bwd_workspace_bytes(ctypes.byref(shape)))


def kron_linear_zcache_bytes(shape: KronShape) -> int:
    """Bytes of the saved Z_i = X B_i cache for shape.N rows (0: no saved path for the shape)."""
    return int(_lib.lib().kron_linear_zcache_bytes(ctypes.byref(shape)))


def new_zcache(x: torch.Tensor, S: Optional[torch.Tensor], A: torch.Tensor, B: torch.Tensor) -> Optional[torch.Tensor]:
    """An uninitialised cache for kron_linear_fwd(..., zcache=) / kron_linear_bwd(..., zcache=)
    over x's rows, or None when the layer's shape has no saved-intermediate path."""
    nb = kron_linear_zcache_bytes(layer_shape(x.shape[0], S, A, B))
    return torch.empty(nb // 4, dtype=torch.float32, device=x.device) if nb > 0 else None


def _zcache_checks(zcache: torch.Tensor, shape: KronShape, device) -> int:
    _dev(zcache, "zcache")
    if zcache.device != device:
        raise ValueError(f"zcache is on {zcache.device}, expected {device}")
    need = kron_linear_zcache_bytes(shape)
    if need == 0 and shape.N > 0:
        raise ValueError("this layer shape has no saved-intermediate path (kron_linear_zcache_bytes is 0)")
    if zcache.numel() * 4 < need:
        raise ValueError(f"zcache holds {zcache.numel() * 4} bytes, {need} needed")
    return zcache.numel() * 4


def kron_linear_fwd(x: torch.Tensor, S: Optional[torch.Tensor], A: torch.Tensor, B: torch.Tensor,
                    bias: Optional[torch.Tensor] = None, relu: bool = False,
                    out: Optional[torch.Tensor] = None, sparse_rows: bool = False,
                    zcache: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = x W + bias with W = sum_i kron(S o A_i, B_i) (optionally ReLU-ed).  sparse_rows:
    S is expected to have whole rows zero; the forward then skips the 16-row tiles of C that
    hold only such rows (KRON_SPARSE_ROWS).  zcache (from new_zcache): also save Z_i = X B_i
    there for kron_linear_bwd(..., zcache=)."""
    for t, nm in ((x, "x"), (S, "S"), (A, "A"), (B, "B")):
        _dev(t, nm)
    shape = layer_shape(x.shape[0], S, A, B, (KRON_RELU_OUT if relu else 0) | (KRON_SPARSE_ROWS if sparse_rows else 0))
    _layer_io_checks(x, shape, S, A, B)
    _need(bias, "bias", (shape.q * shape.n,), device=x.device)
    _need(out, "out", (x.shape[0], shape.q * shape.n), device=x.device)
    y = out if out is not None else torch.empty(x.shape[0], shape.q * shape.n, device=x.device)
    if zcache is not None:
        nb = _zcache_checks(zcache, shape, x.device)
        check("kron_linear_fwd_save", _lib.lib().kron_linear_fwd_save(
            ctypes.byref(shape), _ptr(x), _ptr(S), _ptr(A), _ptr(B), _ptr(bias), _ptr(y), _ptr(zcache),
            ctypes.c_size_t(nb), _stream(x.device)))
        return y
    check("kron_linear_fwd", _lib.lib().kron_linear_fwd(
        ctypes.byref(shape), _ptr(x), _ptr(S), _ptr(A), _ptr(B), _ptr(bias), _ptr(y), _stream(x.device)))
    return y


def kron_linear_bwd(x: torch.Tensor, S: Optional[torch.Tensor], A: torch.Tensor, B: torch.Tensor,
                    dy: torch.Tensor, want_dx: bool = True, want_dbias: bool = True,
                    relu_mask: bool = False, workspace: Optional[torch.Tensor] = None,
                    outs: Optional[dict] = None, sparse_rows: bool = False,
                    zcache: Optional[torch.Tensor] = None) -> dict:
    """Gradients of sum(dy * (x W + bias)): dict(dx, dS, dA, dB, dbias) (None where not asked).
    sparse_rows: the KRON_SPARSE_ROWS hint (S expected to have whole rows zero).  zcache: the
    cache a kron_linear_fwd(..., zcache=) call filled for the same x and B; Z_i = X B_i is
    then read from it instead of recomputed."""
    for t, nm in ((x, "x"), (S, "S"), (A, "A"), (B, "B"), (dy, "dy")):
        _dev(t, nm)
    shape = layer_shape(x.shape[0], S, A, B,
                        (KRON_DX_RELU_MASK if relu_mask else 0) | (KRON_SPARSE_ROWS if sparse_rows else 0))
    _layer_io_checks(x, shape, S, A, B, dy)
    dev = x.device
    o = dict(outs or {})
    _grad_out_checks(o, x, shape)
    dx = o.get("dx") if "dx" in o else (torch.empty_like(x) if want_dx else None)
    dS = o.get("dS") if "dS" in o else (torch.empty_like(S) if S is not None else None)
    dA = o.get("dA") if "dA" in o else torch.empty_like(A)
    dB = o.get("dB") if "dB" in o else torch.empty_like(B)
    dbias = o.get("dbias") if "dbias" in o else (
        torch.empty(shape.q * shape.n, device=dev) if want_dbias else None)
    workspace = _workspace(workspace, kron_linear_bwd_workspace_bytes(shape), dev)
    if zcache is not None:
        nb = _zcache_checks(zcache, shape, dev)
        check("kron_linear_bwd_saved", _lib.lib().kron_linear_bwd_saved(
            ctypes.byref(shape), _ptr(x), _ptr(S), _ptr(A), _ptr(B), _ptr(dy), _ptr(zcache), ctypes.c_size_t(nb),
            _ptr(dx), _ptr(dS), _ptr(dA), _ptr(dB), _ptr(dbias), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
            _stream(dev)))
        return dict(dx=dx, dS=dS, dA=dA, dB=dB, dbias=dbias)
    check("kron_linear_bwd", _lib.lib().kron_linear_bwd(
        ctypes.byref(shape), _ptr(x), _ptr(S), _ptr(A), _ptr(B), _ptr(dy), _ptr(dx), _ptr(dS), _ptr(dA),
        _ptr(dB), _ptr(dbias), _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(dev)))
    return dict(dx=dx, dS=dS, dA=dA, dB=dB, dbias=dbias)


def kron_linear_bwd_noalloc(x: torch.Tensor, S: Optional[torch.Tensor], A: torch.Tensor, B: torch.Tensor,
                            dy: torch.Tensor, outs: dict, relu_mask: bool = False) -> dict:
    """kron_linear_bwd into caller-given buffers (outs: dx or None, dS, dA, dB, dbias or None)
    with the library's fixed scratch as workspace: the call allocates nothing."""
    for t, nm in ((x, "x"), (S, "S"), (A, "A"), (B, "B"), (dy, "dy")):
        _dev(t, nm)
    shape = layer_shape(x.shape[0], S, A, B, KRON_DX_RELU_MASK if relu_mask else 0)
    _layer_io_checks(x, shape, S, A, B, dy)
    o = dict(outs)
    _grad_out_checks(o, x, shape)
    dx, dS, dA, dB, dbias = (o.get(k) for k in ("dx", "dS", "dA", "dB", "dbias"))
    check("kron_linear_bwd_noalloc", _lib.lib().kron_linear_bwd_noalloc(
        ctypes.byref(shape), _ptr(x), _ptr(S), _ptr(A), _ptr(B), _ptr(dy), _ptr(dx), _ptr(dS), _ptr(dA),
        _ptr(dB), _ptr(dbias), _stream(x.device)))
    return dict(dx=dx, dS=dS, dA=dA, dB=dB, dbias=dbias)


def kron_linear_bwd_bf16_workspace_bytes(shape: KronShape) -> int:
    return int(_lib.lib().kron_linear_bwd_bf16_workspace_bytes(ctypes.byref(shape)))


def kron_linear_fwd_bf16(x: torch.Tensor, S: Optional[torch.Tensor], A: torch.Tensor, B: torch.Tensor,
                         bias: Optional[torch.Tensor] = None, relu: bool = False,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 layer: y = x W + bias (bf16 tensors, fp32 accumulation, bf16 y)."""
    bf = torch.bfloat16
    for t, nm in ((x, "x"), (S, "S"), (A, "A"), (B, "B")):
        _dev(t, nm, bf)
    shape = layer_shape(x.shape[0], S, A, B, KRON_RELU_OUT if relu else 0)
    _layer_io_checks(x, shape, S, A, B)
    _need(bias, "bias", (shape.q * shape.n,), bf, x.device)
    _need(out, "out", (x.shape[0], shape.q * shape.n), bf, x.device)
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
    _layer_io_checks(x, shape, S, A, B, dy)
    dev = x.device
    f32 = torch.float32
    o = dict(outs or {})
    _grad_out_checks(o, x, shape, bf)
    dx = o.get("dx") if "dx" in o else (torch.empty_like(x) if want_dx else None)
    dS = o.get("dS") if "dS" in o else (torch.empty(S.shape, device=dev, dtype=f32) if S is not None else None)
    dA = o.get("dA") if "dA" in o else torch.empty(A.shape, device=dev, dtype=f32)
    dB = o.get("dB") if "dB" in o else torch.empty(B.shape, device=dev, dtype=f32)
    dbias = o.get("dbias") if "dbias" in o else (
        torch.empty(shape.q * shape.n, device=dev, dtype=f32) if want_dbias else None)
    workspace = _workspace(workspace, kron_linear_bwd_bf16_workspace_bytes(shape), dev)
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
    if vals.device != x.device:
        raise ValueError(f"vals is on {vals.device}, expected {x.device}")
    return dt


def ks_matmul(x: torch.Tensor, vals: torch.Tensor, a: int, b: int, c: int, d: int,
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = X K for the Kronecker-sparse K with support I_a (x) 1_{b x c} (x) I_d; vals is
    a x d x b x c.  x and vals are float32 or bfloat16 (same dtype); y is float32."""
    dt = _ks_checks(x, vals, a, b, c, d)
    _need(out, "out", (x.shape[0], a * c * d), device=x.device)
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
    _need(out, "out", (x.shape[0], a * c * d), out_dtype, x.device)
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
    _need(dy, "dy", (x.shape[0], a * c * d), x.dtype, x.device)
    o = dict(outs or {})
    dev = x.device
    _need(o.get("dx"), "dx", tuple(x.shape), device=dev)
    if o.get("dvals") is not None:
        _dev(o["dvals"], "dvals")
        if o["dvals"].numel() != a * b * c * d or o["dvals"].device != dev:
            raise ValueError(f"dvals must hold a*b*c*d = {a * b * c * d} values on {dev}")
    dx = o.get("dx") if "dx" in o else (torch.empty(x.shape, device=dev) if want_dx else None)
    dv = o.get("dvals") if "dvals" in o else (torch.empty(a, d, b, c, device=dev) if want_dvals else None)
    workspace = _workspace(workspace, ks_matmul_bwd_workspace_bytes(x.shape[0], a, b, c, d, x.dtype), dev)
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
    width = x.shape[1]
    for i, (v, a, b, c, d) in enumerate(factors):
        _dev(v, "vals", x.dtype)
        if v.numel() != a * b * c * d:
            raise ValueError(f"factor {i}: vals must hold a*b*c*d = {a * b * c * d} values")
        if v.device != x.device:
            raise ValueError(f"factor {i}: vals is on {v.device}, expected {x.device}")
        if a * b * d != width:
            raise ValueError(f"factor {i}: input width a*b*d = {a * b * d} but the previous width is {width}")
        width = a * c * d
        arr[i] = _lib.KsFactor(a, b, c, d, _ptr(v))
    if not factors:
        width = 0
    _need(out, "out", (x.shape[0], width), device=x.device)
    y = out if out is not None else torch.empty(x.shape[0], width, device=x.device)
    check("ks_chain", _lib.lib().ks_chain(x.shape[0], len(factors), arr, dt, _ptr(x), _ptr(y), _stream(x.device)))
    return y


def kron_van_loan(W: torch.Tensor, p: int, q: int, m: int, n: int, r: int, omega: torch.Tensor,
                  iters: int = 8, workspace: Optional[torch.Tensor] = None) -> tuple:
    """Rank-r Van Loan factors (C [r,p,q], B [r,m,n], sigma [r]) of a dense W [p*m, q*n];
    omega [m*n, s] is the random starting block (its width s sets the subspace)."""
    _need(W, "W", (p * m, q * n))
    _dev(omega, "omega")
    if omega.dim() != 2 or omega.shape[0] != m * n or omega.device != W.device:
        raise ValueError(f"omega must be {m * n} x s on {W.device}")
    s = omega.shape[1]
    dev = W.device
    C = torch.empty(r, p, q, device=dev)
    B = torch.empty(r, m, n, device=dev)
    sigma = torch.empty(r, device=dev)
    workspace = _workspace(workspace, int(_lib.lib().kron_van_loan_workspace_bytes(p, q, m, n, s)), dev)
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
            if t.device != params[0].device:
                raise ValueError(f"{nm}[{i}] is on {t.device}, expected {params[0].device}")
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
    if h.dim() != 2 or W.dim() != 2:
        raise ValueError("h must be N x K and W K x C")
    N, K = h.shape
    C = W.shape[1]
    dev = h.device
    _need(W, "W", (K, C), device=dev)
    _need(b, "b", (C,), device=dev)
    _need(labels, "labels", (N,), torch.int64, dev)
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


def kron_relu_bwd(y: torch.Tensor, dy: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dy o [y > 0], the gradient through y = max(z, 0); out may be dy (in place)."""
    _dev(y, "y")
    _need(dy, "dy", tuple(y.shape), device=y.device)
    _need(out, "out", tuple(y.shape), device=y.device)
    o = out if out is not None else torch.empty_like(dy)
    check("kron_relu_bwd", _lib.lib().kron_relu_bwd(y.numel(), _ptr(y), _ptr(dy), _ptr(o), _stream(y.device)))
    return o


def kron_l1_penalty(tensors: Sequence[torch.Tensor], lam: float, loss: Optional[torch.Tensor] = None,
                    accumulate: bool = False) -> torch.Tensor:
    """lam * sum_t sum|t| into a 1-element device tensor (added to `loss` with accumulate)."""
    tensors = [t for t in tensors if t is not None]
    dev = loss.device if loss is not None else (tensors[0].device if tensors else None)
    if dev is None:
        raise ValueError("kron_l1_penalty needs a tensor or a loss buffer to place its result")
    for i, t in enumerate(tensors):
        _dev(t, f"tensors[{i}]")
        if t.device != dev:
            raise ValueError(f"tensors[{i}] is on {t.device}, expected {dev}")
    if loss is None:
        if accumulate:
            raise ValueError("accumulate needs a loss buffer")
        loss = torch.empty(1, device=dev)
    _need(loss, "loss", (1,), device=dev)
    nt = len(tensors)
    arr = (ctypes.c_void_p * max(nt, 1))(*[t.data_ptr() for t in tensors])
    n = (ctypes.c_int64 * max(nt, 1))(*[t.numel() for t in tensors])
    check("kron_l1_penalty", _lib.lib().kron_l1_penalty(nt, arr, n, float(lam), _ptr(loss),
                                                        KRON_ACCUMULATE if accumulate else 0, _stream(dev)))
    return loss


def kron_l1_penalty_grad(S: torch.Tensor, lam: float, g: torch.Tensor,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """lam * g * sign(S) for a 1-element device tensor g (the upstream gradient)."""
    _dev(S, "S")
    if g.numel() != 1:
        raise ValueError("g must hold one value")
    _dev(g, "g")
    if g.device != S.device:
        raise ValueError(f"g is on {g.device}, expected {S.device}")
    _need(out, "out", tuple(S.shape), device=S.device)
    o = out if out is not None else torch.empty_like(S)
    check("kron_l1_penalty_grad", _lib.lib().kron_l1_penalty_grad(S.numel(), _ptr(S), float(lam), _ptr(g), _ptr(o),
                                                                  _stream(S.device)))
    return o
