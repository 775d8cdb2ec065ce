"""The C-ABI library loads, exports every symbol include/kron.h declares, and rejects
bad arguments on the host before any HIP call (CPU only: no compute calls)."""
import ctypes
import os
import re

import pytest

from kronecker_factored_structured_amd import _lib
from kronecker_factored_structured_amd._lib import KronShape

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kron.h")

# Fake, never-dereferenced device addresses: validation fails before any HIP call.
BASE = 0x7f0000000000


def P(off=0):
    return ctypes.c_void_p(BASE + off)


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_python_exports():
    assert set(header_functions()) == set(_lib.EXPORTS)


def test_library_loads_and_exports_every_symbol():
    L = _lib.lib()
    for name in header_functions():
        assert hasattr(L, name), name
    assert L.kron_abi_version() == 1
    assert _lib.status_str(0) == "ok"
    assert _lib.status_str(_lib.KRON_E_WORKSPACE) == "workspace missing or too small"


def check(shape):
    return _lib.lib().kron_linear_check(ctypes.byref(shape))


def test_shape_validation():
    assert check(KronShape(20000, 32, 32, 32, 32, 4, 0)) == 0
    assert check(KronShape(0, 1, 1, 1, 1, 1, 0)) == 0
    assert check(KronShape(-1, 32, 32, 32, 32, 4, 0)) == _lib.KRON_E_SHAPE
    assert check(KronShape(10, 0, 32, 32, 32, 4, 0)) == _lib.KRON_E_SHAPE
    assert check(KronShape(10, 32, 32, 32, 32, 0, 0)) == _lib.KRON_E_SHAPE
    assert check(KronShape(10, 32, 32, 32, 32, 65, 0)) == _lib.KRON_E_UNSUPPORTED
    assert check(KronShape(10, 4096, 32, 32, 32, 1, 0)) == _lib.KRON_E_UNSUPPORTED  # in > 65536
    # the tutorial's 1024 x 1024 layer: 16 x 16 blocks fit the generic kernels' LDS; 8 x 8,
    # 4 x 4 and 2 x 2 blocks (p = q = 128, 256, 512) take the small-block matrix-core path
    # up to rank 16, beyond which only 8 x 8 blocks (S and C_i of 128 x 128) still fit the
    # generic kernels; blocks smaller than 16 x 16 need p and q multiples of 16
    assert check(KronShape(256, 128, 128, 8, 8, 1, 0)) == 0
    assert check(KronShape(256, 64, 64, 16, 16, 4, 0)) == 0
    assert check(KronShape(256, 256, 256, 4, 4, 1, 0)) == 0
    assert check(KronShape(256, 512, 512, 2, 2, 16, 0)) == 0
    assert check(KronShape(256, 128, 128, 8, 8, 17, 0)) == 0
    assert check(KronShape(256, 256, 256, 4, 4, 17, 0)) == _lib.KRON_E_UNSUPPORTED
    assert check(KronShape(256, 250, 256, 4, 4, 1, 0)) == _lib.KRON_E_UNSUPPORTED
    assert check(KronShape(10, 32, 32, 32, 32, 4, 8)) == _lib.KRON_E_ARG           # unknown flag
    assert "flag" in _lib.last_error()
    assert _lib.lib().kron_linear_check(None) == _lib.KRON_E_NULL


def test_workspace_size_depends_on_shape_only():
    L = _lib.lib()
    s = KronShape(20000, 32, 32, 32, 32, 4, 0)
    w = L.kron_linear_bwd_workspace_bytes(ctypes.byref(s))
    assert w > 0 and w % 256 == 0
    assert L.kron_linear_bwd_workspace_bytes(ctypes.byref(s)) == w
    assert L.kron_linear_bwd_workspace_bytes(ctypes.byref(KronShape(-1, 1, 1, 1, 1, 1, 0))) == 0


def test_small_block_workspace():
    """The small-block backward's workspace holds its two partial arrays (dB rows, then
    dC and dbias rows of r*p*q + q*n floats); it grows with N only up to the row-group cap."""
    L = _lib.lib()
    ws = lambda N, p, m, r: L.kron_linear_bwd_workspace_bytes(ctypes.byref(KronShape(N, p, p, m, m, r, 0)))
    for p, m in ((128, 8), (256, 4), (512, 2)):
        w = ws(20000, p, m, 1)
        assert w > 0 and w % 256 == 0
        assert w >= 8 * (p * p + p * m) * 4            # at least 8 row groups of dC + dbias
        assert ws(0, p, m, 1) > 0                        # an empty batch still writes zero partials
        assert ws(10 ** 6, p, m, 1) == ws(2 * 10 ** 6, p, m, 1)
    # more ranks mean more dC tiles per row group and so fewer row groups: the partial
    # storage stays near 512 workgroups' worth
    assert 0.5 < ws(20000, 128, 8, 2) / ws(20000, 128, 8, 1) < 2


def fwd(shape, x, S, A, B, bias, y):
    return _lib.lib().kron_linear_fwd(ctypes.byref(shape), x, S, A, B, bias, y, None)


def test_fwd_argument_errors():
    s = KronShape(4, 2, 2, 2, 2, 1, 0)
    MB = 1 << 20
    assert fwd(s, P(0), None, None, P(2 * MB), None, P(3 * MB)) == _lib.KRON_E_NULL
    assert fwd(s, None, None, P(MB), P(2 * MB), None, P(3 * MB)) == _lib.KRON_E_NULL
    assert fwd(s, P(4), None, P(MB), P(2 * MB), None, P(3 * MB)) == _lib.KRON_E_ALIGN
    assert fwd(s, P(0), None, P(MB), P(2 * MB), None, P(16)) == _lib.KRON_E_ALIAS   # y overlaps x
    assert "overlaps" in _lib.last_error()
    s2 = KronShape(4, 2, 2, 2, 2, 1, _lib.KRON_DX_RELU_MASK)
    assert fwd(s2, P(0), None, P(MB), P(2 * MB), None, P(3 * MB)) == _lib.KRON_E_ARG
    # N == 0 is a valid no-op and launches nothing
    s0 = KronShape(0, 2, 2, 2, 2, 1, 0)
    assert fwd(s0, None, None, P(MB), P(2 * MB), None, None) == 0


def bwd(shape, x, S, A, B, dy, dx, dS, dA, dB, dbias, ws, wsb):
    return _lib.lib().kron_linear_bwd(ctypes.byref(shape), x, S, A, B, dy, dx, dS, dA, dB, dbias, ws,
                                      ctypes.c_size_t(wsb), None)


def test_bwd_argument_errors():
    MB = 1 << 20
    s = KronShape(4, 2, 2, 2, 2, 1, 0)
    need = _lib.lib().kron_linear_bwd_workspace_bytes(ctypes.byref(s))
    args = dict(x=P(0), S=P(MB), A=P(2 * MB), B=P(3 * MB), dy=P(4 * MB), dx=P(5 * MB), dS=P(6 * MB),
                dA=P(7 * MB), dB=P(8 * MB), dbias=P(9 * MB), ws=P(10 * MB), wsb=need)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return bwd(s, **a)

    assert call(dS=None) == _lib.KRON_E_NULL                  # S given but no dS
    assert call(S=None) == _lib.KRON_E_NULL                   # dS given but no S
    assert call(dA=None) == _lib.KRON_E_NULL
    assert call(ws=None) == _lib.KRON_E_WORKSPACE
    assert call(wsb=need - 1) == _lib.KRON_E_WORKSPACE
    assert call(ws=P(10 * MB + 16)) == _lib.KRON_E_ALIGN      # workspace must be 256-B aligned
    assert call(dx=P(4 * MB)) == _lib.KRON_E_ALIAS            # dx overlaps dy
    assert call(dB=P(7 * MB)) == _lib.KRON_E_ALIAS            # two outputs overlap
    assert call(dA=P(10 * MB)) == _lib.KRON_E_ALIAS           # output overlaps workspace
    sr = KronShape(4, 2, 2, 2, 2, 1, _lib.KRON_RELU_OUT)
    a = dict(args)
    assert bwd(sr, **a) == _lib.KRON_E_ARG
    sm = KronShape(4, 2, 2, 2, 2, 1, _lib.KRON_DX_RELU_MASK)
    a["dx"] = None
    assert bwd(sm, **a) == _lib.KRON_E_ARG


def test_bf16_argument_errors():
    """bf16 layer: unsupported shapes and bad arguments are refused on the host, before any
    HIP call (fake device addresses are never dereferenced)."""
    L = _lib.lib()
    MB = 1 << 20
    bad = KronShape(8, 32, 32, 20, 20, 1, 0)   # m = 20: no bf16 kernel
    gpt2 = KronShape(8, 32, 64, 24, 48, 1, 0)  # m = 24 runs padded to 32
    assert L.kron_linear_bwd_bf16_workspace_bytes(ctypes.byref(gpt2)) > 0
    assert L.kron_linear_fwd_bf16(ctypes.byref(bad), P(0), None, P(MB), P(2 * MB), None, P(3 * MB), None) == \
        _lib.KRON_E_UNSUPPORTED
    assert L.kron_linear_bwd_bf16_workspace_bytes(ctypes.byref(bad)) == 0
    s = KronShape(8, 32, 32, 32, 32, 4, 0)
    need = L.kron_linear_bwd_bf16_workspace_bytes(ctypes.byref(s))
    assert need > 0 and need % 256 == 0
    assert L.kron_linear_fwd_bf16(ctypes.byref(s), P(4), None, P(MB), P(2 * MB), None, P(3 * MB), None) == \
        _lib.KRON_E_ALIGN
    assert L.kron_linear_fwd_bf16(ctypes.byref(s), P(0), None, P(MB), P(2 * MB), None, P(16), None) == \
        _lib.KRON_E_ALIAS
    args = [P(0), None, P(MB), P(2 * MB), P(3 * MB), P(4 * MB), None, P(5 * MB), P(6 * MB), P(7 * MB), P(8 * MB)]
    assert L.kron_linear_bwd_bf16(ctypes.byref(s), *args, ctypes.c_size_t(need - 1), None) == _lib.KRON_E_WORKSPACE
    args_ds = list(args)
    args_ds[6] = P(9 * MB)   # dS without S
    assert L.kron_linear_bwd_bf16(ctypes.byref(s), *args_ds, ctypes.c_size_t(need), None) == _lib.KRON_E_NULL


def test_ks_argument_errors():
    L = _lib.lib()
    MB = 1 << 20
    assert L.ks_matmul(-1, 2, 48, 192, 4, 0, P(0), P(MB), P(2 * MB), None) == _lib.KRON_E_SHAPE
    assert L.ks_matmul(8, 0, 48, 192, 4, 0, P(0), P(MB), P(2 * MB), None) == _lib.KRON_E_SHAPE
    assert L.ks_matmul(8, 2, 48, 192, 4, 7, P(0), P(MB), P(2 * MB), None) == _lib.KRON_E_DTYPE
    assert L.ks_matmul(8, 2, 48, 192, 4, 0, P(0), None, P(2 * MB), None) == _lib.KRON_E_NULL
    assert L.ks_matmul(8, 2, 48, 192, 4, 0, P(2), P(MB), P(2 * MB), None) == _lib.KRON_E_ALIGN
    assert L.ks_matmul(8, 2, 48, 192, 4, 0, P(0), P(MB), P(64), None) == _lib.KRON_E_ALIAS
    assert L.ks_matmul(8, 2, 48, 65536, 4, 0, P(0), P(MB), P(2 * MB), None) == _lib.KRON_E_UNSUPPORTED
    assert L.ks_matmul(0, 2, 48, 192, 4, 1, None, P(MB), None, None) == 0


def test_ks_out_argument_errors():
    L = _lib.lib()
    MB = 1 << 20
    assert L.ks_matmul_out(8, 2, 48, 192, 4, 0, 7, P(0), P(MB), P(2 * MB), None) == _lib.KRON_E_DTYPE
    assert L.ks_matmul_out(8, 2, 48, 192, 4, 7, 1, P(0), P(MB), P(2 * MB), None) == _lib.KRON_E_DTYPE
    assert L.ks_matmul_out(8, 2, 48, 192, 4, 1, 1, P(0), None, P(2 * MB), None) == _lib.KRON_E_NULL
    assert L.ks_matmul_out(8, 2, 48, 192, 4, 1, 1, P(0), P(MB), P(2 * MB + 8), None) == _lib.KRON_E_ALIGN
    # bf16 x of 8 x 384 occupies [0, 6 KiB); a bf16 y (8 x 1536, 24 KiB) from 4 KiB overlaps it
    assert L.ks_matmul_out(8, 2, 48, 192, 4, 1, 1, P(0), P(MB), P(4096), None) == _lib.KRON_E_ALIAS
    assert L.ks_matmul_out(0, 2, 48, 192, 4, 1, 1, None, P(MB), None, None) == 0


def test_ks_bwd_argument_errors():
    L = _lib.lib()
    MB = 1 << 20
    need = L.ks_matmul_bwd_workspace_bytes(8, 2, 48, 192, 4, 0)
    assert need > 0
    assert L.ks_matmul_bwd_workspace_bytes(8, 2, 48, 192, 4, 7) == 0
    assert L.ks_matmul_bwd_workspace_bytes(-1, 2, 48, 192, 4, 0) == 0
    args = lambda **kw: [kw.get("x", P(0)), kw.get("vals", P(MB)), kw.get("dy", P(2 * MB)), kw.get("dx", P(3 * MB)),
                         kw.get("dv", P(4 * MB)), kw.get("ws", P(8 * MB)), ctypes.c_size_t(kw.get("bytes", need)), None]
    assert L.ks_matmul_bwd(8, 2, 48, 192, 4, 7, *args()) == _lib.KRON_E_DTYPE
    assert L.ks_matmul_bwd(-1, 2, 48, 192, 4, 0, *args()) == _lib.KRON_E_SHAPE
    assert L.ks_matmul_bwd(8, 2, 48, 192, 4, 0, *args(vals=None)) == _lib.KRON_E_NULL
    assert L.ks_matmul_bwd(8, 2, 48, 192, 4, 0, *args(dy=None)) == _lib.KRON_E_NULL
    assert L.ks_matmul_bwd(8, 2, 48, 192, 4, 0, *args(x=None)) == _lib.KRON_E_NULL
    assert L.ks_matmul_bwd(8, 2, 48, 192, 4, 0, *args(bytes=need - 1)) == _lib.KRON_E_WORKSPACE
    assert L.ks_matmul_bwd(8, 2, 48, 192, 4, 0, *args(ws=P(8 * MB + 16))) == _lib.KRON_E_ALIGN
    assert L.ks_matmul_bwd(8, 2, 48, 192, 4, 0, *args(dx=P(3 * MB + 4))) == _lib.KRON_E_ALIGN
    assert L.ks_matmul_bwd(8, 2, 48, 192, 4, 0, *args(dv=P(2 * MB))) == _lib.KRON_E_ALIAS   # dvals over dy
    assert L.ks_matmul_bwd(8, 2, 48, 192, 4, 0, *args(dx=P(8 * MB))) == _lib.KRON_E_ALIAS   # dx over workspace
    assert L.ks_matmul_bwd(8, 2, 48, 192, 4, 0, *args(dx=None, dv=None)) == 0              # nothing asked
    assert L.ks_matmul_bwd(8, 1, 65536, 65536, 1, 0, *args()) == _lib.KRON_E_UNSUPPORTED    # a*b*c*d > 2^28


def test_ks_chain_argument_errors():
    L = _lib.lib()
    MB = 1 << 20
    F = _lib.KsFactor
    two = (F * 2)(F(2, 3, 4, 2, P(MB)), F(4, 2, 3, 2, P(2 * MB)))   # 12 -> 16 -> 24
    assert L.ks_chain(8, 0, two, 0, P(0), P(4 * MB), None) == _lib.KRON_E_ARG
    assert L.ks_chain(8, 9, two, 0, P(0), P(4 * MB), None) == _lib.KRON_E_ARG
    assert L.ks_chain(8, 2, None, 0, P(0), P(4 * MB), None) == _lib.KRON_E_NULL
    assert L.ks_chain(8, 2, two, 7, P(0), P(4 * MB), None) == _lib.KRON_E_DTYPE
    bad = (F * 2)(F(2, 3, 4, 2, P(MB)), F(4, 3, 3, 2, P(2 * MB)))   # 16 given, 24 taken
    assert L.ks_chain(8, 2, bad, 0, P(0), P(4 * MB), None) == _lib.KRON_E_SHAPE
    nul = (F * 2)(F(2, 3, 4, 2, P(MB)), F(4, 2, 3, 2, None))
    assert L.ks_chain(8, 2, nul, 0, P(0), P(4 * MB), None) == _lib.KRON_E_NULL
    wide = (F * 1)(F(1, 1, 20000, 1, P(MB)))
    assert L.ks_chain(8, 1, wide, 0, P(0), P(4 * MB), None) == _lib.KRON_E_UNSUPPORTED
    assert L.ks_chain(8, 2, two, 0, P(0), P(2 * MB), None) == _lib.KRON_E_ALIAS        # y over vals
    assert L.ks_chain(8, 2, two, 0, P(8), P(4 * MB), None) == _lib.KRON_E_ALIGN
    assert L.ks_chain(0, 2, two, 0, None, None, None) == 0


def test_van_loan_argument_errors():
    L = _lib.lib()
    MB = 1 << 20
    need = L.kron_van_loan_workspace_bytes(32, 32, 32, 32, 12)
    assert need > 0
    assert L.kron_van_loan_workspace_bytes(32, 32, 32, 32, 33) == 0          # s > 32
    assert L.kron_van_loan_workspace_bytes(128, 128, 4, 4, 12) == 0          # p*q > 8192
    ok = lambda **kw: [kw.get("W", P(0)), kw.get("om", P(8 * MB)), kw.get("C", P(9 * MB)), kw.get("B", P(10 * MB)),
                       kw.get("sig", P(11 * MB)), kw.get("ws", P(12 * MB)), ctypes.c_size_t(kw.get("bytes", need)), None]
    assert L.kron_van_loan(32, 32, 32, 32, 4, 12, 8, *ok(W=None)) == _lib.KRON_E_NULL
    assert L.kron_van_loan(0, 32, 32, 32, 4, 12, 8, *ok()) == _lib.KRON_E_SHAPE
    assert L.kron_van_loan(32, 32, 32, 32, 13, 12, 8, *ok()) == _lib.KRON_E_ARG      # r > s
    assert L.kron_van_loan(32, 32, 32, 32, 4, 12, 101, *ok()) == _lib.KRON_E_ARG     # iters
    assert L.kron_van_loan(2, 2, 32, 32, 2, 5, 8, *ok()) == _lib.KRON_E_ARG          # s > p*q
    assert L.kron_van_loan(32, 32, 32, 32, 4, 12, 8, *ok(bytes=need - 1)) == _lib.KRON_E_WORKSPACE
    assert L.kron_van_loan(32, 32, 32, 32, 4, 12, 8, *ok(ws=P(12 * MB + 64))) == _lib.KRON_E_ALIGN
    assert L.kron_van_loan(32, 32, 32, 32, 4, 12, 8, *ok(C=P(8))) == _lib.KRON_E_ALIGN
    assert L.kron_van_loan(32, 32, 32, 32, 4, 12, 8, *ok(C=P(MB))) == _lib.KRON_E_ALIAS   # C over W


def test_adam_argument_errors():
    L = _lib.lib()
    arr = ctypes.c_void_p * 1
    p, g, m, v = arr(BASE), arr(BASE + (1 << 20)), arr(BASE + (2 << 20)), arr(BASE + (3 << 20))
    n = (ctypes.c_int64 * 1)(10)
    assert L.kron_adam_l1_step(0, None, None, None, None, None, None, 1, 1e-3, 0.9, 0.999, 1e-8, None) == 0
    assert L.kron_adam_l1_step(1, p, g, m, v, n, None, 0, 1e-3, 0.9, 0.999, 1e-8, None) == _lib.KRON_E_ARG
    assert L.kron_adam_l1_step(1, p, g, m, v, n, None, 1, 1e-3, 1.0, 0.999, 1e-8, None) == _lib.KRON_E_ARG
    assert L.kron_adam_l1_step(1, None, g, m, v, n, None, 1, 1e-3, 0.9, 0.999, 1e-8, None) == _lib.KRON_E_NULL
    m2 = arr(BASE + 8)
    assert L.kron_adam_l1_step(1, p, g, m2, v, n, None, 1, 1e-3, 0.9, 0.999, 1e-8, None) == _lib.KRON_E_ALIGN
    m3 = arr(BASE + 16)      # m overlaps the parameter
    assert L.kron_adam_l1_step(1, p, g, m3, v, n, None, 1, 1e-3, 0.9, 0.999, 1e-8, None) == _lib.KRON_E_ALIAS


def test_head_argument_errors():
    L = _lib.lib()
    MB = 1 << 20
    need = L.kron_head_ce_workspace_bytes(100, 1024, 10)
    assert need > 0
    args = [100, 1024, 10, P(0), P(MB), P(2 * MB), P(3 * MB), P(4 * MB), P(5 * MB), P(6 * MB), P(7 * MB), 0,
            P(8 * MB), ctypes.c_size_t(need), None]
    bad = list(args); bad[2] = 65
    assert L.kron_head_ce(*bad) == _lib.KRON_E_UNSUPPORTED
    bad = list(args); bad[13] = ctypes.c_size_t(need - 1)
    assert L.kron_head_ce(*bad) == _lib.KRON_E_WORKSPACE
    bad = list(args); bad[11] = 1
    assert L.kron_head_ce(*bad) == _lib.KRON_E_ARG
    bad = list(args); bad[7] = None
    assert L.kron_head_ce(*bad) == _lib.KRON_E_NULL
    bad = list(args); bad[8] = P(0)   # dh overlaps h
    assert L.kron_head_ce(*bad) == _lib.KRON_E_ALIAS


def test_relu_bwd_and_l1_argument_errors():
    L = _lib.lib()
    MB = 1 << 20
    assert L.kron_relu_bwd(0, None, None, None, None) == 0                     # nothing to do
    assert L.kron_relu_bwd(-1, P(0), P(MB), P(2 * MB), None) == _lib.KRON_E_SHAPE
    assert L.kron_relu_bwd(10, None, P(MB), P(2 * MB), None) == _lib.KRON_E_NULL
    assert L.kron_relu_bwd(10, P(4), P(MB), P(2 * MB), None) == _lib.KRON_E_ALIGN
    assert L.kron_relu_bwd(10, P(0), P(MB), P(16), None) == _lib.KRON_E_ALIAS      # out over y
    assert L.kron_relu_bwd(10, P(0), P(MB), P(MB + 16), None) == _lib.KRON_E_ALIAS  # out partly over dy
    arr = ctypes.c_void_p * 2
    n = (ctypes.c_int64 * 2)(100, 50)
    T = arr(BASE, BASE + MB)
    assert L.kron_l1_penalty(65, T, n, 1.0, P(2 * MB), 0, None) == _lib.KRON_E_ARG
    assert L.kron_l1_penalty(2, T, n, 1.0, None, 0, None) == _lib.KRON_E_NULL
    assert L.kron_l1_penalty(2, None, n, 1.0, P(2 * MB), 0, None) == _lib.KRON_E_NULL
    assert L.kron_l1_penalty(2, T, n, 1.0, P(2 * MB), 2, None) == _lib.KRON_E_ARG          # unknown flag
    assert L.kron_l1_penalty(2, T, n, float("nan"), P(2 * MB), 0, None) == _lib.KRON_E_ARG
    assert L.kron_l1_penalty(2, T, (ctypes.c_int64 * 2)(100, -1), 1.0, P(2 * MB), 0, None) == _lib.KRON_E_ARG
    assert L.kron_l1_penalty(2, T, n, 1.0, P(MB + 64), 0, None) == _lib.KRON_E_ALIAS        # loss in a tensor
    assert L.kron_l1_penalty(2, arr(BASE, BASE + MB + 4), n, 1.0, P(2 * MB), 0, None) == _lib.KRON_E_ALIGN
    assert L.kron_l1_penalty_grad(-1, P(0), 1.0, P(MB), P(2 * MB), None) == _lib.KRON_E_SHAPE
    assert L.kron_l1_penalty_grad(0, None, 1.0, None, None, None) == 0
    assert L.kron_l1_penalty_grad(10, P(0), 1.0, None, P(2 * MB), None) == _lib.KRON_E_NULL
    assert L.kron_l1_penalty_grad(10, P(0), float("inf"), P(MB), P(2 * MB), None) == _lib.KRON_E_ARG
    assert L.kron_l1_penalty_grad(10, P(0), 1.0, P(MB), P(16), None) == _lib.KRON_E_ALIAS   # dS over S
    assert L.kron_l1_penalty_grad(10, P(0), 1.0, P(32), P(16), None) == _lib.KRON_E_ALIAS


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    import kronecker_factored_structured_amd as K
    x = torch.zeros(4, 4)
    A = torch.zeros(1, 2, 2)
    B = torch.zeros(1, 2, 2)
    with pytest.raises(ValueError, match="GPU tensor"):
        K.kron_linear_fwd(x, None, A, B)


def test_saved_path_argument_errors():
    """kron_linear_zcache_bytes / kron_linear_fwd_save / kron_linear_bwd_saved refuse what
    they cannot run before any HIP call."""
    L = _lib.lib()
    MB = 1 << 20
    s = KronShape(64, 32, 32, 32, 32, 4, 0)
    zc_bytes = L.kron_linear_zcache_bytes(ctypes.byref(s))
    per_rank = 64 * 32 * 32 * 4                               # N * p * n floats per saved rank
    assert zc_bytes % per_rank == 0 and 1 <= zc_bytes // per_rank <= 4
    for other in (KronShape(64, 32, 32, 32, 32, 2, 0), KronShape(64, 16, 16, 64, 64, 2, 0),
                  KronShape(64, 8, 8, 8, 8, 1, 0), KronShape(-1, 32, 32, 32, 32, 4, 0)):
        assert L.kron_linear_zcache_bytes(ctypes.byref(other)) == 0
    assert L.kron_linear_zcache_bytes(ctypes.byref(KronShape(0, 32, 32, 32, 32, 4, 0))) == 0

    def fs(shape, zc=P(80 * MB), zb=zc_bytes, x=P(0), y=P(16 * MB)):
        return L.kron_linear_fwd_save(ctypes.byref(shape), x, None, P(32 * MB), P(48 * MB), None, y, zc,
                                      ctypes.c_size_t(zb), None)

    assert fs(s, zc=None) == _lib.KRON_E_NULL
    assert fs(s, zb=zc_bytes - 4) == _lib.KRON_E_WORKSPACE
    assert fs(s, zc=P(80 * MB + 4)) == _lib.KRON_E_ALIGN
    assert fs(s, zc=P(128 * 1024)) == _lib.KRON_E_ALIAS          # the cache overlaps x
    assert fs(s, zc=P(16 * MB + 64)) == _lib.KRON_E_ALIAS        # the cache overlaps y
    assert fs(KronShape(64, 32, 32, 32, 32, 2, 0)) == _lib.KRON_E_UNSUPPORTED
    assert fs(KronShape(64, 32, 32, 32, 32, 4, _lib.KRON_SPARSE_ROWS)) == _lib.KRON_E_ARG
    assert fs(KronShape(0, 32, 32, 32, 32, 4, 0), zc=None, x=None, y=None) == 0   # N == 0: no-op

    ws = L.kron_linear_bwd_workspace_bytes(ctypes.byref(s))

    def bs(shape, zc=P(80 * MB), zb=zc_bytes, dx=P(96 * MB)):
        return L.kron_linear_bwd_saved(ctypes.byref(shape), P(0), P(16 * MB), P(32 * MB), P(48 * MB), P(64 * MB),
                                       zc, ctypes.c_size_t(zb), dx, P(112 * MB), P(128 * MB), P(144 * MB),
                                       P(160 * MB), P(192 * MB), ctypes.c_size_t(ws), None)

    assert bs(s, zc=None) == _lib.KRON_E_NULL
    assert bs(s, zb=zc_bytes - 4) == _lib.KRON_E_WORKSPACE
    assert bs(s, zc=P(80 * MB + 8)) == _lib.KRON_E_ALIGN
    assert bs(s, dx=P(80 * MB + 256)) == _lib.KRON_E_ALIAS       # dx overlaps the cache
    assert bs(KronShape(64, 32, 32, 32, 32, 1, 0)) == _lib.KRON_E_UNSUPPORTED
    assert bs(KronShape(64, 32, 32, 32, 32, 4, _lib.KRON_SPARSE_ROWS)) == _lib.KRON_E_ARG
    assert "sparse-row" in _lib.last_error()
