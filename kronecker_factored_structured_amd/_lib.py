"""ctypes declarations of libkron's C ABI (include/kron.h).

Loading fails loudly when the library has not been built: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# KRON_LIB_PATH selects another build of the library (e.g. the host-sanitized one)
LIB_PATH = os.environ.get("KRON_LIB_PATH") or os.path.join(_HERE, "libkron.so")

KRON_OK = 0
KRON_E_NULL = 1
KRON_E_SHAPE = 2
KRON_E_ALIGN = 3
KRON_E_ALIAS = 4
KRON_E_DTYPE = 5
KRON_E_WORKSPACE = 6
KRON_E_UNSUPPORTED = 7
KRON_E_HIP = 8
KRON_E_ARG = 9

KRON_F32 = 0
KRON_BF16 = 1

KRON_RELU_OUT = 1
KRON_DX_RELU_MASK = 2
KRON_SPARSE_ROWS = 4

KRON_ACCUMULATE = 1

# Every symbol include/kron.h declares.
EXPORTS = (
    "kron_abi_version", "kron_status_str", "kron_last_error", "kron_linear_check",
    "kron_linear_bwd_workspace_bytes", "kron_linear_fwd", "kron_linear_bwd", "ks_matmul",
    "kron_adam_l1_step", "kron_head_ce_workspace_bytes", "kron_head_ce",
    "kron_linear_bwd_bf16_workspace_bytes", "kron_linear_fwd_bf16", "kron_linear_bwd_bf16",
    "ks_matmul_out", "ks_matmul_bwd_workspace_bytes", "ks_matmul_bwd", "ks_chain",
    "kron_van_loan_workspace_bytes", "kron_van_loan", "kron_relu_bwd", "kron_l1_penalty",
    "kron_l1_penalty_grad", "kron_linear_bwd_noalloc", "kron_linear_zcache_bytes", "kron_linear_fwd_save",
    "kron_linear_bwd_saved",
)

KRON_NOALLOC_SCRATCH_BYTES = 32 << 20


class KsFactor(ctypes.Structure):
    _fields_ = [("a", ctypes.c_int32), ("b", ctypes.c_int32), ("c", ctypes.c_int32), ("d", ctypes.c_int32),
                ("vals", ctypes.c_void_p)]


class KronShape(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("p", ctypes.c_int32), ("q", ctypes.c_int32),
                ("m", ctypes.c_int32), ("n", ctypes.c_int32), ("r", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


class KronError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        self.status = status
        super().__init__(f"{fn} failed: {status_str(status)} ({status}): {detail}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libkron.so (loaded on first use)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"libkron.so not found at {LIB_PATH}; build it first with "
                "`python -m kronecker_factored_structured_amd.build` (no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t
        shp = ctypes.POINTER(KronShape)
        pp = ctypes.POINTER(ctypes.c_void_p)
        sig = {
            "kron_abi_version": (i32, []),
            "kron_status_str": (ctypes.c_char_p, [i32]),
            "kron_last_error": (ctypes.c_char_p, []),
            "kron_linear_check": (i32, [shp]),
            "kron_linear_bwd_workspace_bytes": (sz, [shp]),
            "kron_linear_fwd": (i32, [shp, vp, vp, vp, vp, vp, vp, vp]),
            "kron_linear_bwd": (i32, [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "kron_linear_zcache_bytes": (sz, [shp]),
            "kron_linear_fwd_save": (i32, [shp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "kron_linear_bwd_saved": (i32, [shp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp, vp, vp, vp, sz, vp]),
            "ks_matmul": (i32, [i64, i32, i32, i32, i32, i32, vp, vp, vp, vp]),
            "ks_matmul_out": (i32, [i64, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp]),
            "ks_matmul_bwd_workspace_bytes": (ctypes.c_size_t, [i64, i32, i32, i32, i32, i32]),
            "ks_matmul_bwd": (i32, [i64, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]),
            "ks_chain": (i32, [i64, i32, ctypes.POINTER(KsFactor), i32, vp, vp, vp]),
            "kron_van_loan_workspace_bytes": (ctypes.c_size_t, [i32, i32, i32, i32, i32]),
            "kron_van_loan": (i32, [i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]),
            "kron_adam_l1_step": (i32, [i32, pp, pp, pp, pp, ctypes.POINTER(ctypes.c_int64),
                                        ctypes.POINTER(ctypes.c_float), i64, ctypes.c_double,
                                        ctypes.c_double, ctypes.c_double, ctypes.c_double, vp]),
            "kron_head_ce_workspace_bytes": (sz, [i64, i32, i32]),
            "kron_head_ce": (i32, [i64, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, u32, vp, sz, vp]),
            "kron_linear_bwd_bf16_workspace_bytes": (sz, [shp]),
            "kron_linear_fwd_bf16": (i32, [shp, vp, vp, vp, vp, vp, vp, vp]),
            "kron_linear_bwd_bf16": (i32, [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
            "kron_linear_bwd_noalloc": (i32, [shp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
            "kron_relu_bwd": (i32, [i64, vp, vp, vp, vp]),
            "kron_l1_penalty": (i32, [i32, pp, ctypes.POINTER(ctypes.c_int64), ctypes.c_float, vp, u32, vp]),
            "kron_l1_penalty_grad": (i32, [i64, vp, ctypes.c_float, vp, vp, vp]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        if L.kron_abi_version() != 1:
            raise ImportError("libkron ABI version mismatch")
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().kron_status_str(status).decode()


def last_error() -> str:
    return lib().kron_last_error().decode()


def check(fn: str, status: int) -> None:
    if status != KRON_OK:
        raise KronError(fn, status, last_error())
