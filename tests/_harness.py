"""Shared helpers of the parity tests: device transfer and the error metric."""
from __future__ import annotations

import numpy as np

TOL_F32 = 1e-5    # max-norm relative error, fp32 inputs
TOL_BF16 = 2e-2   # bf16 inputs, fp32 accumulation


def rel_err(got, want) -> float:
    """max|got - want| / max|want| in fp64 (absolute max when want is all zero)."""
    g = np.asarray(got, dtype=np.float64)
    w = np.asarray(want, dtype=np.float64)
    assert g.shape == w.shape, (g.shape, w.shape)
    if g.size == 0:
        return 0.0
    den = np.abs(w).max()
    num = np.abs(g - w).max()
    return float(num / den) if den > 0 else float(num)


def dev(a, dtype=None):
    import torch
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda").contiguous()


def host(t):
    return None if t is None else t.detach().float().cpu().numpy().astype(np.float64)


def bits(t):
    """Raw fp32 bit patterns of a device tensor (for bitwise comparisons)."""
    return t.detach().cpu().contiguous().view(__import__("torch").int32).numpy()
