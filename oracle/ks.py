"""fp64 oracle of the Kronecker-sparse (KS) matmul (test infrastructure only).

Source: "Fast Inference with Kronecker-Sparse Matrices" (arXiv 2405.15013), abstract:
a KS matrix is one whose support is a Kronecker product of identity and all-ones
blocks.  The pattern used here is I_a (x) 1_{b x c} (x) I_d, an (a*b*d) x (a*c*d)
matrix K with a*b*c*d nonzeros, applied to rows as Y = X K.

The page gives no value layout.  Reading adopted: row-major Kronecker indices,
row (alpha, beta, delta) -> (alpha*b + beta)*d + delta and column
(alpha, gamma, delta) -> (alpha*c + gamma)*d + delta, with the nonzero values
stored as vals[alpha][delta][beta][gamma] (a x d x b x c).
"""
from __future__ import annotations

import numpy as np

from .kron import as64, kron_block


def support(a: int, b: int, c: int, d: int) -> np.ndarray:
    """0/1 support I_a (x) 1_{b x c} (x) I_d, built with the block-by-block Kronecker product."""
    return kron_block(kron_block(np.eye(a), np.ones((b, c))), np.eye(d))


def dense(vals, a: int, b: int, c: int, d: int) -> np.ndarray:
    """Scatter vals[alpha][delta][beta][gamma] into the dense (a*b*d) x (a*c*d) matrix."""
    V = as64(vals).reshape(a, d, b, c)
    K = np.zeros((a * b * d, a * c * d))
    for al in range(a):
        for de in range(d):
            rows = (al * b + np.arange(b)) * d + de
            cols = (al * c + np.arange(c)) * d + de
            K[np.ix_(rows, cols)] = V[al, de]
    return K


def matmul(x, vals, a: int, b: int, c: int, d: int) -> np.ndarray:
    """Y = X K with K the dense KS matrix."""
    return as64(x) @ dense(vals, a, b, c, d)


def backward(x, vals, dy, a: int, b: int, c: int, d: int) -> dict:
    """Gradients of the scalar <dY, X K> (by calculus from Y = X K with K the dense KS
    matrix): dX = dY K^T, and dK = X^T dY, of which only the support entries are free
    parameters; they are gathered back into the vals[alpha][delta][beta][gamma] layout."""
    K = dense(vals, a, b, c, d)
    dx = as64(dy) @ K.T
    dK = as64(x).T @ as64(dy)
    dv = np.empty((a, d, b, c))
    for al in range(a):
        for de in range(d):
            rows = (al * b + np.arange(b)) * d + de
            cols = (al * c + np.arange(c)) * d + de
            dv[al, de] = dK[np.ix_(rows, cols)]
    return {"dx": dx, "dvals": dv}


def chain(x, factors) -> np.ndarray:
    """Y = X K_1 K_2 ... K_F for Kronecker-sparse factors given as (a, b, c, d, vals): the
    product of the dense KS matrices, applied left to right (each factor's input width
    a*b*d equals the previous factor's output width a*c*d)."""
    y = as64(x)
    for (a, b, c, d, vals) in factors:
        y = y @ dense(vals, a, b, c, d)
    return y


def kron3_factors(A, B, C):
    """A (x) B (x) C as three KS factors (mixed-product rule):
    (A (x) I_{p2 p3}) (I_{q1} (x) B (x) I_{p3}) (I_{q1 q2} (x) C), with every block of a
    factor holding the same small matrix."""
    A, B, C = as64(A), as64(B), as64(C)
    (p1, q1), (p2, q2), (p3, q3) = A.shape, B.shape, C.shape
    f1 = (1, p1, q1, p2 * p3, np.broadcast_to(A, (1, p2 * p3, p1, q1)).copy())
    f2 = (q1, p2, q2, p3, np.broadcast_to(B, (q1, p3, p2, q2)).copy())
    f3 = (q1 * q2, p3, q3, 1, np.broadcast_to(C, (q1 * q2, 1, p3, q3)).copy())
    return [f1, f2, f3]
