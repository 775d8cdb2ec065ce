"""fp64 oracle of the Van Loan rank-r Kronecker projection (test infrastructure only).

Source: "Replicating & Extending Krony-PT on GPT-2 Small", section "Core Algorithm - Van
Loan Kronecker Decomposition": the best sum of r Kronecker products to a dense W in the
Frobenius norm comes from the rearrangement of W (a block permutation) and the rank-r
truncated SVD of the rearranged matrix; each term's factors are the singular vectors
reshaped to the factor shapes, each scaled by the square root of its singular value.

Orientation of this library's layer: W is in x out with in = p*m, out = q*n, and
W = sum_i kron(C_i, B_i) with C_i p x q, B_i m x n.  The rearrangement is
R[(j*q + k), (a*n + b)] = W[j*m + a, k*n + b], so that R = sum_i vec(C_i) vec(B_i)^T.
Sign of each pair (the SVD leaves it free; the product C_i (x) B_i does not depend on it):
the entry of C_i largest in magnitude (first such in row-major order) is positive.
"""
from __future__ import annotations

import numpy as np

from .kron import as64


def rearrange(W, p: int, q: int, m: int, n: int) -> np.ndarray:
    """R[(j*q + k), (a*n + b)] = W[j*m + a, k*n + b]."""
    return as64(W).reshape(p, m, q, n).transpose(0, 2, 1, 3).reshape(p * q, m * n)


def project(W, p: int, q: int, m: int, n: int, r: int):
    """Rank-r Van Loan factors (C [r,p,q], B [r,m,n], sigma [r]) from LAPACK's SVD of R."""
    U, s, Vt = np.linalg.svd(rearrange(W, p, q, m, n), full_matrices=False)
    C = np.empty((r, p, q))
    B = np.empty((r, m, n))
    for i in range(r):
        u, v = U[:, i], Vt[i]
        sgn = 1.0 if u[int(np.argmax(np.abs(u)))] >= 0 else -1.0
        C[i] = sgn * np.sqrt(s[i]) * u.reshape(p, q)
        B[i] = sgn * np.sqrt(s[i]) * v.reshape(m, n)
    return C, B, s[:r].copy()


def reconstruct(C, B) -> np.ndarray:
    """sum_i kron(C_i, B_i) with numpy.kron."""
    return sum(np.kron(as64(C[i]), as64(B[i])) for i in range(len(C)))
