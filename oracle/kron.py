"""fp64 oracle of the Kronecker-factored linear layer (test infrastructure only).

Source: "A Kronecker layer benchmark" tutorial (khalilimahdi.github.io, 2026/10).
  * Intro: each weight matrix is a sum of Kronecker products, W = sum_i kron(S o A_i, B_i),
    with an l1 penalty on S; zeros of S give zero blocks of W whose size is that of B_i.
  * "Build W, then multiply": S and A_i are p x q, B_i is m x n, W is (p*m) x (q*n),
    oriented in x out; the layer returns x W + bias with a per-column bias.

The oracle is that definition written out: build each Kronecker product block by
block, sum over the rank, multiply densely.  Gradients are the calculus of
y = x W + bias taken through W:
    dX = dY W^T,  dW = X^T dY,  dbias = sum over rows of dY,
    dC_i[j,k] = sum_{a,b} dW[j*m+a, k*n+b] * B_i[a,b]     (C_i = S o A_i)
    dB_i[a,b] = sum_{j,k} dW[j*m+a, k*n+b] * C_i[j,k]
    dS = sum_i A_i o dC_i,   dA_i = S o dC_i   (dA_i = dC_i when S is absent, S == 1).
Nothing here uses the vec trick; the HIP path does, and the tests compare the two.
"""
from __future__ import annotations

import numpy as np


def as64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def kron_block(C: np.ndarray, B: np.ndarray) -> np.ndarray:
    """kron(C, B) built block by block: block (j, k) of the result is C[j, k] * B."""
    C = as64(C)
    B = as64(B)
    p, q = C.shape
    m, n = B.shape
    K = np.zeros((p * m, q * n))
    for j in range(p):
        for k in range(q):
            K[j * m:(j + 1) * m, k * n:(k + 1) * n] = C[j, k] * B
    return K


def factors_C(S, A) -> np.ndarray:
    """C_i = S o A_i (elementwise); S None means S == 1."""
    A = as64(A)
    if S is None:
        return A.copy()
    return as64(S)[None, :, :] * A


def weight(S, A, B) -> np.ndarray:
    """W = sum_i kron(S o A_i, B_i), shape (p*m) x (q*n)."""
    C = factors_C(S, A)
    B = as64(B)
    W = np.zeros((C.shape[1] * B.shape[1], C.shape[2] * B.shape[2]))
    for i in range(C.shape[0]):
        W += kron_block(C[i], B[i])
    return W


def forward(x, S, A, B, bias=None, relu: bool = False) -> np.ndarray:
    """y = x W + bias (optionally followed by max(., 0))."""
    y = as64(x) @ weight(S, A, B)
    if bias is not None:
        y = y + as64(bias)[None, :]
    if relu:
        y = np.maximum(y, 0.0)
    return y


def backward(x, S, A, B, dy, want_dx: bool = True, W: np.ndarray | None = None):
    """Gradients of sum(dy * (x W + bias)) with respect to x, S, A, B and bias.

    Returns dict(dx, dS, dA, dB, dbias); dS is None when S is None, dx is None when
    not wanted.
    """
    x = as64(x)
    dy = as64(dy)
    B = as64(B)
    C = factors_C(S, A)
    r, p, q = C.shape
    _, m, n = B.shape
    if W is None:
        W = weight(S, A, B)
    dx = dy @ W.T if want_dx else None
    dW = x.T @ dy
    dbias = dy.sum(axis=0)
    dC = np.zeros((r, p, q))
    dB = np.zeros((r, m, n))
    for j in range(p):
        for k in range(q):
            blk = dW[j * m:(j + 1) * m, k * n:(k + 1) * n]
            for i in range(r):
                dC[i, j, k] = np.sum(blk * B[i])
                dB[i] += blk * C[i, j, k]
    if S is None:
        dS = None
        dA = dC
    else:
        S64 = as64(S)
        dS = np.sum(as64(A) * dC, axis=0)
        dA = S64[None, :, :] * dC
    return dict(dx=dx, dS=dS, dA=dA, dB=dB, dbias=dbias)


# ---------------------------------------------------------------------------------
# Cost model and parameter counts (tutorial, "The vec trick" and the two results
# sections): the vec trick needs about r/m of the dense multiply-adds, and the
# rank-1 8x8 layer has ~33k parameters against ~1.05M for dense.
# ---------------------------------------------------------------------------------

def param_count(in_features: int, out_features: int, m: int, r: int, n: int | None = None) -> int:
    """Parameters of one layer: S (p x q), A (r x p x q), B (r x m x n), bias (out)."""
    n = m if n is None else n
    p, q = in_features // m, out_features // n
    return p * q + r * p * q + r * m * n + out_features


def dense_param_count(in_features: int, out_features: int) -> int:
    return in_features * out_features + out_features


def vec_trick_macs_per_row(p: int, q: int, m: int, n: int, r: int) -> int:
    """Multiply-adds per row of the X B_i-first evaluation sum_i (S o A_i)^T X B_i:
    X B_i costs p*m*n and the product with (S o A_i)^T costs q*p*n, per rank."""
    return r * (p * m * n + q * p * n)


def dense_macs_per_row(in_features: int, out_features: int) -> int:
    return in_features * out_features
