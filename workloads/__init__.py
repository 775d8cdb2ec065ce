"""Seeded synthetic inputs for the Kronecker-factored layer and the Kronecker-sparse matmul.

This module only draws numbers and rounds them to the storage precision.  It holds
none of the method's arithmetic, so the fp64 oracle and the HIP path can both take
their inputs from here without sharing any computation.

Recipe (the same for every workload):
  * numpy PCG64, one SeedSequence per workload; every tensor has its own child
    stream, spawned in the fixed order listed in ``_STREAMS`` so that adding a
    tensor never changes the others.
  * Values are drawn in fp64 and rounded to fp32 with round-to-nearest-even
    (numpy's ``astype(float32)``); for bf16 inputs the fp32 values are rounded
    again to bf16 with round-to-nearest-even, and the oracle sees exactly the
    rounded values.
  * Variances follow the layer's initialisation on the Kronecker-layer tutorial
    ("Build W, then multiply" code: A drawn as randn/sqrt(p), B as randn/sqrt(block)),
    i.e. N(0, 1/fan_in) with fan_in = p for A and m for B.

Shapes follow the pages' workloads: the 1024x1024 MLP hidden layer at 20,000 rows
(tutorial, "Setup": 197 tokens per image, 20,000 rows ~ 100 images), the GPT-2
small FFN (768 <-> 3072) at 8 x 1024 token rows, and the ViT-S/16 MLP shape for the
Kronecker-sparse matmul (128 images x 197 tokens).  No dataset or weights are used.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# Order in which child streams are spawned from a workload's SeedSequence.
_STREAMS = ("x", "S", "A", "B", "bias", "dy", "labels", "head_w", "head_b",
            "x2", "A2", "B2", "S2", "bias2", "dy2", "vals")


def _rng(seed: int, name: str) -> np.random.Generator:
    children = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return np.random.Generator(np.random.PCG64(children[_STREAMS.index(name)]))


def f32(a: np.ndarray) -> np.ndarray:
    """Round fp64 draws to fp32 (round-to-nearest-even) and make them contiguous."""
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))


def bf16_bits(a32: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round-to-nearest-even); return the 16-bit patterns.

    Finite inputs only (the generators never produce NaN or Inf).
    """
    u = np.ascontiguousarray(a32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to the fp32 values they represent (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(seed: int, name: str, shape, var: float = 1.0) -> np.ndarray:
    return f32(_rng(seed, name).standard_normal(shape) * np.sqrt(var))


@dataclass
class KronShape:
    N: int
    p: int
    q: int
    m: int
    n: int
    r: int

    @property
    def in_features(self) -> int:
        return self.p * self.m

    @property
    def out_features(self) -> int:
        return self.q * self.n


@dataclass
class KronInputs:
    shape: KronShape
    x: np.ndarray                 # N x (p*m) fp32
    S: Optional[np.ndarray]       # p x q fp32, or None for S == 1
    A: np.ndarray                 # r x p x q fp32
    B: np.ndarray                 # r x m x n fp32
    bias: Optional[np.ndarray]    # q*n fp32 or None
    dy: np.ndarray                # N x (q*n) fp32
    seed: int = 0
    meta: dict = field(default_factory=dict)


def kron_inputs(seed: int, N: int, p: int, q: int, m: int, n: int, r: int, *,
                s_mode: str = "none", bias_mode: str = "zeros",
                zero_frac: float = 0.5, names=("x", "S", "A", "B", "bias", "dy")) -> KronInputs:
    """Draw one Kronecker-layer workload.

    s_mode: "none" (S absent, S == 1), "ones" (S stored, all ones), "uniform"
    (U(0,1)), "uniform_zeroed" (U(0,1) with exactly round(zero_frac*p*q) entries set
    to 0 at positions chosen by a seeded permutation), "rows_zeroed" (U(0,1) with
    round(zero_frac*p) whole rows set to 0 at seeded positions: the structured sparsity
    an l1-pruned mask can leave), "blocks_zeroed" (U(0,1) with round(zero_frac * number of
    16 x 16 blocks) whole blocks set to 0 at seeded positions; p and q multiples of 16),
    "integer" (small integers, for exact-arithmetic tests).
    bias_mode: "none", "zeros", "normal".
    """
    nx, nS, nA, nB, nb, ndy = names
    x = normal(seed, nx, (N, p * m))
    A = normal(seed, nA, (r, p, q), 1.0 / p)
    B = normal(seed, nB, (r, m, n), 1.0 / m)
    S = None
    if s_mode == "ones":
        S = np.ones((p, q), np.float32)
    elif s_mode in ("uniform", "uniform_zeroed", "rows_zeroed", "blocks_zeroed"):
        g = _rng(seed, nS)
        S = f32(g.uniform(0.0, 1.0, (p, q)))
        if s_mode == "uniform_zeroed":
            nz = int(round(zero_frac * p * q))
            idx = g.permutation(p * q)[:nz]
            S.reshape(-1)[idx] = 0.0
        elif s_mode == "rows_zeroed":
            rows = g.permutation(p)[:int(round(zero_frac * p))]
            S[rows, :] = 0.0
        elif s_mode == "blocks_zeroed":
            bj, bk = p // 16, q // 16
            for blk in g.permutation(bj * bk)[:int(round(zero_frac * bj * bk))]:
                S[16 * (blk // bk):16 * (blk // bk) + 16, 16 * (blk % bk):16 * (blk % bk) + 16] = 0.0
    elif s_mode != "none":
        raise ValueError(s_mode)
    bias = None
    if bias_mode == "zeros":
        bias = np.zeros(q * n, np.float32)
    elif bias_mode == "normal":
        bias = normal(seed, nb, (q * n,))
    dy = normal(seed, ndy, (N, q * n))
    return KronInputs(KronShape(N, p, q, m, n, r), x, S, A, B, bias, dy, seed)


def integer_kron_inputs(seed: int, N: int, p: int, q: int, m: int, n: int, r: int,
                        with_S: bool = True, lo: int = -3, hi: int = 4) -> KronInputs:
    """Small-integer-valued inputs: every product and sum the layer forms is exact in fp64
    (and in fp32 for small shapes), so identities can be checked bit for bit."""
    g = _rng(seed, "x")
    def ints(shape):
        return g.integers(lo, hi, size=shape).astype(np.float32)
    x = ints((N, p * m))
    S = ints((p, q)) if with_S else None
    A = ints((r, p, q))
    B = ints((r, m, n))
    bias = ints((q * n,))
    dy = ints((N, q * n))
    return KronInputs(KronShape(N, p, q, m, n, r), x, S, A, B, bias, dy, seed)


# --------------------------------------------------------------------------------------
# The five named workloads.
# --------------------------------------------------------------------------------------

def tiny_layer(seed: int = 1) -> KronInputs:
    """64 rows, 64x64 layer, m = 8 (p = q = 8), r = 2, S = ones, zero bias."""
    return kron_inputs(seed, 64, 8, 8, 8, 8, 2, s_mode="ones", bias_mode="zeros")


def headline_layer(seed: int = 2, N: int = 20000) -> KronInputs:
    """20,000 rows, 1024x1024 layer, m = n = 32 (S, A_i 32x32), r = 4; S ~ U(0,1) with
    exactly half of its 1024 entries zeroed (block-sparse W)."""
    return kron_inputs(seed, N, 32, 32, 32, 32, 4, s_mode="uniform_zeroed", bias_mode="zeros")


def gpt2_ffn_layers(r: int, seed: int = 4, N: int = 8192):
    """GPT-2 small FFN shape: 768 -> 3072 with A_i 32x64, B_i 24x48 (no S), and the
    transposed 3072 -> 768 layer with A_i 64x32, B_i 48x24, independent draws."""
    up = kron_inputs(seed * 100 + r, N, 32, 64, 24, 48, r, s_mode="none", bias_mode="zeros")
    down = kron_inputs(seed * 100 + r, N, 64, 32, 48, 24, r, s_mode="none", bias_mode="zeros",
                       names=("x2", "S2", "A2", "B2", "bias2", "dy2"))
    return up, down


@dataclass
class MLPInputs:
    x: np.ndarray            # N x 1024
    labels: np.ndarray       # N int64 in [0, 10)
    layers: list             # two dicts with S, A, B, bias (fp32)
    head_w: np.ndarray       # 1024 x 10 (row-vector convention: z = h @ head_w + head_b)
    head_b: np.ndarray       # 10
    m: int
    r: int
    lam: float
    lr: float


def mlp_step_inputs(seed: int = 3, N: int = 20000, hidden: int = 1024, classes: int = 10,
                    m: int = 64, r: int = 2, lam: float = 1e-4, lr: float = 1e-3) -> MLPInputs:
    """MLP 1024 -> 1024 -> 1024 -> 10 with ReLU; both hidden layers Kronecker (m = 64,
    p = q = 16, r = 2), S initialised to ones and bias to zeros as in the tutorial's
    layer; a dense head with U(-1/sqrt(1024), 1/sqrt(1024)) weight and bias."""
    p = hidden // m
    x = normal(seed, "x", (N, hidden))
    labels = _rng(seed, "labels").integers(0, classes, size=N).astype(np.int64)
    layers = []
    for li, (nA, nB) in enumerate((("A", "B"), ("A2", "B2"))):
        layers.append(dict(S=np.ones((p, p), np.float32),
                           A=normal(seed, nA, (r, p, p), 1.0 / p),
                           B=normal(seed, nB, (r, m, m), 1.0 / m),
                           bias=np.zeros(hidden, np.float32)))
    bound = 1.0 / np.sqrt(hidden)
    head_w = f32(_rng(seed, "head_w").uniform(-bound, bound, (hidden, classes)))
    head_b = f32(_rng(seed, "head_b").uniform(-bound, bound, (classes,)))
    return MLPInputs(x, labels, layers, head_w, head_b, m, r, lam, lr)


@dataclass
class KSInputs:
    a: int
    b: int
    c: int
    d: int
    x: np.ndarray        # N x (a*b*d) fp32 (bf16-representable when dtype is bf16)
    vals: np.ndarray     # a x d x b x c fp32 (bf16-representable when dtype is bf16)
    dtype: str           # "f32" or "bf16"
    x_bits: Optional[np.ndarray] = None     # bf16 patterns when dtype == "bf16"
    vals_bits: Optional[np.ndarray] = None


def ks_inputs(seed: int, N: int, a: int, b: int, c: int, d: int, dtype: str = "f32",
              nonzero: bool = True) -> KSInputs:
    """Kronecker-sparse matmul inputs: values ~ N(0, 1/b) stored as vals[alpha][delta][beta][gamma].

    With ``nonzero`` the values are redrawn until none is an exact zero (so that the
    support of the dense matrix is unambiguous)."""
    x = normal(seed, "x", (N, a * b * d))
    g = _rng(seed, "vals")
    while True:
        vals = f32(g.standard_normal((a, d, b, c)) / np.sqrt(b))
        if dtype == "bf16":
            vb = bf16_bits(vals)
            vals = bf16_to_f32(vb).reshape(vals.shape)
        if not nonzero or np.all(vals != 0):
            break
    out = KSInputs(a, b, c, d, x, vals, dtype)
    if dtype == "bf16":
        out.x_bits = bf16_bits(x).reshape(x.shape)
        out.x = bf16_to_f32(out.x_bits).reshape(x.shape)
        out.vals_bits = bf16_bits(vals).reshape(vals.shape)
    return out


def vit_ks(dtype: str = "f32", seed: int = 5, N: int = 25216) -> KSInputs:
    """ViT-S/16 MLP shape: (a,b,c,d) = (2,48,192,4), a 384 x 1536 matrix, 25,216 rows
    (128 images x 197 tokens)."""
    return ks_inputs(seed, N, 2, 48, 192, 4, dtype)
