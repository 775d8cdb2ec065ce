"""Pins of the fp64 oracle against facts fixed outside it (CPU only).

Each test names what it pins.  None of them re-types the oracle's own formula:
they use textbook identities, library routines (numpy's kron, einsum, LAPACK SVD,
scipy's block_diag, torch autograd), finite differences that are exact for affine
functions, and the quantities the tutorial prints.
"""
import json
import os

import numpy as np
import pytest
import scipy.linalg

import oracle
from oracle import kron as OK
from oracle import ks as OKS
from oracle import vanloan as OVL
from workloads import integer_kron_inputs, kron_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _shape_cases():
    # (p, q, m, n, r): square, rectangular, degenerate
    return [(2, 3, 2, 2, 1), (3, 2, 2, 3, 2), (2, 2, 3, 1, 3), (1, 1, 2, 3, 2), (3, 4, 1, 1, 2)]


# ----------------------------------------------------------------------------------
# Kronecker product and W
# ----------------------------------------------------------------------------------

def test_kron_textbook_example():
    """Hand-worked 2x2 (x) 2x2 example and the layer on it."""
    g = json.load(open(os.path.join(GOLDEN, "kron_textbook_2x2.json")))
    K = OK.kron_block(np.array(g["C"], float), np.array(g["B"], float))
    assert np.array_equal(K, np.array(g["kron_CB"], float))
    y = OK.forward(np.array(g["x"], float), None, np.array([g["C"]], float),
                   np.array([g["B"]], float), np.array(g["bias"], float))
    assert np.array_equal(y, np.array(g["y"], float))


@pytest.mark.parametrize("shapes", [((2, 3), (4, 2)), ((1, 5), (3, 1)), ((3, 3), (2, 2))])
def test_kron_matches_numpy(shapes):
    """Library routine: numpy.kron."""
    rng = np.random.default_rng(0)
    C = rng.standard_normal(shapes[0])
    B = rng.standard_normal(shapes[1])
    assert np.array_equal(OK.kron_block(C, B), np.kron(C, B))


def test_mixed_product_identity():
    """(A (x) B)(C (x) D) = (AC) (x) (BD), integer inputs -> exact in fp64."""
    rng = np.random.default_rng(1)
    A = rng.integers(-3, 4, (2, 3)).astype(float)
    C = rng.integers(-3, 4, (3, 4)).astype(float)
    B = rng.integers(-3, 4, (3, 2)).astype(float)
    D = rng.integers(-3, 4, (2, 5)).astype(float)
    lhs = OK.kron_block(A, B) @ OK.kron_block(C, D)
    rhs = OK.kron_block(A @ C, B @ D)
    assert np.array_equal(lhs, rhs)


@pytest.mark.parametrize("case", _shape_cases())
def test_weight_is_sum_of_numpy_krons(case):
    """W = sum_i kron(S o A_i, B_i), checked with numpy.kron; S absent means S == 1."""
    p, q, m, n, r = case
    for with_S in (True, False):
        inp = integer_kron_inputs(3, 2, p, q, m, n, r, with_S=with_S)
        S = inp.S if with_S else np.ones((p, q), np.float32)
        ref = sum(np.kron(S.astype(float) * inp.A[i], inp.B[i].astype(float)) for i in range(r))
        assert np.array_equal(OK.weight(inp.S, inp.A, inp.B), ref)


@pytest.mark.parametrize("case", _shape_cases())
def test_forward_vec_trick_identity(case):
    """Tutorial 'The vec trick': reshape each row to X (p x m) row-major; the row of the
    output is vec_row(sum_i (S o A_i)^T X B_i) + bias.  Integer inputs -> exact."""
    p, q, m, n, r = case
    inp = integer_kron_inputs(4, 5, p, q, m, n, r)
    X = inp.x.astype(float).reshape(5, p, m)
    C = inp.S.astype(float)[None] * inp.A.astype(float)
    # plain per-row loop with numpy matmul, written from the page's formula
    Y = np.zeros((5, q, n))
    for row in range(5):
        for i in range(r):
            Y[row] += C[i].T @ X[row] @ inp.B[i].astype(float)
    ref = Y.reshape(5, q * n) + inp.bias.astype(float)[None]
    assert np.array_equal(OK.forward(inp.x, inp.S, inp.A, inp.B, inp.bias), ref)


def test_one_hot_rows_reproduce_W():
    """forward(I_in, bias=0) gives the rows of W, and W matches numpy.kron sums."""
    inp = kron_inputs(7, 1, 4, 3, 2, 5, 2, s_mode="uniform_zeroed")
    eye = np.eye(inp.shape.in_features)
    Wref = sum(np.kron(inp.S.astype(float) * inp.A[i], inp.B[i].astype(float)) for i in range(2))
    np.testing.assert_allclose(OK.forward(eye, inp.S, inp.A, inp.B, None), Wref, rtol=0, atol=1e-15)


def test_rank1_block_frobenius_closed_form():
    """Rank 1: ||W_jk||_F = |S_jk A_jk| ||B||_F for every m x n block (block sparsity of W)."""
    inp = kron_inputs(8, 1, 5, 6, 3, 4, 1, s_mode="uniform_zeroed")
    W = OK.weight(inp.S, inp.A, inp.B)
    nb = np.linalg.norm(inp.B[0].astype(float))
    for j in range(5):
        for k in range(6):
            blk = W[j * 3:(j + 1) * 3, k * 4:(k + 1) * 4]
            want = abs(float(inp.S[j, k]) * float(inp.A[0, j, k])) * nb
            assert abs(np.linalg.norm(blk) - want) <= 1e-14 * max(1.0, want)
            if inp.S[j, k] == 0:
                assert not blk.any()


@pytest.mark.parametrize("r", [1, 2, 3])
def test_van_loan_rearrangement_rank(r):
    """Van Loan rearrangement R(W)[(j,k),(a,b)] = W[j*m+a, k*n+b] equals
    sum_i C_i[j,k] B_i[a,b] (outer products), so rank R(W) <= r (LAPACK SVD)."""
    p, q, m, n = 4, 3, 3, 5
    inp = kron_inputs(9, 1, p, q, m, n, r, s_mode="uniform")
    W = OK.weight(inp.S, inp.A, inp.B)
    R = W.reshape(p, m, q, n).transpose(0, 2, 1, 3).reshape(p * q, m * n)
    C = inp.S.astype(float)[None] * inp.A.astype(float)
    outer = sum(np.outer(C[i].reshape(-1), inp.B[i].astype(float).reshape(-1)) for i in range(r))
    np.testing.assert_allclose(R, outer, rtol=0, atol=1e-14)
    sv = np.linalg.svd(R, compute_uv=False)
    assert np.all(sv[r:] <= 1e-12 * sv[0])
    assert sv[r - 1] > 1e-6 * sv[0]


def test_van_loan_recovers_an_exact_kronecker_sum():
    """W = sum of three Kronecker products (numpy.kron): the rank-3 projection rebuilds W,
    and a rank-4 projection adds nothing (its fourth singular value is zero)."""
    rng = np.random.default_rng(11)
    p, q, m, n = 4, 3, 5, 2
    W = sum(np.kron(rng.standard_normal((p, q)), rng.standard_normal((m, n))) for _ in range(3))
    C, B, s = OVL.project(W, p, q, m, n, 3)
    np.testing.assert_allclose(OVL.reconstruct(C, B), W, rtol=0, atol=1e-12 * np.abs(W).max())
    _, _, s4 = OVL.project(W, p, q, m, n, 4)
    assert s4[3] <= 1e-12 * s4[0]


def test_van_loan_eckart_young_closed_form():
    """Orthonormal vec(C_i) and vec(B_i) (QR) with weights w: R has singular values w, each
    term is w_i C_i (x) B_i, and the rank-2 error is the sqrt of the dropped weights squared."""
    rng = np.random.default_rng(12)
    p, q, m, n = 4, 5, 3, 6
    w = np.array([5.0, 3.0, 2.0, 1.0, 0.5])
    Qc, _ = np.linalg.qr(rng.standard_normal((p * q, 5)))
    Qb, _ = np.linalg.qr(rng.standard_normal((m * n, 5)))
    W = sum(w[i] * np.kron(Qc[:, i].reshape(p, q), Qb[:, i].reshape(m, n)) for i in range(5))
    C, B, s = OVL.project(W, p, q, m, n, 2)
    np.testing.assert_allclose(s, w[:2], rtol=1e-12)
    for i in range(2):
        np.testing.assert_allclose(np.kron(C[i], B[i]),
                                   w[i] * np.kron(Qc[:, i].reshape(p, q), Qb[:, i].reshape(m, n)), atol=1e-12)
    err = np.linalg.norm(W - OVL.reconstruct(C, B))
    assert np.isclose(err, np.sqrt(np.sum(w[2:] ** 2)), rtol=1e-12)
    # sign convention: the largest entry of each C_i is positive
    for i in range(2):
        assert C[i].reshape(-1)[np.argmax(np.abs(C[i]))] > 0


@pytest.mark.parametrize("p,q,m,n,r", [(1, 5, 1, 1, 1)])
def test_special_case_diagonal_scaling(p, q, m, n, r):
    """p = 1, m = n = 1: the layer is x -> x * (S o A_1) row vector (q outputs)."""
    inp = integer_kron_inputs(10, 3, p, q, m, n, r)
    y = OK.forward(inp.x, inp.S, inp.A, inp.B, None)
    ref = inp.x.astype(float) @ (inp.S.astype(float) * inp.A[0].astype(float) * float(inp.B[0, 0, 0]))
    assert np.array_equal(y, ref)


def test_special_cases_reduce_to_gemm():
    """m = n = 1: W = S o sum_i A_i B_i (scalars).  p = q = 1: W = sum_i c_i B_i.
    r = 1, S == 1: W = numpy.kron(A, B)."""
    inp = integer_kron_inputs(11, 1, 4, 3, 1, 1, 3)
    W = OK.weight(inp.S, inp.A, inp.B)
    ref = inp.S.astype(float) * sum(inp.A[i].astype(float) * float(inp.B[i, 0, 0]) for i in range(3))
    assert np.array_equal(W, ref)
    inp = integer_kron_inputs(12, 1, 1, 1, 3, 4, 3)
    W = OK.weight(inp.S, inp.A, inp.B)
    ref = sum(float(inp.S[0, 0] * inp.A[i, 0, 0]) * inp.B[i].astype(float) for i in range(3))
    assert np.array_equal(W, ref)
    inp = integer_kron_inputs(13, 1, 3, 2, 2, 4, 1, with_S=False)
    assert np.array_equal(OK.weight(None, inp.A, inp.B), np.kron(inp.A[0].astype(float), inp.B[0].astype(float)))


# ----------------------------------------------------------------------------------
# Gradients
# ----------------------------------------------------------------------------------

def _loss(x, S, A, B, bias, dy):
    return float(np.sum(dy * OK.forward(x, S, A, B, bias)))


@pytest.mark.parametrize("case", [(2, 3, 2, 2, 2), (3, 2, 1, 3, 1), (2, 2, 2, 1, 3)])
@pytest.mark.parametrize("with_S", [True, False])
def test_gradients_exact_finite_differences(case, with_S):
    """L = <dY, x W + bias> is affine in every single scalar of x, S, A, B and bias, so
    the central difference with h = 1 is the exact partial derivative; with small
    integer inputs every value is exact in fp64 and the comparison is bitwise."""
    p, q, m, n, r = case
    inp = integer_kron_inputs(14, 3, p, q, m, n, r, with_S=with_S)
    x, S, A, B, bias, dy = (None if a is None else a.astype(float)
                            for a in (inp.x, inp.S, inp.A, inp.B, inp.bias, inp.dy))
    g = OK.backward(x, S, A, B, dy)
    named = dict(x=(x, g["dx"]), A=(A, g["dA"]), B=(B, g["dB"]), bias=(bias, g["dbias"]))
    if with_S:
        named["S"] = (S, g["dS"])
    else:
        assert g["dS"] is None
    for name, (arr, grad) in named.items():
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            args = dict(x=x, S=S, A=A, B=B, bias=bias)
            plus = arr.copy(); plus[idx] += 1.0
            minus = arr.copy(); minus[idx] -= 1.0
            args[name] = plus
            lp = _loss(args["x"], args["S"], args["A"], args["B"], args["bias"], dy)
            args[name] = minus
            lm = _loss(args["x"], args["S"], args["A"], args["B"], args["bias"], dy)
            fd[idx] = (lp - lm) / 2.0
        assert np.array_equal(fd, grad), name


def test_gradients_euler_identities():
    """Homogeneity: with zero bias, <x,dX> = <S,dS> = sum_i <A_i,dA_i> = sum_i <B_i,dB_i>
    = <dY, x W>, and entrywise S o dS = sum_i A_i o dA_i."""
    inp = kron_inputs(15, 37, 6, 5, 4, 3, 3, s_mode="uniform_zeroed", bias_mode="zeros")
    g = OK.backward(inp.x, inp.S, inp.A, inp.B, inp.dy)
    y = OK.forward(inp.x, inp.S, inp.A, inp.B, None)
    ref = np.sum(inp.dy.astype(float) * y)
    vals = [np.sum(inp.x * g["dx"]), np.sum(inp.S * g["dS"]), np.sum(inp.A * g["dA"]),
            np.sum(inp.B * g["dB"])]
    for v in vals:
        assert abs(v - ref) <= 1e-11 * abs(ref)
    np.testing.assert_allclose(inp.S * g["dS"], np.sum(inp.A * g["dA"], axis=0), rtol=1e-12, atol=1e-13)


def test_gradients_match_torch_autograd():
    """Library routine: torch autograd in float64 through torch.kron."""
    torch = pytest.importorskip("torch")
    inp = kron_inputs(16, 11, 4, 3, 3, 2, 2, s_mode="uniform_zeroed", bias_mode="normal")
    t = {k: torch.tensor(getattr(inp, k).astype(np.float64), requires_grad=True)
         for k in ("x", "S", "A", "B", "bias")}
    W = sum(torch.kron(t["S"] * t["A"][i], t["B"][i]) for i in range(2))
    y = t["x"] @ W + t["bias"]
    (y * torch.tensor(inp.dy.astype(np.float64))).sum().backward()
    g = OK.backward(inp.x, inp.S, inp.A, inp.B, inp.dy)
    for k, gk in (("x", "dx"), ("S", "dS"), ("A", "dA"), ("B", "dB"), ("bias", "dbias")):
        np.testing.assert_allclose(g[gk], t[k].grad.numpy(), rtol=1e-12, atol=1e-12)


def test_transpose_identity():
    """(C (x) B)^T = C^T (x) B^T: the backward's dX equals the forward of the transposed
    layer (p<->q, m<->n, A_i -> A_i^T, B_i -> B_i^T, S -> S^T) applied to dY."""
    inp = kron_inputs(17, 9, 4, 6, 3, 2, 3, s_mode="uniform_zeroed")
    g = OK.backward(inp.x, inp.S, inp.A, inp.B, inp.dy)
    yT = OK.forward(inp.dy, inp.S.T, inp.A.transpose(0, 2, 1), inp.B.transpose(0, 2, 1), None)
    np.testing.assert_allclose(g["dx"], yT, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------------
# Kronecker-sparse matrices
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("abcd", [(2, 3, 4, 2), (1, 3, 2, 1), (3, 1, 1, 2), (2, 2, 3, 1), (1, 1, 1, 3)])
def test_ks_support_is_kron_of_identity_and_ones(abcd):
    """KS abstract: support is a Kronecker product of identity and all-ones blocks;
    checked with numpy.kron, and the dense matrix of nonzero values has that support."""
    a, b, c, d = abcd
    ref = np.kron(np.kron(np.eye(a), np.ones((b, c))), np.eye(d))
    assert np.array_equal(OKS.support(a, b, c, d), ref)
    vals = np.random.default_rng(0).uniform(1, 2, (a, d, b, c))
    K = OKS.dense(vals, a, b, c, d)
    assert np.array_equal(K != 0, ref != 0)
    assert np.count_nonzero(K) == a * b * c * d


def test_ks_special_cases():
    """(1,b,c,1) is a dense b x c matrix; (a,b,c,1) is block diagonal (scipy.linalg.block_diag);
    (1,1,1,d) is diagonal."""
    rng = np.random.default_rng(1)
    v = rng.standard_normal((1, 1, 4, 5))
    assert np.array_equal(OKS.dense(v, 1, 4, 5, 1), v[0, 0])
    v = rng.standard_normal((3, 1, 2, 4))
    assert np.array_equal(OKS.dense(v, 3, 2, 4, 1), scipy.linalg.block_diag(*[v[i, 0] for i in range(3)]))
    v = rng.standard_normal((1, 6, 1, 1))
    assert np.array_equal(OKS.dense(v, 1, 1, 1, 6), np.diag(v.reshape(-1)))


def test_ks_d_interleave_matches_permutation_form():
    """I_a (x) M (x) I_d with M block values: for d > 1 the KS matrix is P^T blockdiag P,
    where P de-interleaves the delta index.  Checked against numpy.kron for a = 1."""
    rng = np.random.default_rng(2)
    b, c, d = 3, 2, 4
    M = rng.standard_normal((b, c))
    v = np.broadcast_to(M, (1, d, b, c)).copy()      # same block for every delta
    assert np.array_equal(OKS.dense(v, 1, b, c, d), np.kron(M, np.eye(d)))


@pytest.mark.parametrize("abcd", [(2, 3, 4, 3), (2, 1, 2, 3), (3, 2, 1, 2)])
def test_ks_value_layout_against_kron_sum(abcd):
    """The value layout vals[alpha][delta][beta][gamma]: with E_kk the one-hot k-th
    diagonal unit matrix, K = sum over (alpha, delta) of E_alpha,alpha (x) V[alpha][delta]
    (x) E_delta,delta, built with numpy.kron.  Every (alpha, delta) block holds distinct
    integers, so a swapped alpha/delta order or a transposed block changes K exactly."""
    a, b, c, d = abcd
    V = np.arange(1, a * d * b * c + 1, dtype=float).reshape(a, d, b, c)
    V = V * np.where(np.arange(V.size).reshape(V.shape) % 2, 1.0, -1.0)
    K = np.zeros((a * b * d, a * c * d))
    for al in range(a):
        Ea = np.zeros((a, a))
        Ea[al, al] = 1.0
        for de in range(d):
            Ed = np.zeros((d, d))
            Ed[de, de] = 1.0
            K += np.kron(np.kron(Ea, V[al, de]), Ed)
    assert np.array_equal(OKS.dense(V.reshape(-1), a, b, c, d), K)
    # the same, as the product X K on an integer X (exact in fp64)
    x = np.random.default_rng(7).integers(-3, 4, (5, a * b * d)).astype(float)
    assert np.array_equal(OKS.matmul(x, V, a, b, c, d), x @ K)


@pytest.mark.parametrize("abcd", [(2, 3, 4, 2), (1, 5, 2, 1), (3, 1, 2, 3)])
def test_ks_backward_exact_finite_differences(abcd):
    """L(x, vals) = <dY, X K> is linear in x and in vals, so the central difference with
    h = 1 is exact: on integer inputs every entry of dX and dvals equals its difference
    quotient bit for bit."""
    a, b, c, d = abcd
    rng = np.random.default_rng(7)
    N = 3
    x = rng.integers(-3, 4, (N, a * b * d)).astype(float)
    v = rng.integers(-3, 4, (a, d, b, c)).astype(float)
    dy = rng.integers(-3, 4, (N, a * c * d)).astype(float)
    L = lambda xx, vv: float(np.sum(dy * OKS.matmul(xx, vv, a, b, c, d)))
    g = OKS.backward(x, v, dy, a, b, c, d)
    for idx in np.ndindex(*x.shape):
        e = np.zeros_like(x); e[idx] = 1.0
        assert (L(x + e, v) - L(x - e, v)) / 2 == g["dx"][idx]
    for idx in np.ndindex(*v.shape):
        e = np.zeros_like(v); e[idx] = 1.0
        assert (L(x, v + e) - L(x, v - e)) / 2 == g["dvals"][idx]


def test_ks_backward_transpose_pattern_and_adjoint():
    """dX is the forward product with the transposed pattern I_a (x) 1_{c x b} (x) I_d and
    values vals[alpha][delta][gamma][beta] (K^T of a KS matrix is KS); and the adjoint
    identities <dX, X> = <dvals, vals> = <dY, X K> hold (the form is bilinear)."""
    a, b, c, d = 2, 5, 3, 4
    rng = np.random.default_rng(8)
    x = rng.standard_normal((6, a * b * d))
    v = rng.standard_normal((a, d, b, c))
    dy = rng.standard_normal((6, a * c * d))
    g = OKS.backward(x, v, dy, a, b, c, d)
    np.testing.assert_allclose(g["dx"], OKS.matmul(dy, v.transpose(0, 1, 3, 2), a, c, b, d), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(OKS.dense(v.transpose(0, 1, 3, 2), a, c, b, d), OKS.dense(v, a, b, c, d).T)
    form = np.sum(dy * OKS.matmul(x, v, a, b, c, d))
    assert np.isclose(np.sum(g["dx"] * x), form, rtol=1e-12)
    assert np.isclose(np.sum(g["dvals"] * v), form, rtol=1e-12)


@pytest.mark.parametrize("dims", [((2, 3), (3, 2), (2, 4)), ((1, 4), (5, 1), (3, 3)), ((4, 2), (2, 2), (1, 3))])
def test_ks_chain_triple_kronecker_matches_numpy(dims):
    """A (x) B (x) C as a chain of three KS factors equals numpy.kron(numpy.kron(A, B), C)
    bit for bit on integer values (mixed-product rule)."""
    rng = np.random.default_rng(9)
    A, B, C = (rng.integers(-3, 4, dm).astype(float) for dm in dims)
    x = rng.integers(-3, 4, (5, dims[0][0] * dims[1][0] * dims[2][0])).astype(float)
    want = x @ np.kron(np.kron(A, B), C)
    assert np.array_equal(OKS.chain(x, OKS.kron3_factors(A, B, C)), want)


def test_ks_chain_single_factor_and_associativity():
    """A one-factor chain is the KS matmul; a chain equals the product of its dense factors
    in any grouping."""
    rng = np.random.default_rng(10)
    f1 = (2, 3, 4, 2, rng.standard_normal((2, 2, 3, 4)))   # 12 -> 16
    f2 = (4, 2, 3, 2, rng.standard_normal((4, 2, 2, 3)))   # 16 -> 24
    x = rng.standard_normal((3, 12))
    assert np.array_equal(OKS.chain(x, [f1]), OKS.matmul(x, f1[4], *f1[:4]))
    K1, K2 = OKS.dense(f1[4], *f1[:4]), OKS.dense(f2[4], *f2[:4])
    np.testing.assert_allclose(OKS.chain(x, [f1, f2]), x @ (K1 @ K2), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("case", [(3, 2, 2, 3, 2), (2, 3, 3, 2, 1), (4, 4, 2, 2, 3)])
def test_kron_layer_equals_chain_of_two_ks_factors(case):
    """The layer factors as (I_p (x) B_all) followed by a KS factor carrying the C_i:
    x W = ks(p, m, r*n, 1; V1) then ks(1, r*p, q, n; V2) with V1[j][0][a][i*n+b] = B_i[a,b]
    and V2[0][b][j*r+i][k] = C_i[j,k]."""
    p, q, m, n, r = case
    inp = kron_inputs(18, 7, p, q, m, n, r, s_mode="uniform_zeroed")
    C = inp.S.astype(float)[None] * inp.A.astype(float)
    V1 = np.zeros((p, 1, m, r * n))
    for j in range(p):
        for i in range(r):
            V1[j, 0, :, i * n:(i + 1) * n] = inp.B[i]
    V2 = np.zeros((1, n, r * p, q))
    for b in range(n):
        for j in range(p):
            for i in range(r):
                V2[0, b, j * r + i, :] = C[i, j, :]
    z = OKS.matmul(inp.x, V1, p, m, r * n, 1)
    y = OKS.matmul(z, V2, 1, r * p, q, n)
    np.testing.assert_allclose(y, OK.forward(inp.x, inp.S, inp.A, inp.B, None), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------------
# Printed quantities
# ----------------------------------------------------------------------------------

def test_tutorial_printed_quantities():
    g = json.load(open(os.path.join(GOLDEN, "tutorial_printed_quantities.json")))
    f = g["facts"]
    L = f[0]["layer"]
    assert OK.param_count(L["in"], L["out"], L["m"], L["r"]) // 1000 == f[0]["kron_params_thousands_truncated"]
    assert round(OK.dense_param_count(L["in"], L["out"]) / 1e6, 2) == f[0]["dense_params_millions_rounded_2dp"]
    L = f[1]["layer"]
    p = L["in"] // L["m"]
    ratio = OK.vec_trick_macs_per_row(p, p, L["m"], L["m"], L["r"]) / OK.dense_macs_per_row(L["in"], L["out"])
    assert round(100 * ratio) == f[1]["mac_percent_rounded"]
    L = f[2]["layer"]
    assert L["in"] // L["m"] == f[2]["S_side"]
    assert (OK.param_count(L["in"], L["out"], L["m"], L["r"]) > OK.dense_param_count(L["in"], L["out"])) == f[2]["kron_exceeds_dense"]
    L = f[3]["layer"]
    inp = kron_inputs(19, 1, L["in"] // L["m"], L["out"] // L["m"], L["m"], L["m"], L["r"], s_mode="ones")
    assert inp.S.shape == (f[3]["S_side"], f[3]["S_side"]) and inp.A.shape[1:] == inp.S.shape
    L = f[4]["layer"]
    p = L["in"] // L["m"]
    ratio = OK.vec_trick_macs_per_row(p, p, L["m"], L["m"], L["r"]) / OK.dense_macs_per_row(L["in"], L["out"])
    rm = L["r"] / L["m"]
    assert abs(ratio - rm) <= f[4]["ratio_close_to_r_over_m_within"] * rm


def test_oracle_header_marks_test_infrastructure():
    assert "TEST INFRASTRUCTURE ONLY" in oracle.__doc__
    assert "parity unpinned" in oracle.__doc__  # states that no function is unpinned
