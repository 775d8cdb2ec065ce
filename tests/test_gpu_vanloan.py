"""GPU parity of the Van Loan rank-r projection (kron_van_loan, through the C ABI) against
the oracle's LAPACK SVD of the rearranged matrix.  The GPU runs block subspace iteration in
fp32 from a seeded random start; bars: singular values within 2e-5 relative, factors and the
rank-r reconstruction within 1e-4 (max-norm relative).  The factor bar is looser than the
singular values' because the small s x s eigenproblem is solved on sigma^2, which costs
relative precision in the smaller terms (about eps * (sigma_1 / sigma_r)^2)."""
import numpy as np
import pytest

from _harness import dev, host, rel_err
from oracle import vanloan as OVL

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL_SIGMA = 2e-5
TOL_FACTOR = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def K():
    import kronecker_factored_structured_amd as mod
    return mod


def kron_sum(rng, p, q, m, n, weights, noise=0.0):
    W = sum(w * np.kron(rng.standard_normal((p, q)) / np.sqrt(p * q), rng.standard_normal((m, n)) / np.sqrt(m * n))
            for w in weights)
    if noise:
        W = W + noise * rng.standard_normal(W.shape) / np.sqrt(W.size)
    return W.astype(np.float32)


def run(W, p, q, m, n, r, s, iters, seed=0):
    omega = np.random.default_rng(seed).standard_normal((m * n, s)).astype(np.float32)
    print(f"[van loan] p={p} q={q} m={m} n={n} r={r} s={s} iters={iters}", flush=True)
    C, B, sig = K().kron_van_loan(dev(W), p, q, m, n, r, dev(omega), iters=iters)
    torch.cuda.synchronize()
    return host(C), host(B), host(sig)


def check(W, p, q, m, n, r, s, iters):
    C, B, sig = run(W, p, q, m, n, r, s, iters)
    Co, Bo, so = OVL.project(W, p, q, m, n, r)
    es, ec, eb = rel_err(sig, so), rel_err(C, Co), rel_err(B, Bo)
    er = rel_err(OVL.reconstruct(C, B), OVL.reconstruct(Co, Bo))
    print(f"   rel errors sigma {es:.2e} C {ec:.2e} B {eb:.2e} reconstruction {er:.2e}", flush=True)
    assert es <= TOL_SIGMA and ec <= TOL_FACTOR and eb <= TOL_FACTOR and er <= TOL_FACTOR
    assert np.all(np.diff(sig) <= 0)


def test_headline_layer_shape_decaying_spectrum():
    """1024 x 1024 W (p = q = m = n = 32): twelve Kronecker terms with weights 0.6^i plus
    noise, projected to r = 4 with a subspace of 12 and 8 power iterations."""
    rng = np.random.default_rng(80)
    W = kron_sum(rng, 32, 32, 32, 32, 0.6 ** np.arange(12), noise=1e-4)
    check(W, 32, 32, 32, 32, 4, 12, 8)


def test_exact_kronecker_sum_is_recovered():
    rng = np.random.default_rng(81)
    W = kron_sum(rng, 16, 16, 8, 8, [3.0, 2.0, 1.0])
    C, B, sig = run(W, 16, 16, 8, 8, 3, 8, 4)
    assert rel_err(OVL.reconstruct(C, B), W) <= TOL_FACTOR


def test_rectangular_factors():
    rng = np.random.default_rng(82)
    W = kron_sum(rng, 4, 8, 16, 6, [2.0, 1.5, 0.5, 0.2, 0.1], noise=1e-3)
    check(W, 4, 8, 16, 6, 2, 6, 10)


def test_deterministic():
    rng = np.random.default_rng(83)
    W = kron_sum(rng, 32, 32, 32, 32, 0.5 ** np.arange(6))
    a = run(W, 32, 32, 32, 32, 3, 8, 6)
    b = run(W, 32, 32, 32, 32, 3, 8, 6)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_odd_sizes():
    """Sides that are not multiples of 4 (scalar staging of the panels) and output tiles
    that run past the end of the rows."""
    rng = np.random.default_rng(84)
    W = kron_sum(rng, 3, 5, 7, 3, [3.0, 1.5, 0.6, 0.2], noise=1e-3)
    check(W, 3, 5, 7, 3, 2, 6, 12)


def test_tall_panel():
    """p*q = 4096 rows in the R side, above the 1024 that one workgroup holds in registers:
    the panel is orthonormalised in memory."""
    rng = np.random.default_rng(85)
    W = kron_sum(rng, 64, 64, 8, 8, [4.0, 2.0, 1.0, 0.5, 0.25, 0.12], noise=1e-3)
    check(W, 64, 64, 8, 8, 3, 10, 8)


def test_wide_subspace():
    """s = 20 (more than 16 panel columns): the register kernels' widest instantiation."""
    rng = np.random.default_rng(86)
    W = kron_sum(rng, 16, 16, 16, 16, 0.7 ** np.arange(24), noise=1e-4)
    check(W, 16, 16, 16, 16, 3, 20, 6)
