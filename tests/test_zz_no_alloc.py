"""kron_linear_bwd_noalloc (the backward with the library's fixed scratch as workspace)
against kron_linear_bwd (caller workspace), both called through the C ABI with ctypes:
the same kernels on the same inputs, so the results must agree bit for bit.  Two calls in
a row, the second smaller, show that what the first left in the scratch does not leak."""
import ctypes

import numpy as np
import pytest

from workloads import kron_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def lib():
    from kronecker_factored_structured_amd import _lib
    return _lib


def P(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _run(inp, noalloc, relu_mask=False):
    L = lib()
    sh = L.KronShape(inp.shape.N, inp.shape.p, inp.shape.q, inp.shape.m, inp.shape.n, inp.shape.r,
                     L.KRON_DX_RELU_MASK if relu_mask else 0)
    d = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    x, S, A, B, dy = (d(a) for a in (inp.x, inp.S, inp.A, inp.B, inp.dy))
    # outputs start as NaN so a skipped write cannot pass
    nan = lambda *s: torch.full(s, float("nan"), device="cuda")
    p, q, m, n, r, N = sh.p, sh.q, sh.m, sh.n, sh.r, sh.N
    dx, dA, dB, db = nan(N, p * m), nan(r, p, q), nan(r, m, n), nan(q * n)
    dS = nan(p, q) if S is not None else None
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if noalloc:
        st = L.lib().kron_linear_bwd_noalloc(ctypes.byref(sh), P(x), P(S), P(A), P(B), P(dy), P(dx), P(dS), P(dA),
                                             P(dB), P(db), stream)
    else:
        need = L.lib().kron_linear_bwd_workspace_bytes(ctypes.byref(sh))
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        st = L.lib().kron_linear_bwd(ctypes.byref(sh), P(x), P(S), P(A), P(B), P(dy), P(dx), P(dS), P(dA), P(dB),
                                     P(db), P(ws), ctypes.c_size_t(need), stream)
    assert st == 0, L.last_error()
    torch.cuda.synchronize()
    return {k: None if t is None else t.cpu().numpy() for k, t in
            dict(dx=dx, dS=dS, dA=dA, dB=dB, dbias=db).items()}


def _same(a, b):
    for k in a:
        if a[k] is None:
            assert b[k] is None
            continue
        assert np.array_equal(a[k].view(np.uint32), b[k].view(np.uint32)), k


@pytest.mark.parametrize("first,second", [
    # 20,000 rows of the 1024 x 1024 layer (m = 32, r = 4), then 1,031 rows of it
    ((20000, 32, 32, 32, 32, 4), (1031, 32, 32, 32, 32, 4)),
    # the training step's hidden layer, then a smaller rank-1 layer of other blocks
    ((3000, 16, 16, 64, 64, 2), (257, 32, 64, 24, 48, 1)),
])
def test_noalloc_matches_workspace_entry(first, second):
    for i, shp in enumerate((first, second)):
        N, p, q, m, n, r = shp
        print(f"[noalloc] call {i + 1}: N={N} p={p} q={q} m={m} n={n} r={r}", flush=True)
        inp = kron_inputs(50 + i, N, p, q, m, n, r, s_mode="uniform_zeroed", bias_mode="normal")
        ref = _run(inp, noalloc=False)
        got = _run(inp, noalloc=True)
        _same(ref, got)
        assert not np.isnan(got["dA"]).any()


def test_noalloc_relu_mask_and_no_S():
    inp = kron_inputs(53, 777, 32, 32, 32, 32, 4, s_mode="none", bias_mode="normal")
    _same(_run(inp, noalloc=False, relu_mask=True), _run(inp, noalloc=True, relu_mask=True))


def test_noalloc_refuses_shapes_beyond_the_scratch():
    """88 MiB of partial rows (the 1024 x 1024 layer with 16 x 16 blocks, r = 4, 20,000
    rows) exceed the 32 MiB scratch: refused on the host, nothing launched."""
    L = lib()
    sh = L.KronShape(20000, 64, 64, 16, 16, 4, 0)
    assert L.lib().kron_linear_bwd_workspace_bytes(ctypes.byref(sh)) > L.KRON_NOALLOC_SCRATCH_BYTES
    base = 0x7f0000000000
    ptrs = [ctypes.c_void_p(base + (k << 28)) for k in range(10)]
    st = L.lib().kron_linear_bwd_noalloc(ctypes.byref(sh), *ptrs, None)
    assert st == L.KRON_E_UNSUPPORTED
    assert "scratch" in L.last_error()
