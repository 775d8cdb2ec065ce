"""GPU parity of ks_matmul (through the C ABI) against the fp64 oracle: fp32 and bf16
inputs (fp32 accumulation and output), support pattern bit-exact."""
import numpy as np
import pytest

from _harness import TOL_BF16, TOL_F32, dev, host, rel_err
from oracle import ks as OKS
from workloads import ks_inputs, vit_ks

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def K():
    import kronecker_factored_structured_amd as mod
    return mod


def run(inp):
    print(f"[ks] N={inp.x.shape[0]} abcd=({inp.a},{inp.b},{inp.c},{inp.d}) dtype={inp.dtype}", flush=True)
    if inp.dtype == "bf16":
        x = dev(inp.x_bits.view(np.int16)).view(torch.bfloat16)
        v = dev(inp.vals_bits.view(np.int16)).view(torch.bfloat16)
    else:
        x, v = dev(inp.x), dev(inp.vals)
    y = K().ks_matmul(x, v, inp.a, inp.b, inp.c, inp.d)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_vit_shape_full_size(dtype):
    """(a,b,c,d) = (2,48,192,4), 25,216 rows."""
    inp = vit_ks(dtype)
    y = run(inp)
    want = OKS.matmul(inp.x, inp.vals, inp.a, inp.b, inp.c, inp.d)
    e = rel_err(host(y), want)
    print(f"   rel error {e:.2e}", flush=True)
    assert e <= (TOL_F32 if dtype == "f32" else TOL_BF16)
    # both sides see the same bf16-rounded values, so fp32 accumulation is the only error
    assert e <= TOL_F32


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("abcd", [(2, 48, 192, 4), (2, 192, 48, 4), (1, 5, 7, 1), (3, 4, 2, 5), (4, 1, 1, 3),
                                  (1, 64, 64, 1), (2, 3, 130, 2)])
def test_support_bit_exact(dtype, abcd):
    """Identity input: Y = K exactly, values on the support and +0.0 off it."""
    a, b, c, d = abcd
    inp = ks_inputs(41, a * b * d, a, b, c, d, dtype)
    eye = np.eye(a * b * d, dtype=np.float32)
    if dtype == "bf16":
        from workloads import bf16_bits
        inp.x_bits = bf16_bits(eye)
    inp.x = eye
    y = run(inp)
    want = OKS.dense(inp.vals, a, b, c, d).astype(np.float32)
    got = y.cpu().numpy()
    assert np.array_equal(got.view(np.int32), want.view(np.int32))
    assert np.array_equal(got != 0, OKS.support(a, b, c, d) != 0)


@pytest.mark.parametrize("N", [0, 1, 63, 1001])
def test_ragged_rows(N):
    inp = ks_inputs(42, N, 2, 48, 192, 4, "f32")
    y = run(inp)
    if N:
        assert rel_err(host(y), OKS.matmul(inp.x, inp.vals, 2, 48, 192, 4)) <= TOL_F32
    else:
        assert y.shape == (0, 1536)


def test_kron_layer_equals_chain_of_ks_on_gpu():
    """The Kronecker layer factors as two KS matmuls: (I_p (x) B_all) then the C_i factor."""
    from workloads import kron_inputs
    p, q, m, n, r = 8, 6, 4, 5, 3
    inp = kron_inputs(43, 300, p, q, m, n, r, s_mode="uniform_zeroed")
    C = inp.S[None] * inp.A
    V1 = np.zeros((p, 1, m, r * n), np.float32)
    for j in range(p):
        for i in range(r):
            V1[j, 0, :, i * n:(i + 1) * n] = inp.B[i]
    V2 = np.zeros((1, n, r * p, q), np.float32)
    for b in range(n):
        for j in range(p):
            for i in range(r):
                V2[0, b, j * r + i, :] = C[i, j, :]
    z = K().ks_matmul(dev(inp.x), dev(V1), p, m, r * n, 1)
    y2 = K().ks_matmul(z, dev(V2), 1, r * p, q, n)
    y1 = K().kron_linear_fwd(dev(inp.x), dev(inp.S), dev(inp.A), dev(inp.B), None)
    assert rel_err(host(y2), host(y1)) <= TOL_F32


def _ks_dev_inputs(inp):
    if inp.dtype == "bf16":
        return (dev(inp.x_bits.view(np.int16)).view(torch.bfloat16),
                dev(inp.vals_bits.view(np.int16)).view(torch.bfloat16))
    return dev(inp.x), dev(inp.vals)


def _bf16_host(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bf16_output_vit_shape(dtype):
    """ks_matmul_out with a bf16 y (ViT shape, 25,216 rows).  Against the fp64 oracle each
    value is within a bf16 rounding (2^-9 relative for nearest even; truncation would
    reach 2^-7) plus the fp32 accumulation error; and it is exactly the nearest-even
    rounding of the same kernel's fp32 result (same products, same order)."""
    from workloads import bf16_bits, bf16_to_f32
    inp = vit_ks(dtype)
    x, v = _ks_dev_inputs(inp)
    print(f"[ks bf16 out] N={x.shape[0]} dtype={dtype}", flush=True)
    y16 = K().ks_matmul_out(x, v, inp.a, inp.b, inp.c, inp.d, out_dtype=torch.bfloat16)
    y32 = K().ks_matmul(x, v, inp.a, inp.b, inp.c, inp.d)
    torch.cuda.synchronize()
    assert y16.dtype == torch.bfloat16 and y16.shape == y32.shape
    bits = _bf16_host(y16)
    got = bf16_to_f32(bits).astype(np.float64)
    want = OKS.matmul(inp.x, inp.vals, inp.a, inp.b, inp.c, inp.d)
    scale = np.abs(want).max()
    assert np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(want) + TOL_F32 * scale)
    assert rel_err(got, want) <= TOL_BF16
    assert np.array_equal(bits, bf16_bits(y32.cpu().numpy()))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("abcd", [(2, 48, 192, 4), (1, 5, 7, 1), (1, 64, 64, 1), (3, 4, 2, 5)])
def test_bf16_output_support_bit_exact(dtype, abcd):
    """Identity input, bf16 y: the nearest-even bf16 of K on the support, +0 off it."""
    from workloads import bf16_bits
    a, b, c, d = abcd
    inp = ks_inputs(44, a * b * d, a, b, c, d, dtype)
    eye = np.eye(a * b * d, dtype=np.float32)
    if dtype == "bf16":
        inp.x_bits = bf16_bits(eye)
    inp.x = eye
    x, v = _ks_dev_inputs(inp)
    y = K().ks_matmul_out(x, v, a, b, c, d, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    dense = OKS.dense(inp.vals, a, b, c, d).astype(np.float32)
    assert np.array_equal(_bf16_host(y), bf16_bits(dense))


@pytest.mark.parametrize("N", [0, 1, 1001])
def test_bf16_output_ragged_rows(N):
    inp = ks_inputs(45, N, 2, 48, 192, 4, "bf16")
    x, v = _ks_dev_inputs(inp)
    y = K().ks_matmul_out(x, v, 2, 48, 192, 4, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert y.shape == (N, 1536)
    if N:
        from workloads import bf16_to_f32
        got = bf16_to_f32(_bf16_host(y)).astype(np.float64)
        assert rel_err(got, OKS.matmul(inp.x, inp.vals, 2, 48, 192, 4)) <= TOL_BF16


def _ks_bwd_case(inp, dy64, want_dx=True, want_dvals=True):
    x, v = _ks_dev_inputs(inp)
    if inp.dtype == "bf16":
        from workloads import bf16_bits, bf16_to_f32
        bits = bf16_bits(dy64.astype(np.float32))
        dy_host = bf16_to_f32(bits).reshape(dy64.shape)
        dy = dev(bits.view(np.int16)).view(torch.bfloat16)
    else:
        dy_host = dy64.astype(np.float32)
        dy = dev(dy_host)
    g = K().ks_matmul_bwd(x, v, dy, inp.a, inp.b, inp.c, inp.d, want_dx=want_dx, want_dvals=want_dvals)
    torch.cuda.synchronize()
    want = OKS.backward(inp.x, inp.vals, dy_host, inp.a, inp.b, inp.c, inp.d)
    return g, want


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ks_backward_vit_shape_full_size(dtype):
    """dx = dy K^T and dvals at (a,b,c,d) = (2,48,192,4), 25,216 rows, against the oracle
    on the same (bf16-rounded) inputs; both sides see identical values, so fp32
    accumulation is the only error."""
    inp = vit_ks(dtype)
    dy64 = np.random.default_rng(50).standard_normal((inp.x.shape[0], inp.a * inp.c * inp.d))
    print(f"[ks bwd] N={inp.x.shape[0]} dtype={dtype}", flush=True)
    g, want = _ks_bwd_case(inp, dy64)
    ex, ev = rel_err(host(g["dx"]), want["dx"]), rel_err(host(g["dvals"]), want["dvals"])
    print(f"   rel errors dx {ex:.2e} dvals {ev:.2e}", flush=True)
    assert ex <= TOL_F32 and ev <= TOL_F32


@pytest.mark.parametrize("N", [0, 1, 37, 300])
@pytest.mark.parametrize("abcd", [(1, 5, 7, 1), (3, 4, 2, 5), (2, 3, 130, 2), (4, 1, 1, 3), (1, 64, 64, 1),
                                  (2, 300, 3, 1), (2, 48, 192, 4), (1, 48, 192, 4)])
def test_ks_backward_shapes_and_ragged_rows(abcd, N):
    a, b, c, d = abcd
    inp = ks_inputs(46, N, a, b, c, d, "f32")
    dy64 = np.random.default_rng(51).standard_normal((N, a * c * d))
    g, want = _ks_bwd_case(inp, dy64)
    assert g["dx"].shape == (N, a * b * d) and g["dvals"].shape == (a, d, b, c)
    if N:
        assert rel_err(host(g["dx"]), want["dx"]) <= TOL_F32
        assert rel_err(host(g["dvals"]), want["dvals"]) <= TOL_F32
    else:
        assert np.all(host(g["dvals"]) == 0)


def test_ks_backward_single_outputs_and_determinism():
    inp = ks_inputs(47, 1000, 2, 48, 192, 4, "f32")
    dy64 = np.random.default_rng(52).standard_normal((1000, 1536))
    g1, want = _ks_bwd_case(inp, dy64, want_dx=False)
    assert g1["dx"] is None and rel_err(host(g1["dvals"]), want["dvals"]) <= TOL_F32
    g2, _ = _ks_bwd_case(inp, dy64, want_dvals=False)
    assert g2["dvals"] is None and rel_err(host(g2["dx"]), want["dx"]) <= TOL_F32
    g3, _ = _ks_bwd_case(inp, dy64)
    assert torch.equal(g3["dvals"], g1["dvals"]) and torch.equal(g3["dx"], g2["dx"])


def _chain_dev(factors, dtype):
    out = []
    for (a, b, c, d, v) in factors:
        v32 = np.ascontiguousarray(v, dtype=np.float32)
        if dtype == "bf16":
            from workloads import bf16_bits, bf16_to_f32
            bits = bf16_bits(v32)
            out.append(((a, b, c, d, bf16_to_f32(bits).reshape(v32.shape)),
                        dev(bits.view(np.int16)).view(torch.bfloat16)))
        else:
            out.append(((a, b, c, d, v32), dev(v32)))
    return out


def _run_chain(x32, factors, dtype="f32"):
    fs = _chain_dev(factors, dtype)
    if dtype == "bf16":
        from workloads import bf16_bits, bf16_to_f32
        bits = bf16_bits(x32)
        x_host = bf16_to_f32(bits).reshape(x32.shape)
        x = dev(bits.view(np.int16)).view(torch.bfloat16)
    else:
        x_host, x = x32, dev(x32)
    print(f"[ks chain] N={x32.shape[0]} factors={[f[0][:4] for f in fs]} dtype={dtype}", flush=True)
    y = K().ks_chain(x, [(t, *f[:4]) for f, t in fs])
    torch.cuda.synchronize()
    return host(y), OKS.chain(x_host, [f for f, _ in fs])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ks_chain_triple_kronecker(dtype):
    """x (A (x) B (x) C) for a 1024 x 1024 triple Kronecker product (8x8, 16x16, 8x8) as a
    fused three-factor chain, against the oracle's product of dense factors."""
    rng = np.random.default_rng(60)
    A, B, C = (rng.standard_normal(s) / np.sqrt(s[0]) for s in ((8, 8), (16, 16), (8, 8)))
    factors = OKS.kron3_factors(A, B, C)
    x = rng.standard_normal((2053, 1024)).astype(np.float32)
    y, want = _run_chain(x, factors, dtype)
    e = rel_err(y, want)
    print(f"   rel error {e:.2e}", flush=True)
    assert e <= TOL_F32


def test_ks_chain_monarch_two_factors():
    """A Monarch-style product: block-diagonal (a=32 blocks of 32x32), then the same
    pattern across the interleaved index (a=1, d=32), each block with its own values."""
    rng = np.random.default_rng(61)
    f1 = (32, 32, 32, 1, rng.standard_normal((32, 1, 32, 32)) / np.sqrt(32))
    f2 = (1, 32, 32, 32, rng.standard_normal((1, 32, 32, 32)) / np.sqrt(32))
    x = rng.standard_normal((1000, 1024)).astype(np.float32)
    y, want = _run_chain(x, [f1, f2])
    assert rel_err(y, want) <= TOL_F32


@pytest.mark.parametrize("N", [0, 1, 17])
def test_ks_chain_ragged_and_rectangular(N):
    rng = np.random.default_rng(62)
    f1 = (2, 3, 5, 4, rng.standard_normal((2, 4, 3, 5)))    # 24 -> 40
    f2 = (5, 8, 3, 1, rng.standard_normal((5, 1, 8, 3)))    # 40 -> 15
    f3 = (1, 15, 7, 1, rng.standard_normal((1, 1, 15, 7)))  # 15 -> 7
    x = rng.standard_normal((N, 24)).astype(np.float32)
    y, want = _run_chain(x, [f1, f2, f3])
    assert y.shape == (N, 7)
    if N:
        assert rel_err(y, want) <= TOL_F32


@pytest.mark.parametrize("N", [1, 16, 37, 600])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ks_chain_matrix_core_ragged_blocks(N, dtype):
    """Row widths that are multiples of 4 (the matrix-core chain) with b and c that are not
    multiples of 4 or 16 (3, 5, 6, 60, 28: zero padding of the 16x16x4 tiles), b longer than
    one chunk of beta steps (60), and a last row tile that is partly past N."""
    rng = np.random.default_rng(63)
    f1 = (4, 3, 5, 4, rng.standard_normal((4, 4, 3, 5)))      # 48 -> 80
    f2 = (5, 8, 6, 2, rng.standard_normal((5, 2, 8, 6)))      # 80 -> 60
    f3 = (1, 60, 28, 1, rng.standard_normal((1, 1, 60, 28)))  # 60 -> 28
    x = rng.standard_normal((N, 48)).astype(np.float32)
    y, want = _run_chain(x, [f1, f2, f3], dtype)
    assert y.shape == (N, 28)
    assert rel_err(y, want) <= TOL_F32   # bf16 inputs are exact in fp32; accumulation is fp32


@pytest.mark.parametrize("N", [5, 77])
@pytest.mark.parametrize("case", ["three", "two"])
def test_ks_chain_register_layouts_partly_used(N, case):
    """Chains that the register-resident kernels take with slots to spare: fewer tasks per
    wavefront and fewer beta steps than the layout holds, and c = 4 (one quarter of a
    16-column tile live)."""
    rng = np.random.default_rng(64)
    if case == "three":
        fs = [(1, 4, 8, 64, rng.standard_normal((1, 64, 4, 8))),     # 256 -> 512
              (8, 16, 8, 4, rng.standard_normal((8, 4, 16, 8))),     # 512 -> 256
              (64, 4, 4, 1, rng.standard_normal((64, 1, 4, 4)))]     # 256 -> 256
        w0 = 256
    else:
        fs = [(16, 32, 16, 1, rng.standard_normal((16, 1, 32, 16))),  # 512 -> 256
              (1, 16, 32, 16, rng.standard_normal((1, 16, 16, 32)))]  # 256 -> 512
        w0 = 512
    x = rng.standard_normal((N, w0)).astype(np.float32)
    y, want = _run_chain(x, fs)
    assert rel_err(y, want) <= TOL_F32


@pytest.mark.parametrize("N", [1, 17, 1000])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_bf16_vit_shape_ragged_rows(N, out_dtype):
    """bf16 inputs at the ViT shape (bf16 matrix instructions) with row counts that leave a
    partial 16-row tile, fp32 and bf16 outputs."""
    inp = ks_inputs(48, N, 2, 48, 192, 4, "bf16")
    x, v = _ks_dev_inputs(inp)
    od = torch.float32 if out_dtype == "f32" else torch.bfloat16
    y = K().ks_matmul_out(x, v, 2, 48, 192, 4, out_dtype=od)
    torch.cuda.synchronize()
    want = OKS.matmul(inp.x, inp.vals, 2, 48, 192, 4)
    if out_dtype == "f32":
        assert rel_err(host(y), want) <= TOL_F32
    else:
        from workloads import bf16_to_f32
        assert rel_err(bf16_to_f32(_bf16_host(y)).astype(np.float64), want) <= TOL_BF16


@pytest.mark.parametrize("N", [1, 37, 300])
@pytest.mark.parametrize("abcd", [(2, 48, 192, 4), (1, 16, 32, 4), (2, 32, 48, 4), (1, 64, 16, 4), (1, 16, 256, 4)])
def test_ks_backward_bf16_shapes_and_ragged_rows(abcd, N):
    """bf16 inputs: dvals on bf16 matrix instructions for each number of 16-wide beta tiles
    (b = 16 .. 64), the fp32-instruction kernel for c = 256 (more gamma tiles than the bf16
    kernel's workgroup holds), dx through the bf16 split-contraction kernel at the ViT shape;
    row counts that end inside a 16-row step."""
    a, b, c, d = abcd
    inp = ks_inputs(49, N, a, b, c, d, "bf16")
    dy64 = np.random.default_rng(53).standard_normal((N, a * c * d))
    g, want = _ks_bwd_case(inp, dy64)
    assert rel_err(host(g["dx"]), want["dx"]) <= TOL_F32
    assert rel_err(host(g["dvals"]), want["dvals"]) <= TOL_F32
