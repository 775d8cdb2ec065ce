"""GPU parity of kron_linear_fwd / kron_linear_bwd (through the C ABI) against the fp64
oracle, on the seeded workloads and on edge cases.  Bar: max-norm relative error
<= 1e-5 per output tensor (fp32 inputs); bitwise where the arithmetic is exact."""
import numpy as np
import pytest

from _harness import TOL_F32, bits, dev, host, rel_err
from oracle import kron as OK
from workloads import gpt2_ffn_layers, headline_layer, integer_kron_inputs, kron_inputs, tiny_layer

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def K():
    import kronecker_factored_structured_amd as mod
    return mod


def run_layer(inp, want_dx=True, relu=False, relu_mask=False, sparse_rows=False):
    """Forward and backward on the GPU; returns numpy fp64 results."""
    print(f"[kron] N={inp.shape.N} p={inp.shape.p} q={inp.shape.q} m={inp.shape.m} n={inp.shape.n} "
          f"r={inp.shape.r} S={'yes' if inp.S is not None else 'no'} seed={inp.seed} sparse_rows={sparse_rows}",
          flush=True)
    x, S, A, B, bias, dy = (dev(a) for a in (inp.x, inp.S, inp.A, inp.B, inp.bias, inp.dy))
    y = K().kron_linear_fwd(x, S, A, B, bias, relu=relu, sparse_rows=sparse_rows)
    g = K().kron_linear_bwd(x, S, A, B, dy, want_dx=want_dx, want_dbias=bias is not None, relu_mask=relu_mask,
                            sparse_rows=sparse_rows)
    torch.cuda.synchronize()
    return host(y), {k: host(v) for k, v in g.items()}


def compare_layer(inp, tol=TOL_F32, want_dx=True, sparse_rows=False):
    y, g = run_layer(inp, want_dx=want_dx, sparse_rows=sparse_rows)
    W = OK.weight(inp.S, inp.A, inp.B)
    yo = inp.x.astype(np.float64) @ W + (0.0 if inp.bias is None else inp.bias.astype(np.float64))
    go = OK.backward(inp.x, inp.S, inp.A, inp.B, inp.dy, want_dx=want_dx, W=W)
    errs = {"y": rel_err(y, yo)}
    for k in ("dx", "dS", "dA", "dB", "dbias"):
        if go[k] is None or g[k] is None:
            assert g[k] is None or k == "dbias", k
            continue
        errs[k] = rel_err(g[k], go[k])
    print("   rel errors:", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    for k, e in errs.items():
        assert e <= tol, (k, e)
    return errs


def test_tiny_layer():
    """64 rows, 64x64, m = 8, r = 2, S = ones: forward and all five gradients."""
    compare_layer(tiny_layer())


def test_headline_layer_full_size():
    """20,000 rows, 1024x1024, m = 32, r = 4, half of S zeroed."""
    compare_layer(headline_layer())


# With one workgroup of four row-owning wavefronts per compute unit, 1 and 257 rows are
# split by rank only, 1031 and 3500 leave a split tail after whole rounds, 2000 leaves a
# tail too long to split and 2048 none.
@pytest.mark.parametrize("N", [0, 1, 3, 257, 1031, 2000, 2048, 3500])
def test_headline_shape_ragged_rows(N):
    inp = headline_layer(N=N)
    if N == 0:
        y, g = run_layer(inp)
        assert y.shape == (0, 1024)
        for k in ("dS", "dA", "dB", "dbias"):
            assert not np.any(g[k]), k          # empty batch: zero parameter gradients
        return
    compare_layer(inp)


# Row-sparse S (whole rows of the mask zero): the forward's row map compacts the nonzero
# rows of C = S o A_i to the front and runs only the 16-row tiles that hold them.
@pytest.mark.parametrize("shape,frac", [((32, 32, 32, 32, 4), 0.75),     # 8 rows left: one tile
                                        ((32, 32, 32, 32, 4), 0.5),      # 16 rows: one full tile
                                        ((32, 32, 32, 32, 4), 15 / 32),  # 17 rows: two tiles, permuted
                                        ((32, 32, 32, 32, 4), 1.0),      # S == 0: y = bias
                                        ((32, 32, 32, 32, 1), 0.75),
                                        ((32, 32, 32, 32, 2), 0.25),
                                        ((64, 32, 48, 24, 4), 0.75),     # 16 of 64 rows: one tile
                                        ((64, 32, 48, 24, 2), 0.6),      # 26 rows: two tiles
                                        ((64, 32, 48, 24, 1), 0.3),      # 45 rows: three tiles
                                        ((32, 64, 24, 48, 4), 0.75),
                                        ((16, 16, 64, 64, 2), 0.5)])     # one tile: no map
def test_row_sparse_S(shape, frac):
    p, q, m, n, r = shape
    inp = kron_inputs(44, 1031, p, q, m, n, r, s_mode="rows_zeroed", zero_frac=frac, bias_mode="normal")
    compare_layer(inp, sparse_rows=True)
    compare_layer(inp)                      # without the hint: the dense path, same results


def test_row_sparse_S_full_size_and_relu():
    """20,000 rows of the 1024 x 1024 layer with 24 of S's 32 rows zero, ReLU output."""
    inp = kron_inputs(45, 20000, 32, 32, 32, 32, 4, s_mode="rows_zeroed", zero_frac=0.75, bias_mode="normal")
    compare_layer(inp, sparse_rows=True)
    x, S, A, B, bias = (dev(a) for a in (inp.x, inp.S, inp.A, inp.B, inp.bias))
    y = K().kron_linear_fwd(x, S, A, B, bias, relu=True, sparse_rows=True)
    W = OK.weight(inp.S, inp.A, inp.B)
    rows = np.arange(0, 20000, 97)
    want = np.maximum(inp.x[rows].astype(np.float64) @ W + inp.bias, 0)
    assert rel_err(host(y)[rows], want) <= TOL_F32


def test_zero_rows_of_A_without_S():
    """S absent: rows of C = A_i that are zero in every rank are skipped the same way."""
    inp = kron_inputs(46, 777, 32, 32, 32, 32, 4, s_mode="none", bias_mode="normal")
    inp.A[:, [0, 3, 4, 9, 10, 11, 20, 21, 22, 23, 24, 25, 26, 27, 30, 31, 1, 2], :] = 0.0
    compare_layer(inp, sparse_rows=True)


def _zero_blocks(S, blocks):
    for tj, tk in blocks:
        S[16 * tj:16 * tj + 16, 16 * tk:16 * tk + 16] = 0.0


@pytest.mark.parametrize("case", ["diagonal", "one_block", "rows_and_block", "all_zero"])
def test_block_sparse_S(case):
    """S with whole 16 x 16 blocks zero (the forward's tile mask, taken in the row map's
    order, skips the stage-2 steps over them): block-diagonal S, one zero block, zero rows
    that are not block-aligned together with a zero block, and S = 0.  With and without the
    hint, against the oracle."""
    inp = kron_inputs(47, 1031, 32, 32, 32, 32, 4, s_mode="uniform", bias_mode="normal")
    if case == "diagonal":
        _zero_blocks(inp.S, [(0, 1), (1, 0)])
    elif case == "one_block":
        _zero_blocks(inp.S, [(0, 1)])
    elif case == "rows_and_block":
        inp.S[[2, 5, 7, 11, 13, 17, 19, 23, 29], :] = 0.0
        _zero_blocks(inp.S, [(1, 1)])
    else:
        inp.S[:] = 0.0
    compare_layer(inp, sparse_rows=True)
    compare_layer(inp)


@pytest.mark.parametrize("shape", [(32, 64, 24, 48, 2), (64, 32, 48, 24, 2)])
def test_block_sparse_S_gpt2_shapes(shape):
    """The tile mask on rectangular shapes (2 x 4 and 4 x 2 tiles of C), seeded zero blocks."""
    p, q, m, n, r = shape
    inp = kron_inputs(48, 517, p, q, m, n, r, s_mode="blocks_zeroed", zero_frac=0.5, bias_mode="normal")
    compare_layer(inp, sparse_rows=True)


@pytest.mark.parametrize("frac,relu_mask,want_dx", [(0.75, False, True), (0.75, True, True), (0.5, False, False),
                                                     (15 / 32, True, True), (1.0, False, True), (0.25, False, True)])
def test_row_sparse_S_backward_variants(frac, relu_mask, want_dx):
    """The whole-row backward with the row map: no dX, dX, dX o [x > 0]; 8, 16, 17, 0 and 24
    nonzero rows (one tile, one tile, two permuted tiles, S == 0, two tiles)."""
    inp = kron_inputs(49, 2000, 32, 32, 32, 32, 4, s_mode="rows_zeroed", zero_frac=frac, bias_mode="normal")
    if relu_mask:
        inp.x = np.maximum(inp.x, 0).astype(np.float32)
    y, g = run_layer(inp, want_dx=want_dx, relu_mask=relu_mask, sparse_rows=True)
    W = OK.weight(inp.S, inp.A, inp.B)
    assert rel_err(y, inp.x.astype(np.float64) @ W + inp.bias) <= TOL_F32
    go = OK.backward(inp.x, inp.S, inp.A, inp.B, inp.dy, want_dx=want_dx, W=W)
    if want_dx:
        want = go["dx"] * (inp.x > 0) if relu_mask else go["dx"]
        assert rel_err(g["dx"], want) <= TOL_F32
    else:
        assert g["dx"] is None
    for k in ("dS", "dA", "dB", "dbias"):
        assert rel_err(g[k], go[k]) <= TOL_F32, k


def test_sparse_rows_hint_on_dense_S():
    """The hint on an S with no empty row: identity map, every tile runs, same results."""
    compare_layer(kron_inputs(47, 1031, 32, 32, 32, 32, 4, s_mode="uniform_zeroed", bias_mode="normal"),
                  sparse_rows=True)
    compare_layer(kron_inputs(48, 515, 64, 32, 48, 24, 4, s_mode="uniform_zeroed", bias_mode="normal"),
                  sparse_rows=True)


def test_mlp_hidden_layer_shape():
    """Hidden layer of the training step: 1024x1024, m = 64 (p = q = 16), r = 2."""
    compare_layer(kron_inputs(31, 3000, 16, 16, 64, 64, 2, s_mode="ones"))


@pytest.mark.parametrize("r", [1, 2, 4, 8])
def test_gpt2_ffn_layers(r):
    """768 -> 3072 (A_i 32x64, B_i 24x48) and 3072 -> 768 (A_i 64x32, B_i 48x24), 8192 rows."""
    up, down = gpt2_ffn_layers(r)
    compare_layer(up)
    compare_layer(down)


@pytest.mark.parametrize("shape", [(32, 64, 24, 48), (64, 32, 48, 24)])
def test_gpt2_rank8_without_S_ragged(shape):
    """r = 8 at the GPT-2 pair, where the forward stages one rank's raw factors at a time;
    no S (A alone forms C_i), a ragged row count, bias."""
    p, q, m, n = shape
    compare_layer(kron_inputs(35, 1001, p, q, m, n, 8, s_mode="none", bias_mode="normal"))


@pytest.mark.parametrize("case", [(3, 5, 7, 2, 3), (1, 1, 4, 6, 2), (6, 4, 1, 1, 5), (5, 3, 2, 9, 16),
                                  (2, 7, 3, 3, 1), (33, 17, 5, 3, 2)])
def test_odd_shapes_with_bias_and_S(case):
    p, q, m, n, r = case
    compare_layer(kron_inputs(32, 203, p, q, m, n, r, s_mode="uniform_zeroed", bias_mode="normal"))


@pytest.mark.parametrize("case", [(128, 128, 8, 8, 1), (64, 64, 16, 16, 2)])
def test_tutorial_small_block_layers(case):
    """The tutorial's 1024 x 1024 layer with 8 x 8 and 16 x 16 blocks (generic kernels,
    S and C_i staged in up to 148 KB of LDS)."""
    p, q, m, n, r = case
    compare_layer(kron_inputs(34, 37, p, q, m, n, r, s_mode="uniform_zeroed", bias_mode="normal"))


def test_without_S_and_without_dx():
    compare_layer(kron_inputs(33, 500, 32, 32, 32, 32, 4, s_mode="none", bias_mode="normal"), want_dx=False)


def test_relu_flags():
    """KRON_RELU_OUT on the forward, KRON_DX_RELU_MASK on the backward (dx o [x > 0])."""
    inp = kron_inputs(34, 777, 16, 16, 64, 64, 2, s_mode="ones", bias_mode="normal")
    xr = np.maximum(inp.x, 0).astype(np.float32)       # x as the output of a ReLU
    inp.x = xr
    y, g = run_layer(inp, relu=True, relu_mask=True)
    W = OK.weight(inp.S, inp.A, inp.B)
    yo = np.maximum(xr.astype(np.float64) @ W + inp.bias, 0)
    assert rel_err(y, yo) <= TOL_F32
    go = OK.backward(xr, inp.S, inp.A, inp.B, inp.dy, W=W)
    assert rel_err(g["dx"], go["dx"] * (xr > 0)) <= TOL_F32
    assert np.all(g["dx"][xr <= 0] == 0)


@pytest.mark.parametrize("N", [1031, 1900])
def test_relu_mask_headline_shape(N):
    """dx o [x > 0] on the 32 x 32-block layer with r = 4, with and without rank-split rows."""
    inp = kron_inputs(39, N, 32, 32, 32, 32, 4, s_mode="uniform_zeroed", bias_mode="normal")
    xr = np.maximum(inp.x, 0).astype(np.float32)
    inp.x = xr
    y, g = run_layer(inp, relu_mask=True)
    W = OK.weight(inp.S, inp.A, inp.B)
    go = OK.backward(xr, inp.S, inp.A, inp.B, inp.dy, W=W)
    assert rel_err(g["dx"], go["dx"] * (xr > 0)) <= TOL_F32
    assert np.all(g["dx"][xr <= 0] == 0)
    for k in ("dS", "dA", "dB", "dbias"):
        assert rel_err(g[k], go[k]) <= TOL_F32, k


@pytest.mark.parametrize("shape", [(32, 64, 24, 48), (64, 32, 48, 24)])
def test_rank8_in_chunks_with_S_and_bias(shape):
    """r = 8 runs as two passes of four ranks: dX written then added to, dS summed over
    the passes, dbias from the first pass."""
    p, q, m, n = shape
    compare_layer(kron_inputs(37, 1031, p, q, m, n, 8, s_mode="uniform_zeroed", bias_mode="normal"))


def test_rank8_in_chunks_relu_mask():
    """The ReLU mask of dX is applied once, to the sum over the rank passes."""
    inp = kron_inputs(38, 515, 32, 64, 24, 48, 8, s_mode="uniform", bias_mode="normal")
    xr = np.maximum(inp.x, 0).astype(np.float32)
    inp.x = xr
    y, g = run_layer(inp, relu_mask=True)
    W = OK.weight(inp.S, inp.A, inp.B)
    go = OK.backward(xr, inp.S, inp.A, inp.B, inp.dy, W=W)
    assert rel_err(g["dx"], go["dx"] * (xr > 0)) <= TOL_F32
    assert np.all(g["dx"][xr <= 0] == 0)
    for k in ("dS", "dA", "dB", "dbias"):
        assert rel_err(g[k], go[k]) <= TOL_F32, k


def test_one_hot_rows_bit_exact_rank1():
    """fwd(I_in) with zero bias reproduces W; for r = 1 and S absent every entry of W is a
    single fp32 product A[j,k]*B[a,b], so the GPU result must equal it bit for bit."""
    p, q, m, n = 32, 32, 32, 32
    inp = kron_inputs(35, 1, p, q, m, n, 1, s_mode="none")
    eye = np.eye(p * m, dtype=np.float32)
    x, A, B = dev(eye), dev(inp.A), dev(inp.B)
    y = K().kron_linear_fwd(x, None, A, B, None)
    want = np.kron(inp.A[0], inp.B[0]).astype(np.float32)   # fp32 products, correctly rounded
    got = y.cpu().numpy()
    assert np.array_equal(got.view(np.int32), want.view(np.int32))


def test_one_hot_rows_reproduce_W_with_sparse_S():
    inp = headline_layer(N=1)
    eye = np.eye(1024, dtype=np.float32)
    y = K().kron_linear_fwd(dev(eye), dev(inp.S), dev(inp.A), dev(inp.B), None)
    W = OK.weight(inp.S, inp.A, inp.B)
    assert rel_err(host(y), W) <= TOL_F32
    assert np.all(host(y)[W == 0] == 0)               # zero blocks of S stay exactly zero


def test_integer_inputs_exact():
    """Small-integer inputs keep every partial sum exact in fp32: results equal the oracle bitwise."""
    inp = integer_kron_inputs(36, 300, 8, 8, 8, 8, 2, lo=-2, hi=3)
    y, g = run_layer(inp)
    W = OK.weight(inp.S, inp.A, inp.B)
    assert np.array_equal(y, inp.x.astype(np.float64) @ W + inp.bias)
    go = OK.backward(inp.x, inp.S, inp.A, inp.B, inp.dy, W=W)
    for k in ("dx", "dS", "dA", "dB", "dbias"):
        assert np.array_equal(g[k], go[k]), k


def test_transpose_identity_on_gpu():
    """dX of the backward equals the forward of the transposed layer applied to dY."""
    inp = kron_inputs(37, 900, 32, 64, 24, 48, 2, s_mode="uniform_zeroed")
    S, A, B, dy = dev(inp.S), dev(inp.A), dev(inp.B), dev(inp.dy)
    g = K().kron_linear_bwd(dev(inp.x), S, A, B, dy)
    yT = K().kron_linear_fwd(dy, S.t().contiguous(), A.transpose(1, 2).contiguous(),
                             B.transpose(1, 2).contiguous(), None)
    assert rel_err(host(g["dx"]), host(yT)) <= TOL_F32


def test_euler_identities_on_gpu_outputs():
    """<x,dX> = <S,dS> = sum<A,dA> = sum<B,dB> = <dY, xW> at full headline size."""
    inp = headline_layer()
    y, g = run_layer(inp)
    ref = np.sum(inp.dy.astype(np.float64) * y)
    for v in (np.sum(inp.x * g["dx"]), np.sum(inp.S * g["dS"]), np.sum(inp.A * g["dA"]), np.sum(inp.B * g["dB"])):
        assert abs(v - ref) <= 1e-5 * np.sqrt(np.sum(inp.dy.astype(np.float64) ** 2) * np.sum(y ** 2))


def test_deterministic():
    inp = headline_layer(N=4099)
    x, S, A, B, dy = (dev(a) for a in (inp.x, inp.S, inp.A, inp.B, inp.dy))
    outs = []
    for _ in range(2):
        y = K().kron_linear_fwd(x, S, A, B, None)
        g = K().kron_linear_bwd(x, S, A, B, dy)
        outs.append([bits(y)] + [bits(g[k]) for k in ("dx", "dS", "dA", "dB", "dbias")])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_kron_linear_module_autograd():
    """The torch module's autograd path gives the oracle's gradients."""
    mod = K()
    torch.manual_seed(0)
    layer = mod.KronLinear(256, 512, m=16, r=3, n=32, with_S=True, device="cuda")
    inp = kron_inputs(38, 300, 16, 16, 16, 32, 3, s_mode="uniform_zeroed", bias_mode="normal")
    with torch.no_grad():
        layer.S.copy_(dev(inp.S)); layer.A.copy_(dev(inp.A)); layer.B.copy_(dev(inp.B))
        layer.bias.copy_(dev(inp.bias))
    x = dev(inp.x).requires_grad_(True)
    y = layer(x)
    y.backward(dev(inp.dy))
    go = OK.backward(inp.x, inp.S, inp.A, inp.B, inp.dy)
    assert rel_err(host(y), OK.forward(inp.x, inp.S, inp.A, inp.B, inp.bias)) <= TOL_F32
    for t, k in ((x, "dx"), (layer.S, "dS"), (layer.A, "dA"), (layer.B, "dB"), (layer.bias, "dbias")):
        assert rel_err(host(t.grad), go[k]) <= TOL_F32, k


def test_kron_linear_module_autograd_relu_and_penalty():
    """KronLinear(relu=True): y = max(x W + bias, 0); the loss <R, y> + lam * sum|S| through
    autograd gives the oracle's gradients with dY = R o [y > 0] (the mask taken from the
    GPU's own y, so a sign decided differently at a rounding tie cannot flip a row), and
    dS gains lam * sign(S)."""
    mod = K()
    lam = 3e-3
    layer = mod.KronLinear(1024, 1024, m=32, r=4, with_S=True, relu=True, device="cuda")
    inp = kron_inputs(43, 1031, 32, 32, 32, 32, 4, s_mode="uniform_zeroed", bias_mode="normal")
    with torch.no_grad():
        layer.S.copy_(dev(inp.S)); layer.A.copy_(dev(inp.A)); layer.B.copy_(dev(inp.B))
        layer.bias.copy_(dev(inp.bias))
        layer.S[0, :5] = -layer.S[0, :5]           # negative entries: sign(S) = -1 there
    S_host = host(layer.S).astype(np.float32)
    x = dev(inp.x).requires_grad_(True)
    y = layer(x)
    pen = layer.l1_penalty()
    assert pen.dim() == 0
    loss = (y * dev(inp.dy)).sum() + lam * pen
    loss.backward()
    torch.cuda.synchronize()
    yh = host(y)
    W = OK.weight(S_host, inp.A, inp.B)
    assert rel_err(yh, np.maximum(inp.x.astype(np.float64) @ W + inp.bias, 0)) <= TOL_F32
    assert abs(host(pen) - np.abs(S_host.astype(np.float64)).sum()) <= TOL_F32 * np.abs(S_host).sum()
    dym = inp.dy * (yh > 0)
    go = OK.backward(inp.x, S_host, inp.A, inp.B, dym, W=W)
    go["dS"] = go["dS"] + lam * np.sign(S_host.astype(np.float64))
    for t, k in ((x, "dx"), (layer.S, "dS"), (layer.A, "dA"), (layer.B, "dB"), (layer.bias, "dbias")):
        assert rel_err(host(t.grad), go[k]) <= TOL_F32, k


# ---------------------------------------------------------------------------------
# Small blocks (m = n in {2, 4, 8}, p and q multiples of 16): the matrix-core GEMM path.
# The tutorial's 1024 x 1024 layer with 8 x 8, 4 x 4 and 2 x 2 blocks is p = q = 128, 256, 512.
# ---------------------------------------------------------------------------------

@pytest.mark.parametrize("case", [(128, 8, 1), (128, 8, 2), (128, 8, 4), (256, 4, 1), (256, 4, 2), (512, 2, 1),
                                  (512, 2, 2)])
def test_small_block_layers(case):
    """1031 rows (a ragged 64-row tile), half of S zeroed, bias."""
    p, m, r = case
    compare_layer(kron_inputs(40, 1031, p, p, m, m, r, s_mode="uniform_zeroed", bias_mode="normal"))


@pytest.mark.parametrize("case", [(48, 80, 4, 3), (160, 32, 8, 2), (528, 16, 2, 1), (16, 16, 8, 5)])
def test_small_block_partial_tiles(case):
    """p, q not multiples of the kernels' tile widths (16-multiples only)."""
    p, q, m, r = case
    compare_layer(kron_inputs(41, 333, p, q, m, m, r, s_mode="uniform_zeroed", bias_mode="normal"))


@pytest.mark.parametrize("N", [0, 1, 63, 65])
def test_small_block_ragged_rows(N):
    inp = kron_inputs(42, N, 128, 128, 8, 8, 2, s_mode="uniform_zeroed", bias_mode="normal")
    if N == 0:
        y, g = run_layer(inp)
        assert y.shape == (0, 1024)
        for k in ("dS", "dA", "dB", "dbias"):
            assert not np.any(g[k]), k
        return
    compare_layer(inp)


@pytest.mark.parametrize("case", [(128, 8, 1), (256, 4, 2)])
def test_small_block_full_size(case):
    """20,000 rows of the 1024 x 1024 layer (the tutorial's batch) against the oracle."""
    p, m, r = case
    compare_layer(kron_inputs(43, 20000, p, p, m, m, r, s_mode="uniform_zeroed", bias_mode="normal"))


def test_small_blocks_beyond_rank16_take_the_generic_kernels():
    """r = 17 at 8 x 8 blocks is past the small-block kernels' rank limit and runs on the
    generic kernels (S and C_i of 128 x 128 fit their LDS)."""
    compare_layer(kron_inputs(49, 37, 128, 128, 8, 8, 17, s_mode="uniform_zeroed", bias_mode="normal"))


def test_small_block_rank16_without_S_and_dx():
    compare_layer(kron_inputs(44, 200, 128, 128, 8, 8, 16, s_mode="none", bias_mode="normal"), want_dx=False)
    compare_layer(kron_inputs(45, 200, 256, 256, 4, 4, 16, s_mode="none", bias_mode="none"))


@pytest.mark.parametrize("m", [8, 4, 2])
def test_small_block_relu_flags(m):
    """ReLU on the forward; the dX mask applies once, to the sum over the ranks."""
    p = 1024 // m
    inp = kron_inputs(46, 300, p, p, m, m, 3, s_mode="uniform", bias_mode="normal")
    xr = np.maximum(inp.x, 0).astype(np.float32)
    inp.x = xr
    y, g = run_layer(inp, relu=True, relu_mask=True)
    W = OK.weight(inp.S, inp.A, inp.B)
    assert rel_err(y, np.maximum(xr.astype(np.float64) @ W + inp.bias, 0)) <= TOL_F32
    go = OK.backward(xr, inp.S, inp.A, inp.B, inp.dy, W=W)
    assert rel_err(g["dx"], go["dx"] * (xr > 0)) <= TOL_F32
    assert np.all(g["dx"][xr <= 0] == 0)
    for k in ("dS", "dA", "dB", "dbias"):
        assert rel_err(g[k], go[k]) <= TOL_F32, k


def test_small_block_integer_inputs_exact():
    """Small-integer inputs keep every partial sum exact: the small-block path equals the
    oracle bit for bit (this pins its indexing independently of rounding)."""
    for p, m in ((128, 8), (256, 4)):
        inp = integer_kron_inputs(47, 20, p, p, m, m, 2, lo=-1, hi=2)
        y, g = run_layer(inp)
        W = OK.weight(inp.S, inp.A, inp.B)
        assert np.array_equal(y, inp.x.astype(np.float64) @ W + inp.bias)
        go = OK.backward(inp.x, inp.S, inp.A, inp.B, inp.dy, W=W)
        for k in ("dx", "dS", "dA", "dB", "dbias"):
            assert np.array_equal(g[k], go[k]), (p, k)


def test_small_block_deterministic():
    inp = kron_inputs(48, 4099, 256, 256, 4, 4, 2, s_mode="uniform_zeroed", bias_mode="normal")
    x, S, A, B, dy = (dev(a) for a in (inp.x, inp.S, inp.A, inp.B, inp.dy))
    outs = []
    for _ in range(2):
        y = K().kron_linear_fwd(x, S, A, B, None)
        g = K().kron_linear_bwd(x, S, A, B, dy)
        outs.append([bits(y)] + [bits(g[k]) for k in ("dx", "dS", "dA", "dB", "dbias")])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
