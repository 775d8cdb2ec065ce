"""GPU parity of the fused Adam + l1 update, the dense head + cross-entropy, and the
tutorial's full MLP training step, against the fp64 oracle.

The step is checked call by call: every kernel is compared with the oracle evaluated on
the very fp32 tensors the GPU step fed it (so a ReLU mask decided differently upstream
cannot make a downstream comparison fail).  End-to-end chained differences are printed
with the count of ReLU-mask disagreements, as a report."""
import numpy as np
import pytest

from _harness import TOL_F32, dev, host, rel_err
from oracle import kron as OK
from oracle import mlp as OM
from oracle import optim as OO
from workloads import mlp_step_inputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def K():
    import kronecker_factored_structured_amd as mod
    return mod


@pytest.mark.parametrize("numels", [[10, 1, 4097, 300000], [0, 5, 0]])
def test_adam_l1_multi_tensor(numels):
    print(f"[adam] numels={numels}", flush=True)
    rng = np.random.default_rng(7)
    ths = [rng.standard_normal(n).astype(np.float32) for n in numels]
    for t in ths:
        t[: min(3, t.size)] = 0.0                     # sign(0) = 0
    l1 = [1e-2 if i % 2 == 0 else 0.0 for i in range(len(numels))]
    P = [dev(t) for t in ths]
    M = [torch.zeros_like(p) for p in P]
    V = [torch.zeros_like(p) for p in P]
    ref = [(t.astype(np.float64), np.zeros(t.size), np.zeros(t.size)) for t in ths]
    for step in range(1, 4):
        gs = [rng.standard_normal(n).astype(np.float32) for n in numels]
        K().kron_adam_l1_step(P, [dev(g) for g in gs], M, V, step, 1e-3, l1=l1)
        ref = [OO.adam_l1_step(th, g, m, v, step, 1e-3, lam=lam) for (th, m, v), g, lam in zip(ref, gs, l1)]
        # continue the oracle from the GPU's fp32 state so each step is compared on its own inputs
        torch.cuda.synchronize()
        for i, n in enumerate(numels):
            if n == 0:
                continue
            assert rel_err(host(P[i]), ref[i][0]) <= TOL_F32
            assert rel_err(host(M[i]), ref[i][1]) <= TOL_F32
            assert rel_err(host(V[i]), ref[i][2]) <= TOL_F32
        ref = [(host(P[i]), host(M[i]), host(V[i])) for i in range(len(numels))]


# K = 1024 with C <= 16 takes the matrix-core head; the other shapes the generic kernels.
@pytest.mark.parametrize("N,Kf,C,want_dh,relu", [(20000, 1024, 10, True, True), (1031, 1024, 16, True, True),
                                                 (37, 1024, 1, True, False), (515, 1024, 10, False, False),
                                                 (77, 130, 3, True, True), (1, 64, 10, True, True),
                                                 (513, 200, 40, True, True)])
def test_head_ce(N, Kf, C, want_dh, relu):
    print(f"[head] N={N} K={Kf} C={C} dh={want_dh} relu={relu}", flush=True)
    rng = np.random.default_rng(8)
    h = rng.standard_normal((N, Kf))
    if relu:
        h = np.maximum(h, 0)
    h = h.astype(np.float32)
    W = (rng.standard_normal((Kf, C)) / np.sqrt(Kf)).astype(np.float32)
    b = rng.standard_normal(C).astype(np.float32)
    lab = rng.integers(0, C, N)
    out = K().kron_head_ce(dev(h), dev(W), dev(b), dev(lab), want_dh=want_dh, relu_mask=relu)
    z = h.astype(np.float64) @ W + b
    loss, dz = OM.softmax_ce(z, lab)
    assert abs(host(out["loss"])[0] - loss) <= TOL_F32 * abs(loss)
    assert rel_err(host(out["dW"]), h.T.astype(np.float64) @ dz) <= TOL_F32
    assert rel_err(host(out["db"]), dz.sum(0)) <= TOL_F32
    if want_dh:
        want = dz @ W.T.astype(np.float64)
        if relu:
            want = want * (h > 0)
        assert rel_err(host(out["dh"]), want) <= TOL_F32
    else:
        assert out["dh"] is None


@pytest.mark.parametrize("Kf", [64, 1024])
def test_head_ce_bad_label_gives_nan_loss(Kf):
    h = dev(np.ones((4, Kf), np.float32))
    W = dev(np.ones((Kf, 10), np.float32) * 0.01)
    b = dev(np.zeros(10, np.float32))
    lab = dev(np.array([1, 2, 10, -1], np.int64))
    out = K().kron_head_ce(h, W, b, lab)
    assert np.isnan(host(out["loss"])[0])


def _layers_host(step):
    S1, A1, B1, b1, S2, A2, B2, b2, hw, hb = [p.detach().cpu().numpy() for p in step.params]
    return [dict(S=S1, A=A1, B=B1, bias=b1), dict(S=S2, A=A2, B=B2, bias=b2)], hw, hb


@pytest.mark.parametrize("N", [20000, 999])
def test_mlp_training_step(N):
    """MLP 1024 -> 1024 -> 1024 -> 10, Kronecker hidden layers (m = 64, r = 2), batch N."""
    print(f"[step] N={N}", flush=True)
    inp = mlp_step_inputs(N=N)
    step = K().KronMLPStep(inp.layers, inp.head_w, inp.head_b, inp.lam, inp.lr, "cuda")
    layers, hw, hb = _layers_host(step)
    x, lab = dev(inp.x), dev(inp.labels)
    loss, grads, acts = step.grads(x, lab)
    torch.cuda.synchronize()
    h1, h2, dh2, dh1 = (host(acts[k]) for k in ("h1", "h2", "dh2", "dh1"))
    # call by call, each on the GPU's own inputs
    assert rel_err(h1, OK.forward(inp.x, layers[0]["S"], layers[0]["A"], layers[0]["B"], layers[0]["bias"], relu=True)) <= TOL_F32
    assert rel_err(h2, OK.forward(h1, layers[1]["S"], layers[1]["A"], layers[1]["B"], layers[1]["bias"], relu=True)) <= TOL_F32
    z = h2 @ hw.astype(np.float64) + hb
    ce, dz = OM.softmax_ce(z, inp.labels)
    # the step's loss: mean cross-entropy + lam * (sum|S1| + sum|S2|)
    full = ce + OM.l1_penalty([layers[0]["S"], layers[1]["S"]], inp.lam)
    assert abs(host(loss)[0] - full) <= TOL_F32 * full
    assert rel_err(dh2, (dz @ hw.T.astype(np.float64)) * (h2 > 0)) <= TOL_F32
    assert rel_err(host(grads[8]), h2.T @ dz) <= TOL_F32
    assert rel_err(host(grads[9]), dz.sum(0)) <= TOL_F32
    g2 = OK.backward(h1, layers[1]["S"], layers[1]["A"], layers[1]["B"], dh2)
    assert rel_err(dh1, g2["dx"] * (h1 > 0)) <= TOL_F32
    for i, k in enumerate(("dS", "dA", "dB", "dbias")):
        assert rel_err(host(grads[4 + i]), g2[k]) <= TOL_F32, ("layer2", k)
    g1 = OK.backward(inp.x, layers[0]["S"], layers[0]["A"], layers[0]["B"], dh1, want_dx=False)
    for i, k in enumerate(("dS", "dA", "dB", "dbias")):
        assert rel_err(host(grads[i]), g1[k]) <= TOL_F32, ("layer1", k)
    # the Adam update, on the GPU's gradients
    params0 = [host(p) for p in step.params]
    ghost = [host(g) for g in grads]
    step.step_count += 1
    K().kron_adam_l1_step(step.params, grads, step.m, step.v, 1, inp.lr, l1=step.l1)
    torch.cuda.synchronize()
    for i, (p0, g) in enumerate(zip(params0, ghost)):
        t1, _, _ = OO.adam_l1_step(p0, g, np.zeros_like(p0), np.zeros_like(p0), 1, inp.lr, lam=step.l1[i])
        assert rel_err(host(step.params[i]), t1) <= TOL_F32, i
    # the chained end-to-end step against the oracle's own chain: the loss within the bar,
    # the gradients reported (a ReLU mask flipped at a rounding tie moves them locally)
    oloss, _, _, ogl, oacts = OM.full_step(inp.x, inp.labels, inp.layers, inp.head_w, inp.head_b, inp.lam, inp.lr)
    assert abs(host(loss)[0] - oloss) <= TOL_F32 * oloss
    flips1 = int(np.sum((h1 > 0) != (oacts["h1"] > 0)))
    flips2 = int(np.sum((h2 > 0) != (oacts["h2"] > 0)))
    chained = [rel_err(g, o) for g, o in zip(ghost, ogl)]
    print(f"   chained: loss {host(loss)[0]:.7f} vs {oloss:.7f}; relu mask flips {flips1}+{flips2}; "
          f"max grad rel err {max(chained):.2e}", flush=True)


def test_mlp_three_steps_loss_trajectory():
    """Three consecutive training steps (fwd, CE + lam*sum|S|, bwd, fused Adam with its
    state carried over) on 999 rows, against the oracle stepping its own parameters and
    Adam state: the loss of every step within the fp32 bar.  (Parameters are not compared
    entry by entry: Adam moves an entry by lr * sign(g) at the first step, so an entry whose
    gradient is a rounding error away from zero may move either way.)"""
    print("[step] three steps, N=999", flush=True)
    inp = mlp_step_inputs(N=999)
    step = K().KronMLPStep(inp.layers, inp.head_w, inp.head_b, inp.lam, inp.lr, "cuda")
    x, lab = dev(inp.x), dev(inp.labels)
    layers = [dict(L) for L in inp.layers]
    hw, hb, state = inp.head_w, inp.head_b, None
    for t in range(1, 4):
        loss = host(step.step(x, lab))[0]
        oloss, newp, state, _, _ = OM.full_step(inp.x, inp.labels, layers, hw, hb, inp.lam, inp.lr, step=t,
                                                state=state)
        print(f"   step {t}: loss {loss:.7f} vs oracle {oloss:.7f}", flush=True)
        assert abs(loss - oloss) <= TOL_F32 * oloss, t
        layers = [dict(S=newp[0], A=newp[1], B=newp[2], bias=newp[3]),
                  dict(S=newp[4], A=newp[5], B=newp[6], bias=newp[7])]
        hw, hb = newp[8], newp[9]
