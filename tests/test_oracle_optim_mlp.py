"""Pins of the Adam + l1 oracle and of the full training-step oracle (CPU only).

Library routines used as independent references: torch.optim.Adam and torch autograd
in float64 (cross-entropy, ReLU, torch.kron).
"""
import numpy as np
import pytest

from oracle import mlp as OM
from oracle import optim as OO
from workloads import mlp_step_inputs

torch = pytest.importorskip("torch")


def test_adam_first_step_closed_form():
    """At t = 1 the bias-corrected moments are g and g^2, so each parameter moves by
    lr * g / (|g| + eps)."""
    rng = np.random.default_rng(0)
    th = rng.standard_normal(50)
    g = rng.standard_normal(50)
    t1, m1, v1 = OO.adam_l1_step(th, g, np.zeros(50), np.zeros(50), 1, 1e-3)
    np.testing.assert_allclose(t1, th - 1e-3 * g / (np.abs(g) + 1e-8), rtol=0, atol=1e-15)
    np.testing.assert_allclose(m1, 0.1 * g, rtol=1e-15)
    np.testing.assert_allclose(v1, 0.001 * g * g, rtol=1e-12)


@pytest.mark.parametrize("lam", [0.0, 1e-2])
def test_adam_l1_matches_torch(lam):
    """Several steps against torch.optim.Adam (float64) on the loss <g_t, theta> + lam*sum|theta|,
    whose gradient is g_t + lam*sign(theta) (torch's abs has subgradient 0 at 0)."""
    rng = np.random.default_rng(1)
    th0 = rng.standard_normal(40)
    th0[:5] = 0.0                                   # sign(0) = 0 entries
    p = torch.tensor(th0.copy(), requires_grad=True)
    opt = torch.optim.Adam([p], lr=1e-2, betas=(0.9, 0.999), eps=1e-8)
    th, m, v = th0.copy(), np.zeros(40), np.zeros(40)
    for step in range(1, 6):
        g = rng.standard_normal(40)
        opt.zero_grad()
        loss = (torch.tensor(g) * p).sum() + lam * p.abs().sum()
        loss.backward()
        opt.step()
        th, m, v = OO.adam_l1_step(th, g, m, v, step, 1e-2, lam=lam)
    np.testing.assert_allclose(th, p.detach().numpy(), rtol=1e-12, atol=1e-14)


def test_adam_rejects_step_zero():
    with pytest.raises(ValueError):
        OO.adam_l1_step(np.zeros(1), np.zeros(1), np.zeros(1), np.zeros(1), 0, 1e-3)


def test_softmax_ce_matches_torch():
    rng = np.random.default_rng(2)
    z = rng.standard_normal((30, 10)) * 3
    lab = rng.integers(0, 10, 30)
    loss, dz = OM.softmax_ce(z, lab)
    tz = torch.tensor(z, requires_grad=True)
    tl = torch.nn.functional.cross_entropy(tz, torch.tensor(lab))
    tl.backward()
    assert abs(loss - tl.item()) <= 1e-14 * abs(tl.item())
    np.testing.assert_allclose(dz, tz.grad.numpy(), rtol=1e-12, atol=1e-15)


def _torch_step(inp, N):
    """The tutorial's step written with torch autograd (float64), as an independent reference."""
    x = torch.tensor(inp.x[:N].astype(np.float64))
    lab = torch.tensor(inp.labels[:N])
    params = []
    for L in inp.layers:
        params.append({k: torch.tensor(L[k].astype(np.float64), requires_grad=True)
                       for k in ("S", "A", "B", "bias")})
    hw = torch.tensor(inp.head_w.astype(np.float64), requires_grad=True)
    hb = torch.tensor(inp.head_b.astype(np.float64), requires_grad=True)
    h = x
    for P in params:
        W = sum(torch.kron(P["S"] * P["A"][i], P["B"][i]) for i in range(P["A"].shape[0]))
        h = torch.relu(h @ W + P["bias"])
    z = h @ hw + hb
    loss = torch.nn.functional.cross_entropy(z, lab) + inp.lam * sum(P["S"].abs().sum() for P in params)
    loss.backward()
    return loss.item(), params, hw, hb


def test_mlp_step_gradients_match_torch_autograd():
    """Full step at reduced size (hidden 64, m = 8, r = 2, 96 rows): every gradient of the
    oracle's hand-written backward against torch autograd."""
    inp = mlp_step_inputs(seed=3, N=96, hidden=64, m=8, r=2, lam=1e-2)
    # make S non-trivial so the penalty and dS are exercised with mixed signs and zeros
    rng = np.random.default_rng(5)
    for L in inp.layers:
        L["S"] = rng.integers(-2, 3, L["S"].shape).astype(np.float32)
    loss, grads, _ = OM.step_grads(inp.x, inp.labels, inp.layers, inp.head_w, inp.head_b, inp.lam)
    tloss, tp, thw, thb = _torch_step(inp, 96)
    assert abs(loss - tloss) <= 1e-12 * abs(tloss)
    for g, P, L in zip(grads[:2], tp, inp.layers):
        # the oracle keeps the l1 subgradient for the optimizer; add it here to compare
        np.testing.assert_allclose(g["dS"] + inp.lam * np.sign(L["S"].astype(np.float64)), P["S"].grad.numpy(), rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(g["dA"], P["A"].grad.numpy(), rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(g["dB"], P["B"].grad.numpy(), rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(g["dbias"], P["bias"].grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(grads[2]["dW"], thw.grad.numpy(), rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(grads[2]["db"], thb.grad.numpy(), rtol=1e-10, atol=1e-13)


def test_mlp_full_step_matches_torch_adam():
    """Parameters after one full step against torch autograd + torch.optim.Adam (float64)."""
    inp = mlp_step_inputs(seed=4, N=64, hidden=32, m=8, r=2, lam=1e-3, lr=1e-3)
    _, new_params, _, _, _ = OM.full_step(inp.x, inp.labels, inp.layers, inp.head_w, inp.head_b,
                                          inp.lam, inp.lr)
    _, tp, thw, thb = _torch_step(inp, 64)
    flat = []
    for P in tp:
        flat += [P["S"], P["A"], P["B"], P["bias"]]
    flat += [thw, thb]
    opt = torch.optim.Adam(flat, lr=inp.lr, betas=(0.9, 0.999), eps=1e-8)
    opt.step()
    for a, t in zip(new_params, flat):
        np.testing.assert_allclose(a, t.detach().numpy(), rtol=1e-9, atol=1e-12)
