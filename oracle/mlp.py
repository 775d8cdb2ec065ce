"""fp64 oracle of the tutorial's full training step (test infrastructure only).

Source: "A Kronecker layer benchmark" tutorial, "Setup": a 3-layer MLP
1024 -> 1024 -> 1024 -> 10 with ReLU, the two hidden layers Kronecker layers, the
10-class output layer dense; one step is forward, cross-entropy plus the model's
penalty, backward, and an Adam update.

Readings adopted where the page is silent: the cross-entropy is the mean over rows;
the penalty is lam * (sum|S_1| + sum|S_2|); relu'(0) = 0; the head is stored in x out
(z = h W_h + b_h, the row-vector convention of the layer); Adam as in optim.py.

Forward:   h1 = relu(x W1 + b1),  h2 = relu(h1 W2 + b2),  z = h2 W_h + b_h
Loss:      mean_n [ logsumexp(z_n) - z_n[label_n] ] + lam * sum|S|
Backward:  dz = (softmax(z) - onehot(label)) / N
           dW_h = h2^T dz,  db_h = sum_n dz,  dh2 = (dz W_h^T) o [h2 > 0]
           layer 2 backward with dY = dh2 (kron.backward)
           dh1 = dX_2 o [h1 > 0];  layer 1 backward without dX
           dS_l += lam * sign(S_l)   (applied inside the Adam step)
"""
from __future__ import annotations

import numpy as np

from . import kron, optim
from .kron import as64


def softmax_ce(z, labels):
    """Mean cross-entropy over rows and its gradient with respect to the logits."""
    z = as64(z)
    N = z.shape[0]
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax)
    s = e.sum(axis=1, keepdims=True)
    logp = z - zmax - np.log(s)
    loss = -np.mean(logp[np.arange(N), labels])
    dz = e / s
    dz[np.arange(N), labels] -= 1.0
    dz /= N
    return loss, dz


def l1_penalty(tensors, lam):
    """lam * sum over the tensors of sum|t| (the model's penalty; intro: S is l1-penalised)."""
    return lam * sum(np.abs(as64(t)).sum() for t in tensors)


def forward(x, layers, head_w, head_b):
    """Returns the activations (h1, h2) and the logits z."""
    h1 = kron.forward(x, layers[0]["S"], layers[0]["A"], layers[0]["B"], layers[0]["bias"], relu=True)
    h2 = kron.forward(h1, layers[1]["S"], layers[1]["A"], layers[1]["B"], layers[1]["bias"], relu=True)
    z = h2 @ as64(head_w) + as64(head_b)[None, :]
    return h1, h2, z


def step_grads(x, labels, layers, head_w, head_b, lam):
    """Loss (with the penalty) and every parameter gradient before the l1 subgradient.

    Returns (loss, grads, acts) with grads = [layer1 dict, layer2 dict, head dict]."""
    h1, h2, z = forward(x, layers, head_w, head_b)
    ce, dz = softmax_ce(z, labels)
    penalty = l1_penalty([L["S"] for L in layers], lam)
    head = dict(dW=h2.T @ dz, db=dz.sum(axis=0))
    dh2 = (dz @ as64(head_w).T) * (h2 > 0)
    g2 = kron.backward(h1, layers[1]["S"], layers[1]["A"], layers[1]["B"], dh2, want_dx=True)
    dh1 = g2["dx"] * (h1 > 0)
    g1 = kron.backward(x, layers[0]["S"], layers[0]["A"], layers[0]["B"], dh1, want_dx=False)
    return ce + penalty, [g1, g2, head], dict(h1=h1, h2=h2, z=z, dh2=dh2, dh1=dh1, ce=ce)


def full_step(x, labels, layers, head_w, head_b, lam, lr, step=1, state=None,
              beta1=0.9, beta2=0.999, eps=1e-8):
    """One training step; returns (loss, new parameters, new Adam state, grads).

    Parameters are listed as (name, array, l1) in the order
    S1, A1, B1, bias1, S2, A2, B2, bias2, head_w, head_b."""
    loss, grads, acts = step_grads(x, labels, layers, head_w, head_b, lam)
    params = []
    gl = []
    for L, g in zip(layers, grads[:2]):
        params += [("S", L["S"], lam), ("A", L["A"], 0.0), ("B", L["B"], 0.0), ("bias", L["bias"], 0.0)]
        gl += [g["dS"], g["dA"], g["dB"], g["dbias"]]
    params += [("head_w", head_w, 0.0), ("head_b", head_b, 0.0)]
    gl += [grads[2]["dW"], grads[2]["db"]]
    if state is None:
        state = [(np.zeros(np.shape(p)), np.zeros(np.shape(p))) for _, p, _ in params]
    new_params, new_state = [], []
    for (name, p, l1), g, (m, v) in zip(params, gl, state):
        t, m2, v2 = optim.adam_l1_step(p, g, m, v, step, lr, beta1, beta2, eps, lam=l1)
        new_params.append(t)
        new_state.append((m2, v2))
    return loss, new_params, new_state, gl, acts
