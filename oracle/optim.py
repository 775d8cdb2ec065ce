"""fp64 oracle of the fused Adam + l1-on-S update (test infrastructure only).

Source: "A Kronecker layer benchmark" tutorial, "Setup": a training step is the
forward pass, cross-entropy loss plus the model's penalty (an l1 penalty on S, see
the intro), the backward pass and an Adam update.  The page prints no
hyper-parameters; readings adopted: beta1 = 0.9, beta2 = 0.999, eps = 1e-8,
bias-corrected moments, no weight decay, first step t = 1.  The penalty lam*sum|S|
enters the gradient of S as lam*sign(S), with sign(0) = 0.

Adam (Kingma & Ba, 2015), per element:
    g <- g + lam*sign(theta)              (only for tensors carrying the penalty)
    m <- beta1*m + (1 - beta1)*g
    v <- beta2*v + (1 - beta2)*g^2
    theta <- theta - lr * (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
"""
from __future__ import annotations

import numpy as np

from .kron import as64


def adam_l1_step(theta, g, m, v, step: int, lr: float, beta1: float = 0.9,
                 beta2: float = 0.999, eps: float = 1e-8, lam: float = 0.0):
    """One update of one tensor; returns (theta, m, v) as new fp64 arrays."""
    if step < 1:
        raise ValueError("step must be >= 1")
    theta = as64(theta)
    g = as64(g)
    m = as64(m)
    v = as64(v)
    if lam != 0.0:
        g = g + lam * np.sign(theta)
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    mhat = m / (1.0 - beta1 ** step)
    vhat = v / (1.0 - beta2 ** step)
    theta = theta - lr * mhat / (np.sqrt(vhat) + eps)
    return theta, m, v
