"""torch modules over libkron: the Kronecker-factored layer, the Kronecker-sparse layer
and the tutorial's MLP training step.  Marshalling only; every step runs in libkron.
"""
from __future__ import annotations

import math
from typing import Optional

import torch
from torch import nn

from . import api


class _KronLinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, S, A, B, bias, relu: bool, sparse_rows: bool, save_z: bool = False):
        x = x.contiguous()
        # Z_i = X B_i saved for the backward where the shape has that path (else recomputed)
        zc = api.new_zcache(x, S, A, B) if save_z and not sparse_rows else None
        y = api.kron_linear_fwd(x, S, A, B, bias, relu=relu, sparse_rows=sparse_rows, zcache=zc)
        ctx.zc = zc
        ctx.relu = relu
        ctx.sparse_rows = sparse_rows
        ctx.save_for_backward(x, S, A, B, y if relu else None)
        ctx.has_S = S is not None
        ctx.has_bias = bias is not None
        return y

    @staticmethod
    def backward(ctx, dy):
        x, S, A, B, y = ctx.saved_tensors
        dy = dy.contiguous()
        if ctx.relu:
            dy = api.kron_relu_bwd(y, dy)
        g = api.kron_linear_bwd(x, S, A, B, dy, want_dx=ctx.needs_input_grad[0],
                                want_dbias=ctx.has_bias, sparse_rows=ctx.sparse_rows, zcache=ctx.zc)
        ctx.zc = None
        return g["dx"], g["dS"], g["dA"], g["dB"], g["dbias"], None, None, None


class KronLinear(nn.Module):
    """y = x W + bias, W = sum_i kron(S o A_i, B_i) (Kronecker layer tutorial,
    "Build W, then multiply": S p x q initialised to ones, A_i ~ randn/sqrt(p),
    B_i ~ randn/sqrt(m), bias zeros; p = in/m, q = out/n).  sparse_rows: S is expected
    to have whole rows zero (e.g. after l1 pruning) and the forward skips them.  save_z: the
    forward keeps Z_i = X B_i of the first ranks (kron_linear_zcache_bytes per batch) for the
    backward instead of the backward recomputing it, where the shape has that path."""

    def __init__(self, in_features: int, out_features: int, m: int, r: int, n: Optional[int] = None,
                 with_S: bool = True, relu: bool = False, device=None, sparse_rows: bool = False,
                 save_z: bool = False):
        super().__init__()
        n = m if n is None else n
        if in_features % m or out_features % n:
            raise ValueError("in_features must be a multiple of m and out_features of n")
        p, q = in_features // m, out_features // n
        dev = device
        self.S = nn.Parameter(torch.ones(p, q, device=dev)) if with_S else None
        self.A = nn.Parameter(torch.randn(r, p, q, device=dev) / math.sqrt(p))
        self.B = nn.Parameter(torch.randn(r, m, n, device=dev) / math.sqrt(m))
        self.bias = nn.Parameter(torch.zeros(out_features, device=dev))
        self.relu = relu
        self.sparse_rows = sparse_rows
        self.save_z = save_z

    def forward(self, x):
        return _KronLinearFn.apply(x, self.S, self.A, self.B, self.bias, self.relu, self.sparse_rows, self.save_z)

    def l1_penalty(self):
        """sum|S| as a 0-dim tensor with autograd (sign(S) times the upstream gradient)."""
        return _L1Fn.apply(self.S) if self.S is not None else 0.0


class _L1Fn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, S):
        ctx.save_for_backward(S)
        return api.kron_l1_penalty([S.contiguous()], 1.0).view(())

    @staticmethod
    def backward(ctx, g):
        (S,) = ctx.saved_tensors
        return api.kron_l1_penalty_grad(S.contiguous(), 1.0, g.reshape(1).contiguous())


class KSLinear(nn.Module):
    """Y = X K with K Kronecker-sparse of support I_a (x) 1_{b x c} (x) I_d ("Fast Inference
    with Kronecker-Sparse Matrices"); values a x d x b x c ~ N(0, 1/b).  Forward only."""

    def __init__(self, a: int, b: int, c: int, d: int, dtype=torch.float32, device=None):
        super().__init__()
        self.abcd = (a, b, c, d)
        self.vals = nn.Parameter((torch.randn(a, d, b, c, device=device) / math.sqrt(b)).to(dtype),
                                 requires_grad=False)

    def forward(self, x):
        a, b, c, d = self.abcd
        return api.ks_matmul(x.contiguous(), self.vals, a, b, c, d)


class KronMLPStep:
    """The tutorial's training step (Kronecker layer tutorial, "Setup"): MLP
    in -> hidden -> hidden -> classes with ReLU, both hidden layers Kronecker, a dense
    head, mean cross-entropy + lam * sum|S|, backward, and one fused Adam update.

    Parameters live in flat lists of device tensors in the order
    S1, A1, B1, bias1, S2, A2, B2, bias2, head_w (hidden x classes), head_b.
    One step is 10 kernel launches plus the column reductions, independent of r.
    """

    def __init__(self, layers, head_w, head_b, lam: float, lr: float, device,
                 beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8):
        def t(a):
            return torch.as_tensor(a, dtype=torch.float32, device=device).contiguous()
        self.params = []
        for L in layers:
            self.params += [t(L["S"]), t(L["A"]), t(L["B"]), t(L["bias"])]
        self.params += [t(head_w), t(head_b)]
        self.m = [torch.zeros_like(p) for p in self.params]
        self.v = [torch.zeros_like(p) for p in self.params]
        self.l1 = [lam, 0.0, 0.0, 0.0, lam, 0.0, 0.0, 0.0, 0.0, 0.0]
        self.lam, self.lr = lam, lr
        self.beta1, self.beta2, self.eps = beta1, beta2, eps
        self.step_count = 0
        self.device = device
        self._ws = {}

    def _workspace(self, key, nbytes):
        w = self._ws.get(key)
        if w is None or w.numel() < nbytes:
            w = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=self.device)
            self._ws[key] = w
        return w

    def grads(self, x: torch.Tensor, labels: torch.Tensor):
        """Forward + backward; returns (loss tensor, gradient list, activations).  The loss is
        the mean cross-entropy plus lam * (sum|S1| + sum|S2|); the l1 subgradient of the
        penalty is applied inside the Adam step."""
        S1, A1, B1, b1, S2, A2, B2, b2, hw, hb = self.params
        h1 = api.kron_linear_fwd(x, S1, A1, B1, b1, relu=True)
        h2 = api.kron_linear_fwd(h1, S2, A2, B2, b2, relu=True)
        head = api.kron_head_ce(h2, hw, hb, labels, want_dh=True, relu_mask=True)
        api.kron_l1_penalty([S1, S2], self.lam, loss=head["loss"], accumulate=True)
        shape2 = api.layer_shape(h1.shape[0], S2, A2, B2)
        g2 = api.kron_linear_bwd(h1, S2, A2, B2, head["dh"], want_dx=True, relu_mask=True,
                                 workspace=self._workspace("l2", api.kron_linear_bwd_workspace_bytes(shape2)))
        shape1 = api.layer_shape(x.shape[0], S1, A1, B1)
        g1 = api.kron_linear_bwd(x, S1, A1, B1, g2["dx"], want_dx=False,
                                 workspace=self._workspace("l1", api.kron_linear_bwd_workspace_bytes(shape1)))
        grads = [g1["dS"], g1["dA"], g1["dB"], g1["dbias"], g2["dS"], g2["dA"], g2["dB"], g2["dbias"],
                 head["dW"], head["db"]]
        return head["loss"], grads, dict(h1=h1, h2=h2, dh2=head["dh"], dh1=g2["dx"])

    def step(self, x: torch.Tensor, labels: torch.Tensor):
        """One full training step; returns the loss (cross-entropy + l1 penalty, device tensor)."""
        loss, grads, _ = self.grads(x, labels)
        self.step_count += 1
        api.kron_adam_l1_step(self.params, grads, self.m, self.v, self.step_count, self.lr,
                              self.beta1, self.beta2, self.eps, l1=self.l1)
        return loss
