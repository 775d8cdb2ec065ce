"""Plain, slow, fp64 CPU oracle for the Kronecker-factored layer and the Kronecker-sparse matmul.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import or run anything in this package.  The product path (the
HIP library and its Python binding) never imports it, and this package imports
nothing from the product path.

What it computes, and the passage each function follows:
  * kron.py   -- the layer y = x W + bias with W = sum_i kron(S o A_i, B_i), built
                 explicitly block by block ("A Kronecker layer benchmark" tutorial,
                 "Build W, then multiply"), the dense product, and hand-derived
                 gradients taken through W.
  * ks.py     -- Kronecker-sparse matrices whose support is I_a (x) 1_{b x c} (x) I_d
                 ("Fast Inference with Kronecker-Sparse Matrices", abstract), built
                 densely and multiplied naively.
  * optim.py  -- the Adam update of the training step, with the l1 penalty on S
                 entering through its subgradient (tutorial, "Setup", training step).
  * mlp.py    -- the tutorial's full training step: MLP with two Kronecker hidden
                 layers, ReLU, a dense 10-way head, cross-entropy plus the penalty,
                 backward and Adam (tutorial, "Setup").

Everything is computed in float64 from the exact fp32 (or bf16) input values.
Pins: every function is checked against facts fixed outside this package (closed
forms, textbook identities, library routines, finite differences, printed
quantities); see tests/test_oracle_*.py.  No function here is "parity unpinned".
"""

from . import kron, ks, optim, mlp  # noqa: F401
