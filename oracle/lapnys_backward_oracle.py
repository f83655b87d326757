"""Plain float64 CPU oracle for the gradients of the Laplacian-kernel Nystrom attention forward.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or run anything in this
directory.  The product path never touches it, and this module imports nothing
from the product package.

The pages state that their kernels serve the forward and the backward pass
(EN page, section 3; DE section 3; ZH section 3; KO section 3; JA section 3)
and that the L1 kernel keeps its gradient away from zero near coincident
points (EN section 2.A).  They give no backward formulas: the backward is the
derivative of the forward they define.  This module restates the forward of
``lapnys_oracle`` with PyTorch CPU float64 operations, step for step in the
same order, and takes its derivative with autograd (a library primitive used as
a step).  Two readings of the inverse are offered:

* ``through="unrolled"``: the T Newton-Schulz steps as computed, including the
  scaling alpha = ||W||_1 ||W||_inf (its max entries are differentiated at
  the attained maximum);
* ``through="implicit"``: X taken as the exact inverse W^-1, so dW = -X^T dX X^T;
  the two agree once the iteration has converged.

Pins (``tests/test_backward_oracle.py``): the restated forward equals the numpy
oracle's; central finite differences of a scalar projection of O; the closed
form of the V gradient (O is linear in V); agreement of the two readings at
convergence; and planted mistakes in the restated forward.
"""

from __future__ import annotations

import numpy as np
import torch


def _t(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float64))


def laplacian_kernel_t(x, y, lam):
    """exp(-||x_i - y_j||_1 / lam) (EN page, section 2.A), as a torch expression."""
    return torch.exp(-(x[:, None, :] - y[None, :, :]).abs().sum(dim=2) / lam)


def pool_landmarks_t(k, grid_h, grid_w, pool):
    """Average of K over each pool x pool window of the row-major token grid (EN
    section 2.C.1), windows row-major; the window mean sums rows then columns."""
    g = k.reshape(grid_h // pool, pool, grid_w // pool, pool, k.shape[-1])
    return g.mean(dim=(1, 3)).reshape(-1, k.shape[-1])


def newton_schulz_t(w, iters):
    """X0 = W^T / (||W||_1 ||W||_inf), then X <- X (2I - W X), ``iters`` times (EN 2.C.2)."""
    alpha = w.abs().sum(dim=0).max() * w.abs().sum(dim=1).max()
    x = w.T / alpha
    two_i = 2.0 * torch.eye(w.shape[0], dtype=w.dtype)
    for _ in range(iters):
        x = x @ (two_i - w @ x)
    return x


def whiten_t(c):
    """Per landmark column: subtract the mean over the tokens and divide by the
    population standard deviation (EN 2.B); a zero-variance column becomes 0."""
    mu = c.mean(dim=0)
    dev = c - mu
    sigma = torch.sqrt((dev * dev).mean(dim=0))
    safe = torch.where(sigma > 0, sigma, torch.ones_like(sigma))
    return torch.where(sigma > 0, dev / safe, torch.zeros_like(dev))


def forward_t(q, k, v, *, grid_h, grid_w, pool, lam, eps, ns_iters, whiten=True, through="unrolled"):
    """O of one problem as a torch graph: landmarks, C, B, W, the inverse, Z,
    O = Z (X (B V)) (the order of lapnys_oracle.attention_problem)."""
    if through not in ("unrolled", "implicit"):
        raise ValueError(f"unknown reading {through!r}")
    kt = pool_landmarks_t(k, grid_h, grid_w, pool)
    m = kt.shape[0]
    c = laplacian_kernel_t(q, kt, lam)
    b = laplacian_kernel_t(kt, k, lam)
    w = laplacian_kernel_t(kt, kt, lam) + eps * torch.eye(m, dtype=q.dtype)
    x = newton_schulz_t(w, ns_iters) if through == "unrolled" else torch.linalg.inv(w)
    z = whiten_t(c) if whiten else c
    return z @ (x @ (b @ v))


def backward(q, k, v, d_out, *, grid_h, grid_w, pool, lam, eps, ns_iters, whiten=True, through="unrolled"):
    """Gradients (dq, dk, dv) of sum(d_out * O) for one problem, float64 numpy."""
    qt, kt_, vt = (_t(a).requires_grad_(True) for a in (q, k, v))
    o = forward_t(qt, kt_, vt, grid_h=grid_h, grid_w=grid_w, pool=pool, lam=lam, eps=eps, ns_iters=ns_iters,
                  whiten=whiten, through=through)
    dq, dk, dv = torch.autograd.grad(o, (qt, kt_, vt), grad_outputs=_t(d_out))
    return dq.numpy(), dk.numpy(), dv.numpy()


def forward_values(q, k, v, **kw):
    """The restated forward's O as numpy (for the cross-check with lapnys_oracle)."""
    with torch.no_grad():
        return forward_t(_t(q), _t(k), _t(v), **kw).numpy()
