"""Plain float64 CPU oracle for LaplacianFormer's Laplacian-kernel Nystrom attention forward.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or run anything in this
directory.  The product path (the HIP library and its Python binding) never
touches it, and this module imports nothing from the product package.

Sources.  The method is described by five summary pages of the paper
"LaplacianFormer: Rethinking Linear Attention with Laplacian Kernel" on
gist.science, in English (EN), German (DE), Chinese (ZH), Korean (KO) and
Japanese (JA).  Each function below names the page and section it follows.
Where the pages leave a step open, the reading taken is stated in the
function's docstring and collected in the design doc.

Every quantity is computed in float64 with numpy, one (batch, head) problem
at a time, in the order the method states, with no blocking or fusion beyond
what the definition implies.  Library primitives used as steps: elementwise
abs/exp, ``sum``/``mean`` reductions, and matrix products (``@``).

Pins.  Each function is pinned by CPU tests (``tests/test_oracle.py``) to
facts that do not come from this file: hand-worked kernel values, closed forms
(pooled index ramps, the Newton-Schulz error-squaring closed form via an
eigendecomposition, the pool=1 Nystrom identity), an LU inverse, exact
whitening moments, brute-force O(N^2) attention on tiny inputs, and
metamorphic invariants.  No function here is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

# Rows of the left operand per block when forming kernel matrices, so that the
# |x - y| temporary stays near 64 MB however large N is.  Blocking over rows
# does not change any value: each entry is an independent sum over features.
_BLOCK_BYTES = 64 << 20


def laplacian_kernel(x, y, lam):
    """Laplacian kernel matrix: out[i, j] = exp(-sum_t |x[i, t] - y[j, t]| / lam).

    The L1 (Manhattan) distance replaces the squared L2 distance of a Gaussian
    kernel (EN page section 2.A; DE section 2, kernel item; ZH section 2.1;
    KO section 2.1; JA section 2.1).  The distance is divided by lam exactly as
    the pages write it, with no 1/d or 1/sqrt(d) factor.
    """
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    out = np.empty((x.shape[0], y.shape[0]), dtype=np.float64)
    rows = max(1, _BLOCK_BYTES // max(1, 8 * y.shape[0] * y.shape[1]))
    for s in range(0, x.shape[0], rows):
        dist = np.abs(x[s:s + rows, None, :] - y[None, :, :]).sum(axis=2)
        out[s:s + rows] = np.exp(-dist / lam)
    return out


def gaussian_kernel(x, y, lam):
    """Gaussian kernel matrix: out[i, j] = exp(-sum_t (x[i, t] - y[j, t])^2 / lam).

    The kernel the Laplacian one replaces: similarity decaying with the squared
    L2 distance (EN page, section 1, first flaw, and section 2.A, which swaps
    that distance for the L1 one inside the same exponential).  Reading taken:
    the same scale lam divides the squared distance, with no factor 2 and no
    1/d, so that the two kernels differ only in the distance.  The squared
    differences are summed directly, not through |x|^2 + |y|^2 - 2 x.y.
    """
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    out = np.empty((x.shape[0], y.shape[0]), dtype=np.float64)
    rows = max(1, _BLOCK_BYTES // max(1, 8 * y.shape[0] * y.shape[1]))
    for s in range(0, x.shape[0], rows):
        diff = x[s:s + rows, None, :] - y[None, :, :]
        out[s:s + rows] = np.exp(-(diff * diff).sum(axis=2) / lam)
    return out


def pool_landmarks(k, grid_h, grid_w, pool):
    """Landmark keys: the average of K over each non-overlapping pool x pool window.

    The EN page (section 2.C.1) selects the landmark keys by average pooling.
    Reading taken: tokens lie on a row-major grid (token n = r * grid_w + c),
    windows have stride ``pool`` and no padding, and landmarks are numbered
    row-major on the pooled grid, j = R * (grid_w // pool) + C.  Each window sum
    is accumulated in float64 in a fixed order (window row outer, window column
    inner) and then divided by pool * pool.
    """
    k = np.asarray(k, dtype=np.float64)
    n, d = k.shape
    if n != grid_h * grid_w or grid_h % pool or grid_w % pool:
        raise ValueError("grid does not match N or is not divisible by the pool size")
    gh, gw = grid_h // pool, grid_w // pool
    g = k.reshape(grid_h, grid_w, d)
    acc = np.zeros((gh, gw, d), dtype=np.float64)
    for r in range(pool):
        for c in range(pool):
            acc = acc + g[r::pool, c::pool, :]
    return (acc / float(pool * pool)).reshape(gh * gw, d)


def newton_schulz_inverse(w, iters):
    """Inverse of W by a fixed number of Newton-Schulz steps.

    The pages invert the landmark kernel matrix with Newton-Schulz iteration,
    using only matrix products and sums, after a small diagonal shift has made
    it strictly positive definite (EN section 2.C.2; DE section 2; ZH
    section 2.2; KO section 2.3; JA section 2.3).  Start and step:
    X0 = W^T / (||W||_1 * ||W||_inf), then X <- X (2I - W X), exactly ``iters``
    times with no early exit.
    """
    w = np.asarray(w, dtype=np.float64)
    alpha = np.abs(w).sum(axis=0).max() * np.abs(w).sum(axis=1).max()
    x = w.T / alpha
    two_i = 2.0 * np.eye(w.shape[0])
    for _ in range(iters):
        x = x @ (two_i - w @ x)
    return x


def refine_inverse(w, x):
    """One residual-correction step applied to an approximate inverse X of W.

    An extension beyond the pages' fixed-count iteration (EN section 2.C.2
    fixes the step count and uses matrix products only): R = I - W X, then
    X' = X + X R.  Algebraically I - W X' = R - W X R = R - (I - R) R = R^2,
    so one step squares the residual.  The oracle forms it in float64 like
    everything else.
    """
    w = np.asarray(w, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    r = np.eye(w.shape[0]) - w @ x
    return x + x @ r


def conjugate_gradient(w, rhs, iters):
    """Solve W Y = rhs column by column with a fixed number of conjugate-gradient steps.

    The pages compare Newton-Schulz against a conjugate-gradient solver in
    their ablation (EN page, section 4, solver robustness; DE section 4,
    ablations; ZH, KO and JA section 4) without spelling it out.  Reading
    taken: CG computes the product the inverse is needed for, Y = W^-1 (B V),
    directly: one independent CG run per column of the right-hand side, from
    Y0 = 0, no preconditioner, exactly ``iters`` steps (as the Newton-Schulz
    count is fixed).  Step: a = r.r / p.(W p); y += a p; r -= a W p;
    b = r'.r' / r.r; p = r' + b p.  A column whose residual is exactly zero
    stops changing (a = b = 0 instead of 0/0).
    """
    w = np.asarray(w, dtype=np.float64)
    rhs = np.asarray(rhs, dtype=np.float64)
    y = np.zeros_like(rhs)
    r = rhs.copy()
    p = r.copy()
    rr = (r * r).sum(axis=0)
    for _ in range(iters):
        q = w @ p
        pq = (p * q).sum(axis=0)
        live = rr > 0
        a = np.where(live, rr / np.where(live, pq, 1.0), 0.0)
        y = y + a * p
        r = r - a * q
        rr_new = (r * r).sum(axis=0)
        b = np.where(live, rr_new / np.where(live, rr, 1.0), 0.0)
        p = r + b * p
        rr = rr_new
    return y


def whiten_columns(c):
    """Diagonal whitening of the query-side similarity vectors.

    The injective feature map centres each kernel feature and scales it by a
    diagonal estimate of the inverse square root of its covariance, i.e. by the
    feature's empirical standard deviation (EN section 2.B; KO section 2.2;
    JA section 2.2; DE section 2).  Readings taken: the statistics of landmark
    column j are taken over the N tokens of one (batch, head) problem, the
    variance is the population variance (divide by N) computed in two passes,
    the learned bias is zero, and a column with zero spread maps to zeros.
    Returns (Z, mu, sigma).
    """
    c = np.asarray(c, dtype=np.float64)
    mu = c.mean(axis=0)
    dev = c - mu
    sigma = np.sqrt((dev * dev).mean(axis=0))
    z = np.zeros_like(c)
    nz = sigma > 0
    z[:, nz] = dev[:, nz] / sigma[nz]
    return z, mu, sigma


def attention_problem(q, k, v, *, grid_h, grid_w, pool, lam, eps, ns_iters, whiten=True, refine=False,
                      kernel="laplacian", solver="ns"):
    """Forward of one (batch, head) problem; returns every intermediate.

    Steps, in the method's order:
      landmarks  K~ = avgpool(K)                       (EN 2.C.1)
      C = k(Q, K~)  [N x m],  B = k(K~, K)  [m x N]      (EN 2.A, 2.C.1)
      W = k(K~, K~) + eps I  [m x m]                     (EN 2.C.2)
      X = Newton-Schulz inverse of W                    (EN 2.C.2)
          (refine: one residual correction afterwards, refine_inverse)
      Z = whitened C (or C itself when whitening is off) (EN 2.B)
      O = Z (X (B V)), evaluated right to left so the cost is linear in N.
    Reading taken for the Nystrom form: the ZH page (section 2.2) writes the
    low-rank factorisation C W^+ C^T; for attention between queries and keys the
    key-side factor is B = k(K~, K), and W^+ = W^-1 because W + eps I is
    positive definite.  No row normalisation of the output is applied: the pages
    mention none.  ``kernel="gaussian"`` runs the same steps with gaussian_kernel
    in place of laplacian_kernel for C, B and W (the pages' baseline kernel).
    ``solver="cg"`` replaces X (B V) by conjugate_gradient(W, B V, ns_iters)
    (the pages' solver ablation); X is then not formed and is returned as None.
    """
    if solver not in ("ns", "cg"):
        raise ValueError(f"unknown solver {solver!r}")
    if kernel not in ("laplacian", "gaussian"):
        raise ValueError(f"unknown kernel {kernel!r}")
    kfun = gaussian_kernel if kernel == "gaussian" else laplacian_kernel
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    kt = pool_landmarks(k, grid_h, grid_w, pool)
    m = kt.shape[0]
    c = kfun(q, kt, lam)
    b = kfun(kt, k, lam)
    w = kfun(kt, kt, lam) + eps * np.eye(m)
    if whiten:
        z, mu, sigma = whiten_columns(c)
    else:
        z, mu, sigma = c, np.zeros(m), np.ones(m)
    bv = b @ v
    if solver == "cg":
        x = None
        y = conjugate_gradient(w, bv, ns_iters)
    else:
        x = newton_schulz_inverse(w, ns_iters)
        if refine:
            x = refine_inverse(w, x)
        y = x @ bv
    o = z @ y
    return {"landmarks": kt, "C": c, "B": b, "W": w, "X": x, "Z": z,
            "mu": mu, "sigma": sigma, "BV": bv, "Y": y, "O": o}


def forward(q, k, v, *, grid_h, grid_w, pool, lam, eps, ns_iters, whiten=True, problems=None, refine=False,
            kernel="laplacian", solver="ns"):
    """Forward over [B, H, N, d] inputs; every (b, h) problem is independent.

    ``problems`` optionally lists the (b, h) pairs to compute (a sample of a large
    workload); the result then holds one entry per listed pair, stacked on a
    leading axis, and ``"problems"`` records the pairs.  Without it, results are
    shaped [B, H, ...].
    """
    q = np.asarray(q)
    bsz, heads = q.shape[0], q.shape[1]
    pairs = list(problems) if problems is not None else [(b, h) for b in range(bsz) for h in range(heads)]
    outs = [attention_problem(q[b, h], k[b, h], v[b, h], grid_h=grid_h, grid_w=grid_w, pool=pool,
                              lam=lam, eps=eps, ns_iters=ns_iters, whiten=whiten, refine=refine, kernel=kernel,
                              solver=solver)
            for (b, h) in pairs]
    res = {key: np.stack([o[key] for o in outs]) for key in outs[0] if outs[0][key] is not None}
    if problems is None:
        res = {key: val.reshape((bsz, heads) + val.shape[1:]) for key, val in res.items()}
    res["problems"] = pairs
    return res
