"""Pins for the CPU oracle (no GPU).

Each ``pin_*`` function checks the oracle against something that does not come
from the oracle itself: hand-worked values (tests/golden), closed forms,
library routines (LU inverse, eigendecomposition, numpy mean/std), brute force
on tiny inputs, and invariants the mathematics fixes.  ``test_planted_mistakes``
then plants plausible mistakes in the oracle (on the CPU) and checks that at
least one pin fails for each, so the pins are known to have teeth.
"""

import math
import os

import numpy as np
import pytest

import oracle.lapnys_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "laplacian_kernel_hand.txt")
GOLDEN_GAUSS = os.path.join(os.path.dirname(__file__), "golden", "gaussian_kernel_hand.txt")


def _rng(seed=0):
    return np.random.Generator(np.random.PCG64(seed))


def _heavy(rng, shape):
    return rng.standard_t(3.0, size=shape) * 0.25


def _golden_rows(path=GOLDEN):
    rows = []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            x, y, lam, dist, _ = [s.strip() for s in line.split(";")]
            rows.append((np.array([float(t) for t in x.split(",")]),
                         np.array([float(t) for t in y.split(",")]), float(lam), float(dist)))
    return rows


# ----------------------------------------------------------------------------- pins


def pin_kernel_hand(orc):
    for x, y, lam, dist in _golden_rows():
        got = orc.laplacian_kernel(x[None, :], y[None, :], lam)[0, 0]
        want = math.exp(-dist / lam)
        assert abs(got - want) <= 1e-15 * want, (x, y, lam, got, want)


def pin_kernel_invariants(orc):
    rng = _rng(1)
    x = _heavy(rng, (9, 6))
    kxx = orc.laplacian_kernel(x, x, 4.0)
    assert np.all(np.diag(kxx) == 1.0)
    assert np.array_equal(kxx, kxx.T)
    assert np.all(kxx > 0) and np.all(kxx <= 1)
    # The Laplacian kernel is a product of one-dimensional Laplace kernels, each
    # positive definite, so its Gram matrix on distinct points is positive definite.
    assert np.linalg.eigvalsh(kxx).min() > 0
    y = _heavy(rng, (4, 6))
    assert np.array_equal(orc.laplacian_kernel(x, y, 4.0), orc.laplacian_kernel(y, x, 4.0).T)


def pin_gaussian_hand(orc):
    for x, y, lam, dist2 in _golden_rows(GOLDEN_GAUSS):
        got = orc.gaussian_kernel(x[None, :], y[None, :], lam)[0, 0]
        want = math.exp(-dist2 / lam)
        assert abs(got - want) <= 1e-15 * want, (x, y, lam, got, want)


def pin_gaussian_library_and_invariants(orc):
    from scipy.spatial.distance import cdist
    rng = _rng(12)
    x, y = _heavy(rng, (11, 7)), _heavy(rng, (5, 7))
    lam = 4.0
    got = orc.gaussian_kernel(x, y, lam)
    want = np.exp(-cdist(x, y, "sqeuclidean") / lam)
    assert np.abs(got - want).max() <= 1e-14
    # A product of one-dimensional Gaussians, one per feature.
    prod = np.ones((11, 5))
    for t in range(7):
        prod *= np.exp(-((x[:, t, None] - y[None, :, t]) ** 2) / lam)
    assert np.abs(got - prod).max() <= 1e-14
    kxx = orc.gaussian_kernel(x, x, lam)
    assert np.all(np.diag(kxx) == 1.0)
    assert np.array_equal(kxx, kxx.T)
    assert np.linalg.eigvalsh(kxx).min() > 0  # positive definite on distinct points
    # Against the Laplacian kernel on the same points: where every per-feature
    # difference is below 1 in magnitude, the squared distance is the smaller.
    small = x[:3] * 0.1
    assert np.all(orc.gaussian_kernel(small, small[::-1], lam) >= orc.laplacian_kernel(small, small[::-1], lam))


def pin_gaussian_nystrom_pool1(orc):
    # The pool = 1 identity holds for any kernel: with G = k(K, K) and an exact
    # inverse, C (G + eps I)^-1 G = C - eps C (G + eps I)^-1, here for the
    # Gaussian kernel through the whole forward, against brute force.
    rng = _rng(13)
    gh, gw, d, lam = 3, 4, 3, 4.0
    q, k, v = (_heavy(rng, (gh * gw, d)) for _ in range(3))
    g_qk = np.exp(-np.array([[sum((a - b) ** 2 for a, b in zip(qi, kj)) for kj in k] for qi in q]) / lam)
    g_kk = np.exp(-np.array([[sum((a - b) ** 2 for a, b in zip(ki, kj)) for kj in k] for ki in k]) / lam)
    for eps in [1e-1, 1e-2]:
        res = orc.attention_problem(q, k, v, grid_h=gh, grid_w=gw, pool=1, lam=lam, eps=eps,
                                    ns_iters=120, whiten=False, kernel="gaussian")
        a = g_kk + eps * np.eye(gh * gw)
        want = (g_qk - eps * g_qk @ np.linalg.solve(a, np.eye(gh * gw))) @ v
        assert np.abs(res["O"] - want).max() <= 1e-9 * np.abs(want).max(), eps
        assert np.abs(res["W"] - a).max() <= 1e-15


def _spd(rng, m, eigs):
    qm, _ = np.linalg.qr(rng.standard_normal((m, m)))
    return (qm * np.asarray(eigs, float)) @ qm.T


def pin_cg_finite_termination(orc):
    # In exact arithmetic CG solves an m x m SPD system in at most m steps, and
    # in as many steps as W has distinct eigenvalues.
    rng = _rng(20)
    w = _spd(rng, 6, [0.5, 1.0, 2.0, 3.0, 5.0, 8.0])
    b = rng.standard_normal((6, 3))
    want = np.linalg.solve(w, b)
    got = orc.conjugate_gradient(w, b, 6)
    assert np.abs(got - want).max() <= 1e-10 * np.abs(want).max()
    w3 = _spd(rng, 8, [1.0, 1.0, 1.0, 4.0, 4.0, 9.0, 9.0, 9.0])
    b3 = rng.standard_normal((8, 2))
    got3 = orc.conjugate_gradient(w3, b3, 3)
    assert np.abs(w3 @ got3 - b3).max() <= 1e-10 * np.abs(b3).max()
    got2 = orc.conjugate_gradient(w3, b3, 2)
    assert np.abs(w3 @ got2 - b3).max() > 1e-4  # not yet


def pin_cg_first_step_and_monotone(orc):
    # Step one is a steepest-descent step, y1 = (b.b / b.Wb) b; the W-norm of the
    # error never grows; a zero right-hand side stays zero.
    rng = _rng(21)
    w = _spd(rng, 7, np.geomspace(0.1, 10.0, 7))
    b = rng.standard_normal((7, 2))
    b[:, 1] = 0.0
    y1 = orc.conjugate_gradient(w, b, 1)
    col = b[:, 0]
    assert np.allclose(y1[:, 0], (col @ col) / (col @ w @ col) * col, rtol=1e-13, atol=0)
    assert np.all(y1[:, 1] == 0.0)
    ystar = np.linalg.solve(w, b[:, :1])
    errs = []
    for t in range(0, 8):
        e = orc.conjugate_gradient(w, b, t)[:, :1] - ystar
        errs.append(float(np.sqrt((e.T @ w @ e)[0, 0])))
    assert all(errs[i + 1] <= errs[i] * (1 + 1e-12) for i in range(len(errs) - 1)), errs
    assert errs[3] < 0.9 * errs[0]


def pin_cg_in_forward(orc):
    # solver="cg" feeds Y = CG(W, B V) to the output product: with enough steps it
    # reaches the same output as an exact solve.
    rng = _rng(22)
    gh, gw, d = 6, 6, 4
    q, k, v = (_heavy(rng, (gh * gw, d)) for _ in range(3))
    res = orc.attention_problem(q, k, v, grid_h=gh, grid_w=gw, pool=2, lam=4.0, eps=1e-2, ns_iters=40,
                                solver="cg")
    want = res["Z"] @ np.linalg.solve(res["W"], res["BV"])
    assert np.abs(res["O"] - want).max() <= 1e-9 * np.abs(want).max()
    assert res["X"] is None
    assert np.abs(res["Y"] - orc.conjugate_gradient(res["W"], res["BV"], 40)).max() == 0.0


def pin_pool_ramp(orc):
    # K[n, t] = n + 1000 t on a row-major grid: the window mean has a closed form.
    for gh, gw, p in [(6, 10, 2), (9, 6, 3), (4, 8, 4), (5, 5, 1)]:
        n = np.arange(gh * gw, dtype=np.float64)
        d = 3
        k = n[:, None] + 1000.0 * np.arange(d)[None, :]
        kt = orc.pool_landmarks(k, gh, gw, p)
        R, C = np.divmod(np.arange((gh // p) * (gw // p)), gw // p)
        centre = (R * p + (p - 1) / 2.0) * gw + (C * p + (p - 1) / 2.0)
        want = centre[:, None] + 1000.0 * np.arange(d)[None, :]
        assert kt.shape == want.shape
        assert np.allclose(kt, want, rtol=0, atol=1e-9), (gh, gw, p)


def pin_pool_special_cases(orc):
    rng = _rng(2)
    k = _heavy(rng, (30, 4))
    assert np.array_equal(orc.pool_landmarks(k, 5, 6, 1), k)           # pool 1: identity
    g = _heavy(rng, (36, 4))
    assert np.allclose(orc.pool_landmarks(g, 6, 6, 6)[0], g.mean(axis=0), rtol=0, atol=1e-15)


def pin_pool_fixed_order(orc):
    # The GPU reproduces the landmarks bit for bit, so the float64 summation order
    # is part of the definition: window row outer, window column inner.
    # Values with exponents spread over 2^-40..2^40 make float64 window sums
    # depend on their order, so a different order shows up as a bit change.
    rng = _rng(3)
    gh, gw, p, d = 6, 8, 2, 5
    mant = rng.uniform(1.0, 2.0, size=(gh * gw, d)) * rng.choice([-1.0, 1.0], size=(gh * gw, d))
    k = (mant * np.exp2(rng.integers(-40, 41, size=(gh * gw, d)))).astype(np.float32).astype(np.float64)
    k[0, 0], k[1, 0], k[gw, 0], k[gw + 1, 0] = 2.0 ** 60, 1.0, -(2.0 ** 60), 0.5
    kt = orc.pool_landmarks(k, gh, gw, p)
    assert kt[0, 0] == 0.125  # ((2^60 + 1) - 2^60 + 0.5) / 4 in float64
    for j in range((gh // p) * (gw // p)):
        R, C = divmod(j, gw // p)
        for t in range(d):
            acc = 0.0
            for r in range(p):
                for c in range(p):
                    acc += k[(R * p + r) * gw + (C * p + c), t]
            assert kt[j, t] == acc / (p * p)


def _w_of(rng, m=7, d=4, eps=1e-3):
    kt = _heavy(rng, (m, d))
    return O.laplacian_kernel(kt, kt, 4.0) + eps * np.eye(m)


def pin_ns_closed_form(orc):
    # For symmetric W with X0 = W / alpha, the residual squares each step, so
    # X_T = W^-1 (I - (I - W^2 / alpha)^(2^T)); evaluate it on W's eigenbasis.
    rng = _rng(4)
    w = _w_of(rng)
    alpha = np.linalg.norm(w, 1) * np.linalg.norm(w, np.inf)
    s, u = np.linalg.eigh(w)
    for t in [0, 1, 3, 8]:
        want = (u * ((1.0 - (1.0 - s * s / alpha) ** (2 ** t)) / s)) @ u.T
        got = orc.newton_schulz_inverse(w, t)
        assert np.abs(got - want).max() <= 1e-12 * np.abs(want).max(), t


def pin_ns_lu(orc):
    rng = _rng(5)
    w = _w_of(rng, m=5)
    got = orc.newton_schulz_inverse(w, 60)
    want = np.linalg.solve(w, np.eye(5))
    assert np.abs(got - want).max() <= 1e-12 * np.abs(want).max()


def pin_ns_residual_squares(orc):
    rng = _rng(6)
    w = _w_of(rng, m=6)
    prev = None
    for t in range(6):
        r = np.linalg.norm(np.eye(6) - w @ orc.newton_schulz_inverse(w, t), 2)
        if prev is not None:
            assert abs(r - prev * prev) <= 1e-9 * max(prev * prev, 1e-300) + 1e-15
        prev = r


def pin_whiten_moments(orc):
    rng = _rng(7)
    c = np.exp(-np.abs(_heavy(rng, (50, 6))) * 3)
    z, mu, sigma = orc.whiten_columns(c)
    assert np.allclose(mu, np.mean(c, axis=0), rtol=1e-14, atol=0)
    assert np.allclose(sigma, np.std(c, axis=0, ddof=0), rtol=1e-13, atol=0)
    assert np.abs(z.mean(axis=0)).max() <= 1e-12
    assert np.abs((z * z).mean(axis=0) - 1.0).max() <= 1e-12
    c2 = c.copy()
    c2[:, 2] = 0.25
    z2, _, s2 = orc.whiten_columns(c2)
    assert s2[2] == 0 and np.all(z2[:, 2] == 0)


def _brute_kernel(x, y, lam):
    out = np.empty((x.shape[0], y.shape[0]))
    for i in range(x.shape[0]):
        for j in range(y.shape[0]):
            out[i, j] = math.exp(-sum(abs(a - b) for a, b in zip(x[i], y[j])) / lam)
    return out


def pin_nystrom_pool1(orc):
    # pool = 1 makes every key a landmark.  With an exact inverse the Nystrom
    # product then equals C - eps C (k(K,K) + eps I)^-1 exactly, and tends to
    # the brute-force O(N^2) Laplacian attention k(Q, K) V as eps -> 0.
    rng = _rng(8)
    gh, gw, d, lam = 4, 4, 3, 4.0
    q, k, v = (_heavy(rng, (gh * gw, d)) for _ in range(3))
    g_qk = _brute_kernel(q, k, lam)
    g_kk = _brute_kernel(k, k, lam)
    errs = []
    for eps in [1e-2, 1e-4, 1e-6]:
        res = orc.attention_problem(q, k, v, grid_h=gh, grid_w=gw, pool=1, lam=lam, eps=eps,
                                    ns_iters=80, whiten=False)
        a = g_kk + eps * np.eye(gh * gw)
        want = (g_qk - eps * g_qk @ np.linalg.solve(a, np.eye(gh * gw))) @ v
        assert np.abs(res["O"] - want).max() <= 1e-9 * np.abs(want).max(), eps
        errs.append(np.abs(res["O"] - g_qk @ v).max())
    assert errs[0] > errs[1] > errs[2]
    assert errs[2] < 1e-3 * np.abs(g_qk @ v).max()


def pin_single_landmark(orc):
    # pool = whole grid: one landmark (the mean key), W = 1 + eps, X_T = 1/(1+eps),
    # so O_i = z_i / (1 + eps) * sum_n b_n v_n.
    rng = _rng(9)
    g, d, lam, eps = 5, 4, 4.0, 1e-3
    q, k, v = (_heavy(rng, (g * g, d)) for _ in range(3))
    res = orc.attention_problem(q, k, v, grid_h=g, grid_w=g, pool=g, lam=lam, eps=eps,
                                ns_iters=20, whiten=True)
    kbar = k.mean(axis=0)
    c = np.array([math.exp(-np.abs(qi - kbar).sum() / lam) for qi in q])
    b = np.array([math.exp(-np.abs(kbar - kn).sum() / lam) for kn in k])
    z = (c - c.mean()) / c.std()
    want = np.outer(z / (1.0 + eps), (b[:, None] * v).sum(axis=0))
    assert np.abs(res["O"] - want).max() <= 1e-12 * np.abs(want).max()


def _problem(orc, q, k, v, **kw):
    base = dict(grid_h=6, grid_w=6, pool=2, lam=4.0, eps=1e-3, ns_iters=20, whiten=True)
    base.update(kw)
    return orc.attention_problem(q, k, v, **base)


def pin_metamorphic(orc):
    rng = _rng(10)
    q, k, v, v2 = (_heavy(rng, (36, 5)) for _ in range(4))
    r = _problem(orc, q, k, v)
    # Linear in V.
    r2 = _problem(orc, q, k, v2)
    r3 = _problem(orc, q, k, 2.0 * v - 3.0 * v2)
    assert np.allclose(r3["O"], 2.0 * r["O"] - 3.0 * r2["O"], rtol=0, atol=1e-12 * np.abs(r["O"]).max())
    # Permuting the queries permutes the output rows (whitening statistics are
    # symmetric in the tokens).
    perm = rng.permutation(36)
    rp = _problem(orc, q[perm], k, v)
    assert np.allclose(rp["O"], r["O"][perm], rtol=0, atol=1e-12 * np.abs(r["O"]).max())
    # (Q, K, lambda) -> (2Q, 2K, 2 lambda) leaves every kernel value bit-identical.
    rs = _problem(orc, 2 * q, 2 * k, v, lam=8.0)
    for key in ["C", "B", "W", "X", "O"]:
        assert np.array_equal(rs[key], r[key]), key
    assert np.array_equal(rs["landmarks"], 2 * r["landmarks"])


def pin_forward_layout(orc):
    # forward() runs each (b, h) problem independently on its own slice.
    rng = _rng(11)
    q, k, v = (_heavy(rng, (2, 3, 16, 4)) for _ in range(3))
    kw = dict(grid_h=4, grid_w=4, pool=2, lam=4.0, eps=1e-3, ns_iters=20)
    res = orc.forward(q, k, v, **kw)
    assert res["O"].shape == (2, 3, 16, 4)
    one = orc.attention_problem(q[1, 2], k[1, 2], v[1, 2], **kw)
    assert np.array_equal(res["O"][1, 2], one["O"])
    samp = orc.forward(q, k, v, problems=[(1, 2)], **kw)
    assert np.array_equal(samp["O"][0], one["O"])


def pin_refine_squares_residual(orc):
    # One correction step X' = X + X R, R = I - W X, leaves I - W X' = R^2
    # exactly in exact arithmetic; in float64 to rounding.  The start is a
    # short Newton-Schulz run, so R is far from zero.
    rng = _rng(12)
    lm = _heavy(rng, (30, 6))
    w = orc.laplacian_kernel(lm, lm, 4.0) + 1e-3 * np.eye(30)
    x = orc.newton_schulz_inverse(w, 17)
    r = np.eye(30) - w @ x
    assert 1e-3 < np.abs(r).max() < 0.5
    x2 = orc.refine_inverse(w, x)
    r2 = np.eye(30) - w @ x2
    assert np.abs(r2 - r @ r).max() <= 1e-12
    # and it moves X towards the inverse by the same factor
    inv = np.linalg.inv(w)
    assert np.abs(x2 - inv).max() <= 1.01 * np.abs(r @ r).max() * np.abs(inv).sum(axis=1).max() + 1e-12


PINS = [pin_kernel_hand, pin_kernel_invariants, pin_pool_ramp, pin_pool_special_cases,
        pin_pool_fixed_order, pin_ns_closed_form, pin_ns_lu, pin_ns_residual_squares,
        pin_whiten_moments, pin_nystrom_pool1, pin_single_landmark, pin_metamorphic,
        pin_forward_layout, pin_refine_squares_residual, pin_gaussian_hand,
        pin_gaussian_library_and_invariants, pin_gaussian_nystrom_pool1, pin_cg_finite_termination,
        pin_cg_first_step_and_monotone, pin_cg_in_forward]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(O)


def test_headline_shapes_converge_in_fp64():
    """At the 14x14 tiny shape, 20 float64 steps reach the inverse to ~1e-14."""
    from lapnys_inputs import WORKLOADS, make_inputs
    w = WORKLOADS["tiny_f32"]
    x = make_inputs(w)
    res = O.attention_problem(x.qf[0, 0], x.kf[0, 0], x.vf[0, 0], grid_h=w.grid_h, grid_w=w.grid_w,
                              pool=w.pool, lam=w.lam, eps=w.eps, ns_iters=w.ns_iters)
    r = np.linalg.norm(res["W"] @ res["X"] - np.eye(w.m))
    assert r < 1e-12
    assert np.all(res["C"] > 0) and np.all(res["C"] <= 1)


# ----------------------------------------------------------------- planted mistakes


def _k_signed(x, y, lam):
    x, y = np.asarray(x, float), np.asarray(y, float)
    return np.exp(-(x[:, None, :] - y[None, :, :]).sum(axis=2) / lam)


def _k_l2sq(x, y, lam):
    x, y = np.asarray(x, float), np.asarray(y, float)
    return np.exp(-((x[:, None, :] - y[None, :, :]) ** 2).sum(axis=2) / lam)


def _k_times_lam(x, y, lam):
    x, y = np.asarray(x, float), np.asarray(y, float)
    return np.exp(-np.abs(x[:, None, :] - y[None, :, :]).sum(axis=2) * lam / 16.0)


def _pool_colmajor(k, gh, gw, p):
    k = np.asarray(k, float)
    g = k.reshape(gw, gh, -1).transpose(1, 0, 2)
    acc = sum(g[r::p, c::p] for r in range(p) for c in range(p))
    return (acc / (p * p)).reshape((gh // p) * (gw // p), -1)


def _pool_colmajor_landmarks(k, gh, gw, p):
    k = np.asarray(k, float)
    g = k.reshape(gh, gw, -1)
    acc = sum(g[r::p, c::p] for r in range(p) for c in range(p))
    return (acc / (p * p)).transpose(1, 0, 2).reshape((gh // p) * (gw // p), -1)


def _pool_sum(k, gh, gw, p):
    k = np.asarray(k, float)
    g = k.reshape(gh, gw, -1)
    return sum(g[r::p, c::p] for r in range(p) for c in range(p)).reshape((gh // p) * (gw // p), -1)


def _pool_reversed_order(k, gh, gw, p):
    k = np.asarray(k, float)
    g = k.reshape(gh, gw, -1)
    acc = np.zeros((gh // p, gw // p, g.shape[2]))
    for c in range(p):
        for r in range(p):
            acc = acc + g[r::p, c::p]
    return (acc / (p * p)).reshape((gh // p) * (gw // p), -1)


def _ns_no_alpha(w, iters):
    x = np.asarray(w, float).T.copy()
    for _ in range(iters):
        x = x @ (2 * np.eye(len(w)) - w @ x)
    return x


def _ns_frob_alpha(w, iters):
    x = np.asarray(w, float).T / (np.linalg.norm(w) ** 2)
    for _ in range(iters):
        x = x @ (2 * np.eye(len(w)) - w @ x)
    return x


def _ns_extra_step(w, iters):
    return O.__dict__["_orig_ns"](w, iters + 1)


def _ns_missing_two(w, iters):
    w = np.asarray(w, float)
    x = w.T / (np.abs(w).sum(0).max() * np.abs(w).sum(1).max())
    for _ in range(iters):
        x = x @ (np.eye(len(w)) - w @ x)
    return x


def _whiten_sample_var(c):
    mu = c.mean(axis=0)
    sigma = c.std(axis=0, ddof=1)
    return (c - mu) / sigma, mu, sigma


def _whiten_rows(c):
    mu = c.mean(axis=1, keepdims=True)
    sigma = c.std(axis=1, keepdims=True)
    return (c - mu) / sigma, mu[:, 0], sigma[:, 0]


def _refine_plus_residual(w, x):
    w = np.asarray(w, float)
    x = np.asarray(x, float)
    return x + x @ (np.eye(len(w)) + w @ x)


def _refine_minus(w, x):
    w = np.asarray(w, float)
    x = np.asarray(x, float)
    return x - x @ (np.eye(len(w)) - w @ x)


def _g_unsquared(x, y, lam):
    x, y = np.asarray(x, float), np.asarray(y, float)
    return np.exp(-np.sqrt(((x[:, None, :] - y[None, :, :]) ** 2).sum(axis=2)) / lam)


def _g_half_scale(x, y, lam):
    x, y = np.asarray(x, float), np.asarray(y, float)
    return np.exp(-((x[:, None, :] - y[None, :, :]) ** 2).sum(axis=2) / (2 * lam))


def _g_expansion_sign(x, y, lam):
    x, y = np.asarray(x, float), np.asarray(y, float)
    d2 = (x * x).sum(1)[:, None] + (y * y).sum(1)[None, :] + 2 * x @ y.T
    return np.exp(-d2 / lam)


def _cg_variant(variant):
    def f(w, rhs, iters):
        w = np.asarray(w, float)
        y = np.zeros_like(rhs, dtype=float)
        r = np.array(rhs, dtype=float)
        p = r.copy()
        rr = (r * r).sum(0)
        for _ in range(iters):
            q = w @ p
            den = (p * p).sum(0) if variant == "alpha_pp" else (p * q).sum(0)
            a = np.where(rr > 0, rr / np.where(rr > 0, den, 1.0), 0.0)
            y = y + a * p
            r = r + a * q if variant == "residual_sign" else r - a * q
            rn = (r * r).sum(0)
            bta = np.where(rr > 0, (rr / np.where(rn > 0, rn, 1.0)) if variant == "beta_inverted"
                           else rn / np.where(rr > 0, rr, 1.0), 0.0)
            p = r if variant == "steepest_descent" else r + bta * p
            rr = rn
        return y
    return f


def _attention_variant(variant):
    def f(q, k, v, *, grid_h, grid_w, pool, lam, eps, ns_iters, whiten=True, refine=False, kernel="laplacian",
          solver="ns"):
        kt = O.pool_landmarks(k, grid_h, grid_w, pool)
        m = kt.shape[0]
        kf = O.gaussian_kernel if kernel == "gaussian" else O.laplacian_kernel
        c = kf(q, kt, lam)
        b = kf(kt, q if variant == "b_from_q" else k, lam)
        wk = O.laplacian_kernel if variant == "gaussian_w_laplacian" else kf
        w = wk(kt, kt, lam) + (0.0 if variant == "no_eps" else eps) * np.eye(m)
        x = O.newton_schulz_inverse(w, ns_iters)
        if variant == "skip_inverse":
            x = np.eye(m)
        if refine:
            x = O.refine_inverse(w, x)
        if whiten:
            z, mu, sigma = O.whiten_columns(c)
        else:
            z, mu, sigma = c, np.zeros(m), np.ones(m)
        bv = b @ v
        if solver == "cg":
            x = None
            y = O.conjugate_gradient(w, bv, ns_iters)
            if variant == "skip_inverse":
                y = bv
        else:
            y = x @ bv
        o = z @ y
        return {"landmarks": kt, "C": c, "B": b, "W": w, "X": x, "Z": z,
                "mu": mu, "sigma": sigma, "BV": bv, "Y": y, "O": o}
    return f


MUTANTS = {
    "kernel_signed_difference": ("laplacian_kernel", _k_signed),
    "kernel_squared_l2": ("laplacian_kernel", _k_l2sq),
    "kernel_scale_by_lambda": ("laplacian_kernel", _k_times_lam),
    "pool_column_major_tokens": ("pool_landmarks", _pool_colmajor),
    "pool_column_major_landmarks": ("pool_landmarks", _pool_colmajor_landmarks),
    "pool_sum_not_mean": ("pool_landmarks", _pool_sum),
    "pool_reversed_sum_order": ("pool_landmarks", _pool_reversed_order),
    "ns_no_scaling": ("newton_schulz_inverse", _ns_no_alpha),
    "ns_frobenius_scaling": ("newton_schulz_inverse", _ns_frob_alpha),
    "ns_one_extra_step": ("newton_schulz_inverse", _ns_extra_step),
    "ns_update_missing_two": ("newton_schulz_inverse", _ns_missing_two),
    "whiten_sample_variance": ("whiten_columns", _whiten_sample_var),
    "whiten_per_token": ("whiten_columns", _whiten_rows),
    "key_factor_from_queries": ("attention_problem", _attention_variant("b_from_q")),
    "no_diagonal_shift": ("attention_problem", _attention_variant("no_eps")),
    "inverse_skipped": ("attention_problem", _attention_variant("skip_inverse")),
    "refine_residual_sign": ("refine_inverse", _refine_plus_residual),
    "refine_correction_sign": ("refine_inverse", _refine_minus),
    "gaussian_unsquared_distance": ("gaussian_kernel", _g_unsquared),
    "gaussian_half_scale": ("gaussian_kernel", _g_half_scale),
    "gaussian_expansion_sign": ("gaussian_kernel", _g_expansion_sign),
    "gaussian_w_from_laplacian": ("attention_problem", _attention_variant("gaussian_w_laplacian")),
    "cg_alpha_over_pp": ("conjugate_gradient", _cg_variant("alpha_pp")),
    "cg_residual_sign": ("conjugate_gradient", _cg_variant("residual_sign")),
    "cg_beta_inverted": ("conjugate_gradient", _cg_variant("beta_inverted")),
    "cg_steepest_descent": ("conjugate_gradient", _cg_variant("steepest_descent")),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setitem(O.__dict__, "_orig_ns", O.newton_schulz_inverse)
    monkeypatch.setattr(O, attr, fn)
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(O)
        except (AssertionError, ValueError, FloatingPointError, np.linalg.LinAlgError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {name}"
