"""Pins for the backward oracle (no GPU): the restated forward against the numpy
oracle, central finite differences, the closed-form V gradient, the two readings
of the inverse at convergence, and planted mistakes."""

import numpy as np
import pytest

import oracle.lapnys_backward_oracle as BO
import oracle.lapnys_oracle as O


def _heavy(rng, shape):
    return rng.standard_t(3.0, size=shape) * 0.25


def _problem(seed, gh=4, gw=6, d=3, pool=2):
    rng = np.random.Generator(np.random.PCG64(seed))
    q, k, v, g = (_heavy(rng, (gh * gw, d)) for _ in range(4))
    return q, k, v, g, dict(grid_h=gh, grid_w=gw, pool=pool, lam=4.0, eps=1e-2, ns_iters=30)


def _pin_forward_matches(bo):
    q, k, v, _, kw = _problem(1)
    for whiten in (True, False):
        want = O.attention_problem(q, k, v, whiten=whiten, **kw)["O"]
        got = bo.forward_values(q, k, v, whiten=whiten, **kw)
        assert np.abs(got - want).max() <= 1e-12 * np.abs(want).max()


def _pin_finite_differences(bo):
    q, k, v, g, kw = _problem(2)
    dq, dk, dv = bo.backward(q, k, v, g, **kw)

    def loss(qq, kk, vv):
        return float((bo.forward_values(qq, kk, vv, **kw) * g).sum())

    rng = np.random.Generator(np.random.PCG64(3))
    h = 1e-6
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(6):
            i, t = rng.integers(arr.shape[0]), rng.integers(arr.shape[1])
            plus, minus = arr.copy(), arr.copy()
            plus[i, t] += h
            minus[i, t] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = plus, minus
            fd = (loss(args_p["q"], args_p["k"], args_p["v"]) - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
            assert abs(fd - grad[i, t]) <= 1e-6 * max(1.0, abs(fd)), (name, i, t, fd, grad[i, t])


def _pin_v_closed_form(bo):
    # O = Z X B V is linear in V, so dV = B^T X^T Z^T dO exactly.
    q, k, v, g, kw = _problem(4)
    _, _, dv = bo.backward(q, k, v, g, **kw)
    r = O.attention_problem(q, k, v, **kw)
    want = r["B"].T @ r["X"].T @ r["Z"].T @ g
    assert np.abs(dv - want).max() <= 1e-11 * np.abs(want).max()


def _pin_readings_agree(bo):
    q, k, v, g, kw = _problem(5)
    kw = dict(kw, ns_iters=60)
    a = bo.backward(q, k, v, g, through="unrolled", **kw)
    b = bo.backward(q, k, v, g, through="implicit", **kw)
    for x, y in zip(a, b):
        assert np.abs(x - y).max() <= 1e-8 * np.abs(y).max()
    # Before convergence the unrolled gradient is that of X_T, not of W^-1.
    c = bo.backward(q, k, v, g, through="unrolled", **dict(kw, ns_iters=3))
    assert np.abs(c[0] - b[0]).max() > 1e-3 * np.abs(b[0]).max()


PINS = [_pin_forward_matches, _pin_finite_differences, _pin_v_closed_form, _pin_readings_agree]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_backward_pin(pin):
    pin(BO)


def _k_squared(x, y, lam):
    return BO.torch.exp(-((x[:, None, :] - y[None, :, :]) ** 2).sum(dim=2) / lam)


def _whiten_no_sigma(c):
    return c - c.mean(dim=0)


def _pool_sum(k, grid_h, grid_w, pool):
    g = k.reshape(grid_h // pool, pool, grid_w // pool, pool, k.shape[-1])
    return g.sum(dim=(1, 3)).reshape(-1, k.shape[-1])


MUTANTS = {
    "kernel_squared_l2": ("laplacian_kernel_t", _k_squared),
    "whiten_without_sigma": ("whiten_t", _whiten_no_sigma),
    "pool_sum_not_mean": ("pool_landmarks_t", _pool_sum),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_planted_mistakes(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(BO, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin(BO)
        except (AssertionError, ValueError, RuntimeError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches {name}"
