"""Shared helpers for the GPU parity tests: upload seeded inputs, run the HIP
path through the C ABI (debug form, which also returns the intermediates),
run the oracle on the same values, and compare with the stated tolerances.

Tolerances (per (batch, head) problem):
  * landmarks: bit-exact (float32 rounding of the float64 window mean taken in
    a fixed order, on both sides);
  * output: normwise max relative error max|O_gpu - O_ref| / max|O_ref| <= 1e-4
    for every input type (both sides see the same input values, bf16 inputs
    widened exactly); for bf16 inputs the relative L2 error
    ||O_gpu - O_ref||_2 / ||O_ref||_2 <= 2e-2 is asserted as well;
  * Newton-Schulz iterate X, entry by entry: max|X_gpu - X_ref| <=
    4 u (kappa_1 + m) max|X_ref|, u = 2^-24 and kappa_1 = ||W||_1 ||X_ref||_1
    (the forward error of a float32 inverse, u kappa_1, plus the
    m-term accumulation, u m);
  * Y = X (B V), entry by entry, within what the X and B V gates allow plus
    the product's own float32 rounding (bound in y_bound);
  * Newton-Schulz residual ||W X - I||_F <= 1e-4, evaluated in float64 from the
    GPU's own float32 W and X.
Elementwise relative error is not used for O: outputs pass through zero, so
it is unbounded for a correct float32 result.
"""

from __future__ import annotations

import numpy as np

import oracle
from lapnys_inputs import Workload, make_inputs

O_NORMWISE_F32 = 1e-4
O_REL_L2_BF16 = 2e-2
NS_RESIDUAL = 1e-4
U32 = 2.0 ** -24  # float32 unit roundoff
BV_REL = 1e-4  # B V: max|BV_gpu - BV_ref| <= BV_REL max|BV_ref|


def f32(x):
    return float(np.float32(x))


def torch_mod():
    import torch
    return torch


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


def device_inputs(x, dtype: str):
    torch = torch_mod()

    def conv(a):
        if dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return conv(x.q), conv(x.k), conv(x.v)


def run_gpu(w: Workload, x, *, params=None, debug=True, cached=False):
    """Run the HIP forward on workload ``w`` with inputs ``x``; numpy results."""
    torch = torch_mod()
    import laplacian_nystr_approximation_amd as L
    params = params if params is not None else L.params_for(w)
    q, k, v = device_inputs(x, w.dtype)
    out = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.float32, device="cuda")
    res = {}
    if cached:
        L.lapnys_forward(q, k, v, out, params)
        torch.cuda.synchronize()
    else:
        ws = torch.empty(L.lapnys_workspace_size(params), dtype=torch.uint8, device="cuda")
        if debug:
            P, m = w.P, w.m
            dbg = {
                "landmarks": torch.empty((P, m, w.d), device="cuda"),
                "C_t": torch.empty((P, m, w.N), device="cuda"),
                "W": torch.empty((P, m, m), device="cuda"),
                "X": torch.empty((P, m, m), device="cuda"),
                "BV": torch.empty((P, m, w.d), device="cuda"),
                "Y": torch.empty((P, m, w.d), device="cuda"),
                "mu": torch.empty((P, m), device="cuda"),
                "sigma": torch.empty((P, m), device="cuda"),
            }
            L.lapnys_forward_debug(q, k, v, out, params, ws, dbg)
            res.update({key: t.cpu().numpy() for key, t in dbg.items()})
        else:
            L.lapnys_forward_ws(q, k, v, out, params, ws)
            torch.cuda.synchronize()
    res["O"] = out.cpu().numpy().reshape(w.P, w.N, w.d)
    return res


def run_oracle(w: Workload, x, problems=None):
    """Oracle results for the listed problem indices p = b*H + h (default all)."""
    pairs = None if problems is None else [divmod(p, w.H) for p in problems]
    r = oracle.forward(x.qf, x.kf, x.vf, grid_h=w.grid_h, grid_w=w.grid_w, pool=w.pool, lam=f32(w.lam),
                       eps=f32(w.eps), ns_iters=w.ns_iters, whiten=w.whiten, refine=w.refine,
                       kernel=w.kernel, solver=w.solver, problems=pairs)
    if problems is None:
        r = {k: (v.reshape((w.P,) + v.shape[2:]) if isinstance(v, np.ndarray) else v) for k, v in r.items()}
    return r


def o_errors(o_gpu, o_ref):
    d = o_gpu.astype(np.float64) - o_ref
    normwise = np.abs(d).max() / max(np.abs(o_ref).max(), 1e-300)
    rel_l2 = np.linalg.norm(d) / max(np.linalg.norm(o_ref), 1e-300)
    return normwise, rel_l2


def ns_residual(w_gpu, x_gpu):
    wd = w_gpu.astype(np.float64)
    xd = x_gpu.astype(np.float64)
    return np.linalg.norm(wd @ xd - np.eye(wd.shape[0]))


def x_tolerance(w_ref, x_ref):
    """Relative gate for the Newton-Schulz iterate: 4 u (kappa_1 + m)."""
    m = w_ref.shape[0]
    kappa1 = np.abs(w_ref).sum(axis=0).max() * np.abs(x_ref).sum(axis=0).max()
    return 4.0 * U32 * (kappa1 + m)


def y_bound(x_ref, bv_ref, tol_x):
    """Absolute gate for Y = X (B V): the X gate carried through the product,
    the B V gate carried through X, and the float32 rounding of an m-term
    product (4 u m of |X| |B V|)."""
    m = x_ref.shape[0]
    ax, ab = np.abs(x_ref), np.abs(bv_ref)
    return (tol_x * ax.max() * ab.sum(axis=0).max() + BV_REL * ab.max() * ax.sum(axis=1).max()
            + 4.0 * U32 * m * (ax @ ab).max())


def check_problem(w: Workload, gpu, g, ref, r, *, check_ns=True, check_o=True, report=None):
    """Compare GPU problem index g against oracle entry r; raise AssertionError on failure."""
    lm_ref = ref["landmarks"][r].astype(np.float32)
    assert np.array_equal(gpu["landmarks"][g].view(np.uint32), lm_ref.view(np.uint32)), "landmarks not bit-exact"
    wg = gpu["W"][g]
    assert np.array_equal(wg, wg.T), "W not bit-symmetric"
    diag = np.float32(1.0) + np.float32(w.eps)
    assert np.all(np.diag(wg) == diag), "W diagonal != 1 + eps in float32"
    assert np.abs(wg - ref["W"][r]).max() <= 2e-5, "W"
    if w.solver == "cg":
        # No X: the solve's own relative residual, from the GPU's W, Y and B V.
        wd, yd, bd = (gpu[key][g].astype(np.float64) for key in ("W", "Y", "BV"))
        res = np.linalg.norm(wd @ yd - bd) / np.linalg.norm(bd)
        if report is not None:
            report.setdefault("cg_residual", []).append(res)
    else:
        res = ns_residual(wg, gpu["X"][g])
        if report is not None:
            report.setdefault("ns_residual", []).append(res)
        if check_ns:
            assert res <= NS_RESIDUAL, f"NS residual {res:.3e}"
        # X and Y entry by entry against the oracle's (same W up to the W gate,
        # same step count).
        x_ref, bv_ref = ref["X"][r], ref["BV"][r]
        tol_x = x_tolerance(ref["W"][r], x_ref)
        ex = np.abs(gpu["X"][g].astype(np.float64) - x_ref).max() / np.abs(x_ref).max()
        ey = np.abs(gpu["Y"][g].astype(np.float64) - ref["Y"][r]).max()
        yb = y_bound(x_ref, bv_ref, tol_x)
        if report is not None:
            report.setdefault("x_rel", []).append(ex)
            report.setdefault("x_gate_use", []).append(ex / tol_x)
            report.setdefault("y_gate_use", []).append(ey / yb)
        assert ex <= tol_x, f"X: {ex:.3e} > {tol_x:.3e}"
        assert ey <= yb, f"Y: {ey:.3e} > {yb:.3e}"
    mu_ref, sg_ref = ref["mu"][r], ref["sigma"][r]
    assert np.abs(gpu["mu"][g] - mu_ref).max() <= 1e-5 * np.abs(mu_ref).max() + 1e-7, "mu"
    assert np.abs(gpu["sigma"][g] - sg_ref).max() <= 1e-4 * np.abs(sg_ref).max() + 1e-7, "sigma"
    ct_ref = ref["C"][r].T
    assert np.abs(gpu["C_t"][g] - ct_ref).max() <= 1e-5, "C"
    bv_ref = ref["BV"][r]
    assert np.abs(gpu["BV"][g] - bv_ref).max() <= BV_REL * np.abs(bv_ref).max(), "BV"
    nw, l2 = o_errors(gpu["O"][g], ref["O"][r])
    if report is not None:
        report.setdefault("o_normwise", []).append(nw)
        report.setdefault("o_rel_l2", []).append(l2)
    assert np.all(np.isfinite(gpu["O"][g])), "O not finite"
    if not check_o:
        return
    assert nw <= O_NORMWISE_F32, f"O normwise {nw:.3e}"
    if w.dtype == "bf16":
        assert l2 <= O_REL_L2_BF16, f"O rel L2 {l2:.3e}"


def workload_inputs(w: Workload, seed=None):
    return make_inputs(w, seed)
