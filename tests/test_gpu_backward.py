"""GPU parity of the backward pass (through the C ABI) against the backward
oracle's implicit reading (X = W^-1 in the derivative): dq, dk and dv of every
sampled problem, normwise (max |g - g_ref| / max |g_ref|) within 1e-4, the
forward's float32 bar; the inputs are exact on both sides for bf16 storage."""

import dataclasses
import sys

import numpy as np
import pytest

from gpu_harness import device_inputs, gpu_available, torch_mod, workload_inputs
from lapnys_inputs import WORKLOADS, Workload, make_grad_out

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="no GPU device visible")]


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _cases():
    base = dict(B=1, H=2, lam=4.0, eps=1e-3, ns_iters=20, seed_index=80)
    return [
        (WORKLOADS["tiny_f32"], None),
        (Workload("bwd_ragged_18x14_p2", grid_h=18, grid_w=14, d=64, pool=2, dtype="f32", **base), None),
        (Workload("bwd_nowhiten_14x14", grid_h=14, grid_w=14, d=32, pool=2, dtype="f32", whiten=False, **base), None),
        (Workload("bwd_pool1_7x9", grid_h=7, grid_w=9, d=32, pool=1, dtype="f32", **base), None),
        (Workload("bwd_single_landmark_6x6", grid_h=6, grid_w=6, d=64, pool=6, dtype="f32", **base), None),
        (WORKLOADS["stage3_14x14_bf16"], [0, 7, 319]),
        (WORKLOADS["stage1_56x56_f32"], [0, 31]),
        # the kernel-matrix stage's C and B halves in separate workgroups
        (WORKLOADS["stage2_28x28_bf16"], [0, 37, 63]),
        (dataclasses.replace(WORKLOADS["tiny_f32"], name="tiny_f32_plain", ns_plain=True), None),
        # the tiled solver's sizes: m = 81, 100 and 256
        (Workload("bwd_m81_18x18_p2", grid_h=18, grid_w=18, d=64, pool=2, dtype="f32", **base), None),
        (Workload("bwd_m100_20x20_p2_d32", grid_h=20, grid_w=20, d=32, pool=2, dtype="f32", **base), None),
        (Workload("bwd_m256_16x16_p1", grid_h=16, grid_w=16, d=64, pool=1, dtype="f32",
                  **{**base, "ns_iters": 40}), None),
        (WORKLOADS["sweep_64x64_bf16"], [0]),
        # bf16 with d = 32, the refined inverse, whitening off at m > 64
        (Workload("bwd_ragged_10x30_p5_d32", grid_h=10, grid_w=30, d=32, pool=5, dtype="bf16", **base), None),
        (dataclasses.replace(WORKLOADS["tiny_f32"], name="tiny_f32_refine", refine=True), None),
        (Workload("bwd_nowhiten_m81", grid_h=18, grid_w=18, d=64, pool=2, dtype="f32", whiten=False, **base), None),
    ]


@pytest.mark.parametrize("w,sample", _cases(), ids=lambda c: getattr(c, "name", "s"))
def test_backward_parity(w, sample):
    import laplacian_nystr_approximation_amd as L
    import oracle.lapnys_backward_oracle as BO
    torch = torch_mod()
    _say(f"[bwd] {w.name} P={w.P} N={w.N} m={w.m} d={w.d} {w.dtype} whiten={w.whiten}")
    x = workload_inputs(w)
    g = make_grad_out(w)
    q, k, v = device_inputs(x, w.dtype)
    dout = torch.from_numpy(g).cuda()
    dq, dk, dv = (torch.empty((w.B, w.H, w.N, w.d), dtype=torch.float32, device="cuda") for _ in range(3))
    params = L.params_for(w)
    ws = torch.empty(L.lapnys_backward_workspace_size(params), dtype=torch.uint8, device="cuda")
    L.lapnys_backward_ws(q, k, v, dout, dq, dk, dv, params, ws)
    torch.cuda.synchronize()
    got = [t.cpu().numpy().reshape(w.P, w.N, w.d) for t in (dq, dk, dv)]
    probs = sample if sample is not None else list(range(w.P))
    worst = [0.0, 0.0, 0.0]
    for p in probs:
        b, h = divmod(p, w.H)
        ref = BO.backward(x.qf[b, h], x.kf[b, h], x.vf[b, h], g[b, h].astype(np.float64), grid_h=w.grid_h,
                          grid_w=w.grid_w, pool=w.pool, lam=float(np.float32(w.lam)), eps=float(np.float32(w.eps)),
                          ns_iters=w.ns_iters, whiten=w.whiten, through="implicit")
        for n in range(3):
            assert np.all(np.isfinite(got[n][p]))
            err = np.abs(got[n][p] - ref[n]).max() / np.abs(ref[n]).max()
            worst[n] = max(worst[n], err)
    _say(f"[bwd] {w.name}: normwise dq {worst[0]:.2e} dk {worst[1]:.2e} dv {worst[2]:.2e}")
    assert max(worst) <= 1e-4
