"""lapnys_forward_noalloc: the forward on the library's static device scratch
(for callers that cannot allocate), against lapnys_forward_ws on the same
inputs, on two calls in a row, the second with a smaller input; and the
refusal of a problem whose workspace exceeds the scratch."""

import ctypes
import sys

import numpy as np
import pytest

from gpu_harness import device_inputs, gpu_available, workload_inputs
from lapnys_inputs import WORKLOADS

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="no GPU device visible")]


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _outputs(w):
    import torch
    import laplacian_nystr_approximation_amd as L
    x = workload_inputs(w)
    q, k, v = device_inputs(x, w.dtype)
    params = L.params_for(w)
    ws = torch.empty(L.lapnys_workspace_size(params), dtype=torch.uint8, device="cuda")
    a = torch.empty((w.B, w.H, w.N, w.d), dtype=torch.float32, device="cuda")
    b = torch.full_like(a, float("nan"))
    L.lapnys_forward_ws(q, k, v, a, params, ws)
    L.lapnys_forward_noalloc(q, k, v, b, params)
    torch.cuda.synchronize()
    return a.cpu().numpy(), b.cpu().numpy()


def test_noalloc_matches_workspace_form_twice():
    """Two calls in a row, the second smaller; each bit-identical to
    lapnys_forward_ws (same kernels, same workspace layout), so the stale
    contents the first call leaves in the scratch do not matter."""
    for name in ("stage1_56x56_bf16", "tiny_f32"):
        w = WORKLOADS[name]
        _say(f"[noalloc] {name} P={w.P} N={w.N} m={w.m} {w.dtype}")
        a, b = _outputs(w)
        assert np.all(np.isfinite(b))
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), name


def test_noalloc_refuses_beyond_scratch_and_other_forms():
    """Before anything is enqueued: a workspace beyond the scratch maximum is
    LAPNYS_ERR_SCRATCH; forms that need a second stream are unsupported."""
    import laplacian_nystr_approximation_amd as L
    from laplacian_nystr_approximation_amd import lapnys as B
    lib = L.library()
    a = 1 << 24
    big = L.params_for(WORKLOADS["stage1_56x56_bf16"].with_(B=128))  # 106 MiB of workspace
    assert L.lapnys_workspace_size(big) > B.LAPNYS_SCRATCH_MAX_BYTES
    assert lib.lapnys_forward_noalloc(a, 2 * a, 3 * a, 4 * a, ctypes.byref(big), None) == B.LAPNYS_ERR_SCRATCH
    plain = L.params_for(WORKLOADS["tiny_f32"].with_(ns_plain=True))
    assert lib.lapnys_forward_noalloc(a, 2 * a, 3 * a, 4 * a, ctypes.byref(plain), None) == B.LAPNYS_ERR_UNSUPPORTED
