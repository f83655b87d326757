"""The C ABI without a GPU: the library loads, exports every entry point that
include/lapnys.h declares, and rejects invalid calls with the documented
status before touching any device (no compute call is made here)."""

import ctypes
import os
import re
import subprocess

import pytest

import laplacian_nystr_approximation_amd as L
from laplacian_nystr_approximation_amd import lapnys as B
from lapnys_inputs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lapnys.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lapnys_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert _declared() == sorted([
        "lapnys_backward_workspace_size", "lapnys_backward_ws",
        "lapnys_forward", "lapnys_forward_debug", "lapnys_forward_noalloc", "lapnys_forward_profiled",
        "lapnys_forward_ws",
        "lapnys_landmark_count", "lapnys_release", "lapnys_status_string", "lapnys_workspace_size"])


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (lapnys_\w+)", nm))
    assert exported == set(_declared())


def test_struct_layout_matches_header():
    # 7 int32, 2 float, 2 int32, 1 uint32, no padding
    assert ctypes.sizeof(B.lapnys_params) == 12 * 4
    assert ctypes.sizeof(B.lapnys_debug) == 10 * ctypes.sizeof(ctypes.c_void_p)


def test_status_strings():
    for code in [0, -1, -2, -3, -4, -5, -6]:
        assert L.lapnys_status_string(code) not in ("", "unknown status")
    assert L.lapnys_status_string(-99) == "unknown status"


def _p(**kw):
    base = dict(B=2, H=3, grid_h=14, grid_w=14, d=64, pool=2, lam=4.0, eps=1e-3, ns_iters=20, dtype="bf16")
    base.update(kw)
    return L.make_params(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), B.LAPNYS_ERR_INVALID_ARG),
    (dict(H=-1), B.LAPNYS_ERR_INVALID_ARG),
    (dict(pool=0), B.LAPNYS_ERR_INVALID_ARG),
    (dict(lam=0.0), B.LAPNYS_ERR_INVALID_ARG),
    (dict(lam=float("inf")), B.LAPNYS_ERR_INVALID_ARG),
    (dict(lam=float("nan")), B.LAPNYS_ERR_INVALID_ARG),
    (dict(eps=-1e-3), B.LAPNYS_ERR_INVALID_ARG),
    (dict(ns_iters=-1), B.LAPNYS_ERR_INVALID_ARG),
    (dict(N=195), B.LAPNYS_ERR_SHAPE),
    (dict(pool=3), B.LAPNYS_ERR_SHAPE),
    (dict(d=48), B.LAPNYS_ERR_UNSUPPORTED),
    (dict(d=128), B.LAPNYS_ERR_UNSUPPORTED),
    (dict(dtype=7), B.LAPNYS_ERR_UNSUPPORTED),
    (dict(grid_h=34, grid_w=32, pool=2), B.LAPNYS_ERR_UNSUPPORTED),  # m = 272 > 256
    (dict(B=300, H=300), B.LAPNYS_ERR_UNSUPPORTED),
])
def test_invalid_params_rejected(kw, code):
    p = _p(**kw)
    with pytest.raises(L.LapnysError) as e:
        L.lapnys_workspace_size(p)
    assert e.value.code == code
    assert L.library().lapnys_landmark_count(ctypes.byref(p)) == code
    # The forward entry points validate before any device work; the buffer
    # arguments are never dereferenced on an error path.
    fake = 1 << 20
    rc = L.library().lapnys_forward_ws(fake, fake, fake, fake * 3, ctypes.byref(p), fake * 5, 1 << 30, None)
    assert rc == code
    rc = L.library().lapnys_forward(fake, fake, fake, fake * 3, ctypes.byref(p), None)
    assert rc == code


def test_unknown_flag_bits_rejected():
    p = _p()
    p.flags = 32
    assert L.library().lapnys_landmark_count(ctypes.byref(p)) == B.LAPNYS_ERR_INVALID_ARG


def test_refine_flag_accepted_and_sized():
    """LAPNYS_NS_REFINE is a known flag; with m <= 64 it adds the second
    iterate and the residual buffer (two P x 64 x 64 float32 arrays)."""
    plain, refined = _p(), _p(refine=True)
    assert refined.flags == B.LAPNYS_WHITEN | B.LAPNYS_NS_REFINE
    assert L.library().lapnys_landmark_count(ctypes.byref(refined)) == 49
    grow = L.lapnys_workspace_size(refined) - L.lapnys_workspace_size(plain)
    assert 2 * 6 * 64 * 64 * 4 <= grow <= 2 * 6 * 64 * 64 * 4 + 512
    big = dict(grid_h=32, grid_w=32)  # m = 256: the tiled solver has both buffers already
    assert L.lapnys_workspace_size(_p(refine=True, **big)) == L.lapnys_workspace_size(_p(**big))


def test_gaussian_flag_accepted():
    """LAPNYS_GAUSSIAN is a known flag and needs no other workspace: the
    intermediates are the same as the Laplacian form's."""
    g = _p(kernel="gaussian")
    assert g.flags == B.LAPNYS_WHITEN | B.LAPNYS_GAUSSIAN
    assert L.library().lapnys_landmark_count(ctypes.byref(g)) == 49
    assert L.lapnys_workspace_size(g) == L.lapnys_workspace_size(_p())
    big = dict(grid_h=32, grid_w=32)
    assert L.lapnys_workspace_size(_p(kernel="gaussian", **big)) == L.lapnys_workspace_size(_p(**big))
    with pytest.raises(ValueError):
        _p(kernel="cosine")


def test_binding_checks_tensor_sizes():
    """The binding refuses tensors whose element size or count does not match
    the params (the library sees only pointers), before any device call."""
    import torch
    p = _p(B=1, H=1, dtype="f32")
    n = 196 * 64
    good = torch.zeros(n, dtype=torch.float32)
    with pytest.raises(ValueError, match="q: expected"):
        L.lapnys_forward_ws(torch.zeros(n, dtype=torch.float64), good, good, good, p, 0)
    with pytest.raises(ValueError, match="out: expected"):
        L.lapnys_forward_ws(good, good, good, torch.zeros(n - 1), p, 0)
    with pytest.raises(ValueError, match="W: expected"):
        L.lapnys_forward_debug(good, good, good, good, p, 0, {"W": torch.zeros(10)})
    pb = _p(B=1, H=1, dtype="bf16")
    with pytest.raises(ValueError, match="k: expected"):
        L.lapnys_forward(torch.zeros(n, dtype=torch.int16), good, good, good, pb)


def test_plain_ns_flag():
    """LAPNYS_NS_PLAIN is a known flag and needs no other workspace at any m:
    at m <= 64 it moves the float32 steps into a launch of their own, and
    at m > 64 every step already takes float32 products."""
    pl = _p(ns_plain=True)
    assert pl.flags == B.LAPNYS_WHITEN | B.LAPNYS_NS_PLAIN
    assert L.library().lapnys_landmark_count(ctypes.byref(pl)) == 49
    assert L.lapnys_workspace_size(pl) == L.lapnys_workspace_size(_p())
    big = dict(grid_h=32, grid_w=32)  # m = 256
    assert L.lapnys_workspace_size(_p(ns_plain=True, **big)) == L.lapnys_workspace_size(_p(**big))


def test_backward_workspace_and_support():
    """The backward workspace extends the forward's (at m = 49 and m = 256);
    the Gaussian form and CG are refused as unsupported before any device call."""
    for p in (_p(), _p(grid_h=32, grid_w=32)):
        assert L.lapnys_backward_workspace_size(p) > L.lapnys_workspace_size(p)
    for bad in (_p(kernel="gaussian"), _p(solver="cg")):
        n = ctypes.c_size_t(0)
        assert L.library().lapnys_backward_workspace_size(ctypes.byref(bad), ctypes.byref(n)) == \
            B.LAPNYS_ERR_UNSUPPORTED


def test_cg_flag():
    """LAPNYS_SOLVER_CG is a known flag, refused together with LAPNYS_NS_REFINE;
    at m <= 64 it uses the separate-launch layout (no in-LDS solver)."""
    cg = _p(solver="cg")
    assert cg.flags == B.LAPNYS_WHITEN | B.LAPNYS_SOLVER_CG
    assert L.library().lapnys_landmark_count(ctypes.byref(cg)) == 49
    both = _p(solver="cg", refine=True)
    assert L.library().lapnys_landmark_count(ctypes.byref(both)) == B.LAPNYS_ERR_INVALID_ARG
    assert L.lapnys_workspace_size(cg) > 0
    with pytest.raises(ValueError):
        _p(solver="gmres")


def test_buffer_checks_before_launch():
    p = _p()
    lib = L.library()
    need = L.lapnys_workspace_size(p)
    a = 1 << 24
    q, k, v, out, ws = a, 2 * a, 3 * a, 4 * a, 8 * a
    # null and misaligned pointers
    assert lib.lapnys_forward_ws(None, k, v, out, ctypes.byref(p), ws, need, None) == B.LAPNYS_ERR_INVALID_ARG
    assert lib.lapnys_forward_ws(q + 4, k, v, out, ctypes.byref(p), ws, need, None) == B.LAPNYS_ERR_INVALID_ARG
    # out overlapping an input
    assert lib.lapnys_forward_ws(q, k, v, q + 256, ctypes.byref(p), ws, need, None) == B.LAPNYS_ERR_INVALID_ARG
    # workspace missing, too small, misaligned
    assert lib.lapnys_forward_ws(q, k, v, out, ctypes.byref(p), None, need, None) == B.LAPNYS_ERR_WORKSPACE
    assert lib.lapnys_forward_ws(q, k, v, out, ctypes.byref(p), ws, need - 1, None) == B.LAPNYS_ERR_WORKSPACE
    assert lib.lapnys_forward_ws(q, k, v, out, ctypes.byref(p), ws + 64, need, None) == B.LAPNYS_ERR_WORKSPACE
    # debug / profiled argument checks
    assert lib.lapnys_forward_debug(q, k, v, out, ctypes.byref(p), ws, need, None, None) == B.LAPNYS_ERR_INVALID_ARG
    assert lib.lapnys_forward_profiled(q, k, v, out, ctypes.byref(p), ws, need, None, None) == \
        B.LAPNYS_ERR_INVALID_ARG


def test_landmark_count_and_workspace():
    for name, w in WORKLOADS.items():
        p = L.params_for(w)
        assert L.lapnys_landmark_count(p) == w.m
        n1 = L.lapnys_workspace_size(p)
        assert n1 == L.lapnys_workspace_size(p)
        assert n1 % 256 == 0
        # at least the landmark-major C buffer
        assert n1 >= w.P * w.m * w.N * 4
    # monotone in the token count at fixed landmarks
    sizes = [L.lapnys_workspace_size(_p(grid_h=g, grid_w=g, pool=g // 8, dtype="f32")) for g in (16, 32, 64, 128)]
    assert sizes == sorted(sizes)


def test_binding_refuses_host_tensors():
    """Tensors on the host are refused by the binding before any call into the
    library: their addresses are not device memory."""
    import torch
    p = _p(B=1, H=1, dtype="f32")
    t = torch.zeros(196 * 64, dtype=torch.float32)
    with pytest.raises(ValueError, match="device tensors"):
        L.lapnys_forward_ws(t, t, t, t, p, None)
    with pytest.raises(ValueError, match="device tensors"):
        L.lapnys_forward(t, t, t, t, p)
    with pytest.raises(ValueError, match="device tensors"):
        L.lapnys_forward_debug(t, t, t, t, p, None, {})
    with pytest.raises(ValueError, match="device tensors"):
        L.lapnys_backward_ws(t, t, t, t, t, t, t, p, None)
    # the workspace too
    with pytest.raises(ValueError, match="device tensors"):
        L.lapnys_forward_ws(1 << 24, 2 << 24, 3 << 24, 4 << 24, p, torch.zeros(1024, dtype=torch.uint8))


def test_noalloc_checks_before_any_device_call():
    """lapnys_forward_noalloc refuses, before touching a device, a problem
    whose workspace exceeds the static scratch (LAPNYS_ERR_SCRATCH) and the
    forms that need a second stream (LAPNYS_ERR_UNSUPPORTED)."""
    lib = L.library()
    a = 1 << 24
    big = L.params_for(WORKLOADS["stage1_56x56_bf16"].with_(B=128))
    assert L.lapnys_workspace_size(big) > B.LAPNYS_SCRATCH_MAX_BYTES
    assert lib.lapnys_forward_noalloc(a, 2 * a, 3 * a, 4 * a, ctypes.byref(big), None) == B.LAPNYS_ERR_SCRATCH
    for kw in ({"ns_plain": True}, {"solver": "cg"}, {"kernel": "gaussian"}, {"grid_h": 18, "grid_w": 18}):
        p = L.params_for(WORKLOADS["tiny_f32"].with_(**kw))
        assert lib.lapnys_forward_noalloc(a, 2 * a, 3 * a, 4 * a, ctypes.byref(p), None) == B.LAPNYS_ERR_UNSUPPORTED
    assert L.lapnys_status_string(B.LAPNYS_ERR_SCRATCH).startswith("the problem's workspace exceeds")
