"""MI355X-native forward (and backward) pass of LaplacianFormer's Laplacian-kernel Nystrom attention.

The computation lives in the HIP library ``liblapnys.so`` (C ABI in
``include/lapnys.h``); ``laplacian_nystr_approximation_amd.lapnys`` is its
ctypes binding, whose names are re-exported here.  The library is loaded on
first use of any of them, and that use raises ImportError if it has not been
built (``python -m laplacian_nystr_approximation_amd.build``).
"""

import importlib

_BINDING_NAMES = {
    "HipEvents", "LapnysError", "lapnys_debug", "lapnys_params", "lapnys_forward", "lapnys_forward_ws",
    "lapnys_forward_debug", "lapnys_forward_profiled", "lapnys_landmark_count", "lapnys_workspace_size",
    "lapnys_release", "lapnys_status_string", "make_params", "params_for", "library", "LIB_PATH",
    "DEBUG_FIELDS", "STAGE_NAMES", "LAPNYS_NUM_STAGES", "lapnys_backward_ws", "lapnys_backward_workspace_size",
    "lapnys_forward_noalloc",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        return getattr(importlib.import_module(".lapnys", __name__), name)
    raise AttributeError(name)
