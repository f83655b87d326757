"""Build liblapnys_san.so: the same library with its host code (the C ABI:
validation, planning, the stage sequence) compiled with AddressSanitizer and
UndefinedBehaviorSanitizer.  Device code is compiled as usual.  The tests run
the ABI tests against it (tests/test_abi_sanitized.py) in a process that
preloads the sanitizer runtime (sanitizer_runtime()).

Usage: python -m laplacian_nystr_approximation_amd.build_sanitized [-v]
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import sys

from .build import ARCH, CSRC, DEVICE_FLAGS, INCLUDE, PKG, _hipcc, _run, _runtime_stub

BUILD_DIR = os.path.join(PKG, "_build_san")
LIB = os.path.join(PKG, "liblapnys_san.so")
# Each sanitizer flag applies to the host compilation only.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _clangxx(hipcc: str) -> str:
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc)))
    for cand in [os.path.join(rocm, "llvm", "bin", "clang++"), "/opt/rocm/llvm/bin/clang++"]:
        if os.path.exists(cand):
            return cand
    raise RuntimeError("clang++ of the ROCm toolchain not found")


def sanitizer_runtime() -> str | None:
    """The AddressSanitizer runtime of the ROCm clang, to preload into a
    process that loads liblapnys_san.so (None if not installed)."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.hpp"))
                  + [os.path.join(INCLUDE, "lapnys.h")])


def stale() -> bool:
    """True if the sanitized library is missing or older than a source."""
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(s) > t for s in sources())


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    stub_dir = _runtime_stub(verbose)
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
             "-Wall", "-Wno-unused-result"] + DEVICE_FLAGS + HOST_SANITIZE
    objs, jobs = [], []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = os.path.join(BUILD_DIR, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        jobs.append([hipcc] + flags + ["-c", src, "-o", obj])
    with cf.ThreadPoolExecutor(max(1, min(len(jobs), 16, os.cpu_count() or 1))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc))), "lib")
    tmp = LIB + ".tmp"
    # Host link only (the device code is already bundled in the objects).
    _run([_clangxx(hipcc), "-shared", "-fPIC", "-fsanitize=address", "-fsanitize=undefined", "-shared-libsan",
          "-L", stub_dir, "-Wl,--no-as-needed", f"-Wl,-rpath,{rocm_lib}", "-Wl,--enable-new-dtags", "-o", tmp]
         + objs + ["-lamdhip64"], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv[1:]))
