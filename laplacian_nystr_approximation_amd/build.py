"""Build liblapnys.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m laplacian_nystr_approximation_amd.build [-v]
Each csrc/*.hip file is compiled to an object in parallel, then linked into
laplacian_nystr_approximation_amd/liblapnys.so next to this file.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblapnys.so")
# Measurement tooling built beside the library: the VALU issue-rate probe
# (bench.py --valu-probe); not part of liblapnys.
PROBE_SRC = os.path.join(PKG, "probe", "valu_probe.hip")
PROBE_LIB = os.path.join(PKG, "libvaluprobe.so")
ARCH = "gfx950"

# Packed fp32 instructions are disabled for every device compile.  MFMA
# results are allocated in ordinary vector registers (gfx950 accepts either
# file): the solver's step loops otherwise copy every accumulator out of the
# accumulation registers before using it (48 copies per step).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-result"]


def _hipcc() -> str:
    for cand in [os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"]:
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines() if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def _runtime_stub(verbose) -> str:
    """An empty library whose soname is the unversioned ``libamdhip64.so``.

    Linking against it (HIP symbols stay undefined until load time) records a
    dependency on the name ``libamdhip64.so``.  A process that has already
    loaded a HIP runtime under that name (PyTorch-ROCm loads its bundled one
    that way) then reuses it instead of loading a second runtime; a process
    without one resolves it through the ROCm RUNPATH.
    """
    stub_dir = os.path.join(BUILD_DIR, "stub")
    os.makedirs(stub_dir, exist_ok=True)
    src = os.path.join(stub_dir, "empty.c")
    with open(src, "w") as f:
        f.write("/* link-time stand-in for the HIP runtime */\n")
    _run(["gcc", "-shared", "-fPIC", "-Wl,-soname,libamdhip64.so", "-o", os.path.join(stub_dir, "libamdhip64.so"),
          src], verbose)
    return stub_dir


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every csrc/*.hip for gfx950 and link liblapnys.so; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    stub_dir = _runtime_stub(verbose)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    flags = COMMON + DEVICE_FLAGS + list(extra_flags or [])
    objs = []
    jobs = []
    for src in srcs:
        obj = os.path.join(BUILD_DIR, os.path.basename(src)[:-4] + ".o")
        objs.append(obj)
        jobs.append([hipcc] + flags + ["-c", src, "-o", obj])
    workers = min(len(jobs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    tmp = LIB + ".tmp"
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc))), "lib")
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-L", stub_dir, "-Wl,--no-as-needed",
          f"-Wl,-rpath,{rocm_lib}", "-Wl,--enable-new-dtags", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    pobj = os.path.join(BUILD_DIR, "valu_probe.o")
    _run([hipcc] + flags + ["-c", PROBE_SRC, "-o", pobj], verbose)
    ptmp = PROBE_LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-L", stub_dir, "-Wl,--no-as-needed",
          f"-Wl,-rpath,{rocm_lib}", "-Wl,--enable-new-dtags", "-o", ptmp, pobj], verbose)
    os.replace(ptmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv[1:]))
