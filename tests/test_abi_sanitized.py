"""The C-ABI tests (tests/test_abi.py) against a build of the library whose
host code runs under AddressSanitizer and UndefinedBehaviorSanitizer
(laplacian_nystr_approximation_amd/build_sanitized.py), in a child process
that preloads the sanitizer runtime.  Any report aborts that process, so the
run passes only if every validation path, the planning arithmetic and the
binding's calls stay free of memory errors and undefined behaviour.  No GPU
is needed: the ABI tests stop before any device call."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _env():
    # Imported here: the build script is host tooling that GPU runs do not carry.
    BS = pytest.importorskip("laplacian_nystr_approximation_amd.build_sanitized")
    rt = BS.sanitizer_runtime()
    if rt is None:
        pytest.skip("the ROCm clang AddressSanitizer runtime is not installed")
    if BS.stale():
        try:
            BS.build()
        except RuntimeError as e:  # no toolchain here
            pytest.skip(f"cannot build the sanitized library: {e}")
    env = dict(os.environ)
    env.update({"LD_PRELOAD": rt, "LAPNYS_LIBRARY": BS.LIB,
                "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    return env


def test_sanitized_library_is_the_one_loaded():
    env = _env()
    code = ("import laplacian_nystr_approximation_amd.lapnys as L; L.library(); "
            "maps = open('/proc/self/maps').read(); "
            "print(L.LIB_PATH.endswith('liblapnys_san.so'), 'liblapnys_san.so' in maps, "
            "'libclang_rt.asan' in maps)")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.split() == ["True", "True", "True"], r.stdout


def test_abi_under_sanitizers():
    env = _env()
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:] + r.stderr[-3000:])
    assert "passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]
