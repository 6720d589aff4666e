"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU needed).

The library is linked again with its host sources (argument checks, workspace sizing, launch
set-up) built sanitized and the kernels' objects unchanged; the host-side ABI tests then run
against it in a child process with the shared ASan runtime preloaded.  Any sanitizer report
fails the run."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def test_abi_host_code_sanitized(tmp_path):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no shared ASan runtime in this toolchain")
    from gated_deltanet_hybrid_amd import build
    objs = [os.path.join(build.BUILD, os.path.splitext(s)[0] + ".o") for s in build.SOURCES
            if s not in build.HOST_SOURCES]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("the library's objects are not built")
    lib = build.build_host_sanitized(str(tmp_path / "libhla_san.so"))
    env = dict(os.environ, HLA_LIBRARY=lib, LD_PRELOAD=rt, PYTHONPATH=ROOT,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the child loads the sanitized build
    probe = subprocess.run([sys.executable, "-c", "from gated_deltanet_hybrid_amd import hla; print(hla.library()._name)"],
                           env=env, capture_output=True, text=True, timeout=300, cwd=str(tmp_path))
    assert probe.returncode == 0 and probe.stdout.strip() == lib, probe.stdout + probe.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-q",
                        "-p", "no:cacheprovider"], env=env, capture_output=True, text=True, timeout=600,
                       cwd=str(tmp_path))
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
