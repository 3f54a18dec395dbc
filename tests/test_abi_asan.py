"""The C-ABI host layer under AddressSanitizer.

The library's host code (argument checks, sizing and layout arithmetic,
workspace layout, error strings) is built with ASan (the device code as
usual) and the CPU ABI tests run against that build in a child process with
the ASan runtime preloaded.  Nothing here touches a GPU: every call the ABI
tests make is rejected or answered on the host.
"""
import glob
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "kvq_build", os.path.join(ROOT, "quantized_kv_cache_attend_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    return b


@pytest.mark.skipif(_asan_runtime() is None or not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc or the clang ASan runtime is not installed")
def test_abi_tests_pass_under_asan():
    lib = _build_module().build(asan=True)
    dyn = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in dyn, "the host code of the ASan build is not instrumented"
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), KVQ_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:exitcode=99")
    which = subprocess.run(
        [sys.executable, "-c", "import quantized_kv_cache_attend_amd as k; print(k.LIB_PATH)"],
        env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert which.returncode == 0, which.stderr[-2000:]
    assert which.stdout.strip() == lib
    run = subprocess.run(
        [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-q",
         "-p", "no:cacheprovider", "-m", "not gpu"],
        env=env, capture_output=True, text=True, timeout=900, cwd=ROOT)
    out = run.stdout + run.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert run.returncode == 0, out[-4000:]
    assert " passed" in run.stdout and " failed" not in run.stdout
