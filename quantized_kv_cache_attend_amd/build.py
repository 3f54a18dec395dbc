"""Build ``libkvq.so`` (all HIP sources under ``csrc/``) for gfx950 with hipcc.

Run ``python quantized_kv_cache_attend_amd/build.py`` (by path: importing the package
loads the library) or call :func:`build`.
Every call compiles from scratch into ``_build/`` at the repository root and
then replaces ``quantized_kv_cache_attend_amd/libkvq.so``.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvq.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -fhip-fp32-correctly-rounded-divide-sqrt: IEEE float32 division (the
#   quantizer's scale and quotient must be bit-exact).
# -packed-fp32-ops: no packed FP32 VALU instructions.
# No -ffast-math and no denormal flush: the quantizer keeps subnormals.
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mcode-object-version=5",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


# Extra flags per source.  The matrix-core attend kernels assume finite
# inputs (non-finite inputs are outside the library's contract), so maxima
# need no NaN-quieting canonicalization: -fno-honor-nans.  Infinities stay
# honoured (masked scores are -inf).
EXTRA_CFLAGS = {
    "kvq_attend_mfma.hip": ["-fno-honor-nans"],
    "kvq_attend_mfma32.hip": ["-fno-honor-nans"],
    "kvq_attend_stream.hip": ["-fno-honor-nans"],
}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


LIB_PHASE = os.path.join(PKG, "libkvq_phase.so")
BUILD_PHASE = os.path.join(ROOT, "_build_phase")
# Host AddressSanitizer build of the same sources (device code unchanged):
# the C-ABI layer's argument checks, sizing and error strings run under ASan
# in a CPU test (the GPU code itself is never built with a sanitizer).
BUILD_ASAN = os.path.join(ROOT, "_build_asan")
LIB_ASAN = os.path.join(BUILD_ASAN, "libkvq_asan.so")
ASAN_CFLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *extra, *EXTRA_CFLAGS.get(os.path.basename(src), []), "-c", src, "-o",
           obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, phase_trace: bool = False, asan: bool = False) -> str:
    """Compile every source and link the library.  phase_trace: the
    diagnostic build with per-wave phase timestamps in the matrix-core attend
    kernels (-DKVQ_PHASE_TRACE), written to libkvq_phase.so; asan: host code
    built with AddressSanitizer into _build_asan/libkvq_asan.so (loaded only
    with the ASan runtime preloaded).  The package loads libkvq.so."""
    if asan:
        build_dir, lib, extra = BUILD_ASAN, LIB_ASAN, tuple(ASAN_CFLAGS)
    elif phase_trace:
        build_dir, lib, extra = BUILD_PHASE, LIB_PHASE, ("-DKVQ_PHASE_TRACE",)
    else:
        build_dir, lib, extra = BUILD, LIB, ()
    if os.path.isdir(build_dir):
        shutil.rmtree(build_dir)
    os.makedirs(build_dir)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, extra), srcs))
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-mcode-object-version=5", "-shared", "-fPIC", *objs,
           "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} from {len(srcs)} sources")
    return lib


if __name__ == "__main__":
    build(verbose=True, phase_trace="--phase-trace" in sys.argv[1:], asan="--asan" in sys.argv[1:])
    sys.exit(0)
