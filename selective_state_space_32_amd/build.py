"""Build libssmscan.so in-tree with hipcc for gfx950.

    python -m selective_state_space_32_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libssmscan.so")
SOURCES = ["ssmscan.hip"]   # includes every header in csrc/

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    # packed fp32 instructions stay disabled: every fp32 operation is a plain VALU op
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wall",
]


def build(verbose: bool = False) -> str:
    """Compile the HIP sources into libssmscan.so next to this file (always recompiles)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC, *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines()
                    if "packed-fp32-ops" not in l and "--hip-link" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


def build_sanitized(out: str = "") -> str:
    """The library with AddressSanitizer and UndefinedBehaviorSanitizer on its host code (the
    device code is built as usual, unsanitized), for the argument-validation tests on a machine
    without a GPU.  Returns the path (default _build/libssmscan_asan.so).  Run the tests with
    clang's ASan runtime preloaded:

        LD_PRELOAD=<clang_rt.asan runtime> ASAN_OPTIONS=detect_leaks=0 \
        SSMSCAN_LIBRARY=<that path> python -m pytest tests/test_abi.py
    """
    out = out or os.path.join(ROOT, "_build", "libssmscan_asan.so")
    os.makedirs(os.path.dirname(out), exist_ok=True)
    cmd = [HIPCC, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-fno-omit-frame-pointer", "-fvisibility=hidden", "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc (sanitized host build) failed:\n" + r.stderr)
    return out


def asan_runtime() -> str:
    """The clang ASan runtime matching hipcc's compiler (to LD_PRELOAD)."""
    r = subprocess.run([os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang"),
                        "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path):
        import glob
        hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        path = hits[0] if hits else ""
    return path


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "sanitized":
        print(build_sanitized())
        print(asan_runtime())
    else:
        print(build(verbose=True))
