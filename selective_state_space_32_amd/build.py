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
def sources():
    """The library's translation units: the C ABI (ssmscan.hip) and the instantiations of the
    launch templates (inst_*.hip), compiled separately and in parallel."""
    return sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))


HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    # packed fp32 instructions stay disabled: every fp32 operation is a plain VALU op
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wall",
]


def _quiet(stderr: str) -> str:
    return "\n".join(l for l in (stderr or "").splitlines() if "packed-fp32-ops" not in l and "--hip-link" not in l)


def _compile_all(flags, objdir: str, out: str, verbose: bool, jobs: int = 0) -> str:
    os.makedirs(objdir, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(objdir, os.path.splitext(f)[0] + ".o") for f in srcs]

    def one(src_obj):
        src, obj = src_obj
        cmd = [HIPCC, *flags, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        return src, r.returncode, _quiet(r.stderr)

    from concurrent.futures import ThreadPoolExecutor
    jobs = jobs or max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", "0") or 0) or (os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for src, rc, err in ex.map(one, zip(srcs, objs)):
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n{err}")
            if verbose and err.strip():
                print(err, file=sys.stderr)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *flags, "-shared", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc link failed:\n" + _quiet(r.stderr))
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile the HIP sources into libssmscan.so next to this file (always recompiles)."""
    return _compile_all(FLAGS, os.path.join(ROOT, "_build", "obj"), LIB, verbose)


def build_sanitized(out: str = "") -> str:
    """The library with AddressSanitizer and UndefinedBehaviorSanitizer on its host code (the
    device code is built as usual, unsanitized), for the argument-validation tests on a machine
    without a GPU.  Returns the path (default _build/libssmscan_asan.so).  Run the tests with
    clang's ASan runtime preloaded:

        LD_PRELOAD=<clang_rt.asan runtime> ASAN_OPTIONS=detect_leaks=0 \
        SSMSCAN_LIBRARY=<that path> python -m pytest tests/test_abi.py
    """
    out = out or os.path.join(ROOT, "_build", "libssmscan_asan.so")
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                                                 "-fsanitize=undefined", "-fno-omit-frame-pointer"]
    return _compile_all(flags, os.path.join(ROOT, "_build", "obj_asan"), out, verbose=False)


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
