"""Build libtla.so in-tree with hipcc for gfx950.

    python -m tiled_layout_algebra_amd.build [--changed]

Every source under csrc/ is compiled to an object in _build/ (in parallel),
then linked into tiled_layout_algebra_amd/libtla.so.  Recompiles everything
unless --changed is given (then only sources newer than their object, or
all of them when a header changed).
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libtla.so")
SOURCES = ["api.cpp", "algebra.cpp", "gemm.hip", "gemm_general.hip", "gemm_pingpong.hip",
           "conv_slab.hip", "transpose.hip", "layout_eval.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++20", "-fPIC",
    # packed fp32 instructions stay off for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, err))
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def _stale(src: str) -> bool:
    """True if src's object is missing or older than src or any header."""
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    if not os.path.exists(obj):
        return True
    t = os.path.getmtime(obj)
    deps = [os.path.join(CSRC, src), os.path.join(ROOT, "include", "tla.h")]
    for d, _, files in os.walk(CSRC):
        deps += [os.path.join(d, f) for f in files if f.endswith((".hpp", ".h"))]
    return any(os.path.getmtime(f) > t for f in deps)


def build(verbose: bool = True, only_changed: bool = False) -> str:
    """Compile every source (or, with only_changed, those whose object is
    older than the source or any header) and link libtla.so."""
    os.makedirs(BUILD, exist_ok=True)
    todo = [s for s in SOURCES if not only_changed or _stale(s)]
    with ThreadPoolExecutor(max_workers=max(len(todo), 1)) as ex:
        list(ex.map(_compile, todo))
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(only_changed="--changed" in sys.argv[1:])
