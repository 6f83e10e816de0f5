"""Build and load ``liboracle.so`` (the C part of the oracle).

Test infrastructure only: see the package docstring.  The library is built
with plain ``gcc -O2`` (no fast-math, strict IEEE binary64) and shares no
source with the HIP library.
"""
import ctypes
import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` next to it; return the path."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
               "-fno-fast-math", "-ffp-contract=off", SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


class GemmArgs(ctypes.Structure):
    _fields_ = [
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("A", ctypes.c_void_p), ("a_type", ctypes.c_int32), ("a_order", ctypes.c_int32),
        ("lda", ctypes.c_int64),
        ("B", ctypes.c_void_p), ("b_type", ctypes.c_int32), ("b_order", ctypes.c_int32),
        ("ldb", ctypes.c_int64),
        ("C", ctypes.c_void_p), ("c_type", ctypes.c_int32), ("c_order", ctypes.c_int32),
        ("ldc", ctypes.c_int64),
        ("bias", ctypes.c_void_p), ("bias_type", ctypes.c_int32), ("act", ctypes.c_int32),
        ("alpha", ctypes.c_double), ("beta", ctypes.c_double),
        ("scale_a", ctypes.c_double), ("scale_b", ctypes.c_double),
    ]


class ConvArgs(ctypes.Structure):
    _fields_ = [
        ("N", ctypes.c_int64), ("H", ctypes.c_int64), ("W", ctypes.c_int64),
        ("C", ctypes.c_int64), ("K", ctypes.c_int64), ("R", ctypes.c_int64),
        ("S", ctypes.c_int64),
        ("u", ctypes.c_int32), ("v", ctypes.c_int32), ("ph", ctypes.c_int32),
        ("pw", ctypes.c_int32), ("dh", ctypes.c_int32), ("dw", ctypes.c_int32),
        ("x", ctypes.c_void_p), ("w", ctypes.c_void_p), ("Cres", ctypes.c_void_p),
        ("type", ctypes.c_int32),
        ("bias", ctypes.c_void_p), ("bias_type", ctypes.c_int32), ("act", ctypes.c_int32),
        ("alpha", ctypes.c_double), ("beta", ctypes.c_double),
    ]


def lib() -> ctypes.CDLL:
    """Load the oracle library, building it first if it is missing or stale."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build(force=True)
        L = ctypes.CDLL(LIB)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        L.oracle_decode.argtypes = [I32, P, I64, P]
        L.oracle_decode.restype = I32
        L.oracle_gemm.argtypes = [ctypes.POINTER(GemmArgs), P, I32]
        L.oracle_gemm.restype = I32
        L.oracle_gemm_points.argtypes = [ctypes.POINTER(GemmArgs), P, P, I64, P, I32]
        L.oracle_gemm_points.restype = I32
        L.oracle_transpose.argtypes = [P, I64, P, I64, I64, I64, I32]
        L.oracle_transpose.restype = I32
        L.oracle_copy2d.argtypes = [P, I64, P, I64, I64, I64, I32]
        L.oracle_copy2d.restype = I32
        L.oracle_conv2d.argtypes = [ctypes.POINTER(ConvArgs), P, I32]
        L.oracle_conv2d.restype = I32
        L.oracle_conv2d_points.argtypes = [ctypes.POINTER(ConvArgs), P, P, I64, P, I32]
        L.oracle_conv2d_points.restype = I32
        L.oracle_version.restype = I32
        _lib = L
    return _lib
