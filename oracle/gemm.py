"""ctypes front-end of the C oracle (``oracle.c``): decoders, binary64 GEMM
with the scalar epilogue, sampled GEMM outputs, bit-copy transpose and
pitched 2-D copy.

Test infrastructure only (see the package docstring).  Operands are host
numpy arrays holding the raw storage bits (uint16 for fp16/bf16, uint8 for
e4m3, uint32 for fp32); the oracle decodes them itself.

Storage type codes: 0 fp16, 1 bf16, 2 OCP e4m3fn, 3 fp32.
Orders: 0 row-major, 1 column-major.  Activations: 0 none, 1 ReLU, 2 GELU.
"""
import ctypes
import os

import numpy as np

from ._native import GemmArgs, lib

F16, BF16, E4M3, F32 = 0, 1, 2, 3
ROW, COL = 0, 1
ACT_NONE, ACT_RELU, ACT_GELU = 0, 1, 2

_STORAGE = {F16: np.uint16, BF16: np.uint16, E4M3: np.uint8, F32: np.uint32}


def host_threads() -> int:
    """Host cores this process may use (the oracle's thread count)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def decode(dtype: int, bits: np.ndarray) -> np.ndarray:
    """Decode raw storage bits of ``dtype`` into float64 (same shape)."""
    bits = np.ascontiguousarray(bits, dtype=_STORAGE[dtype])
    out = np.empty(bits.shape, dtype=np.float64)
    rc = lib().oracle_decode(dtype, _ptr(bits), bits.size, _ptr(out))
    if rc:
        raise ValueError("oracle_decode failed (%d)" % rc)
    return out


def _args(M, N, K, A, a_type, a_order, lda, B, b_type, b_order, ldb,
          C, c_type, c_order, ldc, bias, bias_type, alpha, beta, scale_a,
          scale_b, act):
    keep = []

    def flat(x, t):
        if x is None:
            return None
        x = np.ascontiguousarray(x, dtype=_STORAGE[t]).reshape(-1)
        keep.append(x)
        return x

    A, B, C, bias = flat(A, a_type), flat(B, b_type), flat(C, c_type), flat(bias, bias_type)
    args = GemmArgs(M, N, K, _ptr(A), a_type, a_order, lda, _ptr(B), b_type, b_order, ldb,
                    _ptr(C), c_type, c_order, ldc, _ptr(bias), bias_type, act,
                    float(np.float32(alpha)), float(np.float32(beta)),
                    float(np.float32(scale_a)), float(np.float32(scale_b)))
    return args, keep


def gemm(M, N, K, A, a_type, a_order, lda, B, b_type, b_order, ldb,
         C=None, c_type=F16, c_order=ROW, ldc=0, bias=None, bias_type=F16,
         alpha=1.0, beta=0.0, scale_a=1.0, scale_b=1.0, act=ACT_NONE,
         nthreads=None) -> np.ndarray:
    """ref[M,N] (float64, row-major) = act(alpha*sa*sb*A.B + beta*C + bias).

    alpha, beta and the scales are first rounded to float32, the precision in
    which a caller hands them over; the rest is exact binary64 arithmetic.
    """
    args, keep = _args(M, N, K, A, a_type, a_order, lda, B, b_type, b_order, ldb,
                       C, c_type, c_order, ldc, bias, bias_type, alpha, beta,
                       scale_a, scale_b, act)
    ref = np.empty((M, N), dtype=np.float64)
    rc = lib().oracle_gemm(ctypes.byref(args), _ptr(ref), nthreads or host_threads())
    if rc:
        raise ValueError("oracle_gemm failed (%d)" % rc)
    return ref


def gemm_points(ms, ns, M, N, K, A, a_type, a_order, lda, B, b_type, b_order, ldb,
                C=None, c_type=F16, c_order=ROW, ldc=0, bias=None, bias_type=F16,
                alpha=1.0, beta=0.0, scale_a=1.0, scale_b=1.0, act=ACT_NONE,
                nthreads=None) -> np.ndarray:
    """ref(ms[i], ns[i]) for the listed output coordinates only."""
    args, keep = _args(M, N, K, A, a_type, a_order, lda, B, b_type, b_order, ldb,
                       C, c_type, c_order, ldc, bias, bias_type, alpha, beta,
                       scale_a, scale_b, act)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    out = np.empty(ms.shape, dtype=np.float64)
    rc = lib().oracle_gemm_points(ctypes.byref(args), _ptr(ms), _ptr(ns), ms.size,
                                  _ptr(out), nthreads or host_threads())
    if rc:
        raise ValueError("oracle_gemm_points failed (%d)" % rc)
    return out


def transpose(src: np.ndarray, M: int, N: int, ld_src: int, ld_dst: int,
              dst: np.ndarray = None) -> np.ndarray:
    """dst[m + n*ld_dst] = src[m*ld_src + n], raw bits (any itemsize)."""
    src = np.ascontiguousarray(src).reshape(-1)
    eb = src.dtype.itemsize
    if dst is None:
        dst = np.zeros(max(ld_dst * N, 0), dtype=src.dtype)
    rc = lib().oracle_transpose(_ptr(src), ld_src, _ptr(dst), ld_dst, M, N, eb)
    if rc:
        raise ValueError("oracle_transpose failed (%d)" % rc)
    return dst


def copy2d(src: np.ndarray, M: int, N: int, ld_src: int, ld_dst: int,
           dst: np.ndarray = None) -> np.ndarray:
    """dst[m*ld_dst + n] = src[m*ld_src + n], raw bits (any itemsize)."""
    src = np.ascontiguousarray(src).reshape(-1)
    eb = src.dtype.itemsize
    if dst is None:
        dst = np.zeros(max(ld_dst * M, 0), dtype=src.dtype)
    rc = lib().oracle_copy2d(_ptr(src), ld_src, _ptr(dst), ld_dst, M, N, eb)
    if rc:
        raise ValueError("oracle_copy2d failed (%d)" % rc)
    return dst


def within_tolerance(D: np.ndarray, ref: np.ndarray, tol: float):
    """Elementwise bound |D - ref| <= tol*(1 + |ref|); any NaN fails.

    Returns (ok, worst_ratio) where worst_ratio = max |D-ref| / (1+|ref|).
    """
    D = np.asarray(D, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if D.shape != ref.shape:
        return False, float("inf")
    if D.size == 0:
        return True, 0.0
    if np.isnan(D).any() or np.isnan(ref).any():
        return False, float("nan")
    ratio = np.abs(D - ref) / (1.0 + np.abs(ref))
    worst = float(ratio.max())
    return bool(worst <= tol), worst
