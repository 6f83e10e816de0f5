"""Direct convolution -- the oracle for the implicit-GEMM convolution.

Test infrastructure only (see the package docstring).  A thin ctypes layer
over oracle.c's binary64 loops (oracle_conv2d, oracle_conv2d_points).

Definition followed: the PitchLinearStripminedThreadMap walk-through
(lpnh.cn/news/2469163), section 5.2 -- convolution runs as an implicit GEMM
whose one dimension is the output pixel and whose other is the filter
position times the channel.  Reading (the page states no formula): forward
cross-correlation, input x N x H x W x C (NHWC), filter w K x R x S x C
(KRSC), output N x P x Q x K (NPQK),

    s[n,p,q,k] = sum_{r<R, s<S, c<C} x[n, p*u - ph + r*dh, q*v - pw + s*dw, c]
                                     * w[k, r, s, c]

with x = 0 outside the image, followed by the GEMM epilogue at GEMM position
(m = (n*P + p)*Q + q, k): alpha, beta*C[n,p,q,k], bias[k], activation.
"""
import ctypes

import numpy as np

from ._native import ConvArgs, lib
from .gemm import _STORAGE, _ptr, host_threads, ACT_NONE, F16


def out_size(extent, f, stride, pad, dil):
    """Output extent along one axis: floor((extent + 2 pad - dil (f-1) - 1) / stride) + 1."""
    span = extent + 2 * pad - dil * (f - 1) - 1
    return 0 if span < 0 else span // stride + 1


def _args(x, w, N, H, W, C, K, R, S, stride, pad, dil, dtype, Cres, bias, bias_type,
          alpha, beta, act):
    keep = []

    def flat(a, t):
        if a is None:
            return None
        a = np.ascontiguousarray(a, dtype=_STORAGE[t]).reshape(-1)
        keep.append(a)
        return a

    x, w, Cres, bias = flat(x, dtype), flat(w, dtype), flat(Cres, dtype), flat(bias, bias_type)
    args = ConvArgs(N, H, W, C, K, R, S, stride[0], stride[1], pad[0], pad[1], dil[0], dil[1],
                    _ptr(x), _ptr(w), _ptr(Cres), dtype, _ptr(bias), bias_type, act,
                    float(np.float32(alpha)), float(np.float32(beta)))
    return args, keep


def conv2d(x, w, N, H, W, C, K, R, S, stride=(1, 1), pad=(0, 0), dil=(1, 1), dtype=F16,
           Cres=None, bias=None, bias_type=F16, alpha=1.0, beta=0.0, act=ACT_NONE,
           nthreads=None) -> np.ndarray:
    """ref[N*P*Q, K] (float64): the epilogue applied to the convolution sums."""
    P, Q = out_size(H, R, stride[0], pad[0], dil[0]), out_size(W, S, stride[1], pad[1], dil[1])
    args, keep = _args(x, w, N, H, W, C, K, R, S, stride, pad, dil, dtype, Cres, bias,
                       bias_type, alpha, beta, act)
    ref = np.empty((N * P * Q, K), dtype=np.float64)
    rc = lib().oracle_conv2d(ctypes.byref(args), _ptr(ref), nthreads or host_threads())
    if rc:
        raise ValueError("oracle_conv2d failed (%d)" % rc)
    return ref


def conv2d_points(ms, ks, x, w, N, H, W, C, K, R, S, stride=(1, 1), pad=(0, 0), dil=(1, 1),
                  dtype=F16, Cres=None, bias=None, bias_type=F16, alpha=1.0, beta=0.0,
                  act=ACT_NONE, nthreads=None) -> np.ndarray:
    """The output at GEMM positions (ms[i], ks[i])."""
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ks = np.ascontiguousarray(ks, dtype=np.int64)
    args, keep = _args(x, w, N, H, W, C, K, R, S, stride, pad, dil, dtype, Cres, bias,
                       bias_type, alpha, beta, act)
    out = np.empty(ms.size, dtype=np.float64)
    rc = lib().oracle_conv2d_points(ctypes.byref(args), _ptr(ms), _ptr(ks), ms.size, _ptr(out),
                                    nthreads or host_threads())
    if rc:
        raise ValueError("oracle_conv2d_points failed (%d)" % rc)
    return out
