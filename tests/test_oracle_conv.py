"""Pins of the direct-convolution oracle against things other than itself:
scipy's 2-D cross-correlation (single channel; padding as explicit zero
padding, stride as subsampling, dilation as a zero-dilated filter), sums of
per-channel correlations for many channels and filters, the 1x1 convolution
as the (separately pinned) oracle GEMM, the epilogue applied by hand, and
the points mode against the full output."""
import numpy as np
import pytest
from scipy.signal import correlate2d

from oracle import conv as oc
from oracle import gemm as og


def _ints(rng, shape):
    return rng.integers(-3, 4, shape).astype(np.float16)


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint16)


def _dilate(f, dh, dw):
    R, S = f.shape
    out = np.zeros(((R - 1) * dh + 1, (S - 1) * dw + 1))
    out[::dh, ::dw] = f
    return out


@pytest.mark.parametrize("H,W,R,S,stride,pad,dil", [
    (7, 9, 3, 2, (1, 1), (0, 0), (1, 1)),
    (8, 8, 3, 3, (1, 1), (1, 1), (1, 1)),
    (11, 10, 3, 3, (2, 3), (1, 2), (1, 1)),
    (12, 13, 3, 2, (1, 2), (2, 0), (2, 3)),
    (5, 5, 5, 5, (1, 1), (2, 2), (1, 1)),
])
def test_single_channel_is_scipy_correlation(H, W, R, S, stride, pad, dil):
    rng = np.random.default_rng(H * 100 + W)
    x, w = _ints(rng, (H, W)), _ints(rng, (R, S))
    ref = oc.conv2d(_bits(x), _bits(w), 1, H, W, 1, 1, R, S, stride, pad, dil)
    xp = np.pad(x.astype(float), ((pad[0], pad[0]), (pad[1], pad[1])))
    full = correlate2d(xp, _dilate(w.astype(float), *dil), mode="valid")
    want = full[::stride[0], ::stride[1]]
    P, Q = oc.out_size(H, R, stride[0], pad[0], dil[0]), oc.out_size(W, S, stride[1], pad[1], dil[1])
    assert want.shape == (P, Q)
    assert np.array_equal(ref.reshape(P, Q), want)


def test_channels_and_filters_sum_per_channel_correlations():
    rng = np.random.default_rng(4)
    N, H, W, C, K, R, S = 2, 6, 7, 3, 4, 3, 2
    x, w = _ints(rng, (N, H, W, C)), _ints(rng, (K, R, S, C))
    ref = oc.conv2d(_bits(x), _bits(w), N, H, W, C, K, R, S, pad=(1, 1))
    P, Q = oc.out_size(H, R, 1, 1, 1), oc.out_size(W, S, 1, 1, 1)
    want = np.zeros((N, P, Q, K))
    for n in range(N):
        for k in range(K):
            for c in range(C):
                xp = np.pad(x[n, :, :, c].astype(float), 1)
                want[n, :, :, k] += correlate2d(xp, w[k, :, :, c].astype(float), mode="valid")
    assert np.array_equal(ref.reshape(N, P, Q, K), want)


def test_one_by_one_is_the_gemm():
    rng = np.random.default_rng(5)
    N, H, W, C, K = 2, 5, 6, 16, 12
    x, w = _ints(rng, (N, H, W, C)), _ints(rng, (K, 1, 1, C))
    ref = oc.conv2d(_bits(x), _bits(w), N, H, W, C, K, 1, 1)
    # A = x as (N*H*W) x C row-major; B = w as C x K, i.e. column-major with ld C
    g = og.gemm(N * H * W, K, C, _bits(x), og.F16, og.ROW, C, _bits(w), og.F16, og.COL, C)
    assert np.array_equal(ref, g)


def test_epilogue_by_hand():
    rng = np.random.default_rng(6)
    N, H, W, C, K, R, S = 1, 6, 6, 4, 5, 3, 3
    x, w = _ints(rng, (N, H, W, C)), _ints(rng, (K, R, S, C))
    P = Q = oc.out_size(6, 3, 1, 0, 1)
    cres = _ints(rng, (N * P * Q, K))
    bias = (rng.integers(-8, 9, K) / 8).astype(np.float16)
    raw = oc.conv2d(_bits(x), _bits(w), N, H, W, C, K, R, S)
    for act in (og.ACT_NONE, og.ACT_RELU):
        got = oc.conv2d(_bits(x), _bits(w), N, H, W, C, K, R, S, Cres=_bits(cres),
                        bias=_bits(bias), bias_type=og.F16, alpha=1.5, beta=0.5, act=act)
        y = 1.5 * raw + 0.5 * cres.astype(float) + bias.astype(float)[None, :]
        if act == og.ACT_RELU:
            y = np.maximum(y, 0)
        assert np.array_equal(got, y)


def test_points_match_full():
    rng = np.random.default_rng(7)
    N, H, W, C, K, R, S = 2, 9, 8, 6, 7, 3, 3
    x, w = _ints(rng, (N, H, W, C)), _ints(rng, (K, R, S, C))
    full = oc.conv2d(_bits(x), _bits(w), N, H, W, C, K, R, S, (2, 1), (1, 1), (1, 2))
    ms = rng.integers(0, full.shape[0], 200)
    ks = rng.integers(0, K, 200)
    pts = oc.conv2d_points(ms, ks, _bits(x), _bits(w), N, H, W, C, K, R, S, (2, 1), (1, 1), (1, 2))
    assert np.array_equal(pts, full[ms, ks])
