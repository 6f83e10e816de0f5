"""Implicit-GEMM convolution parity: tla_conv2d_fprop through the C ABI
against the direct-convolution oracle on the same seeded inputs.

* integer-valued inputs: every partial sum is exact in fp32, so y must be
  the oracle's exact result rounded to y's type, bit for bit -- over stride,
  padding and dilation, channel counts that do and do not fill a 16-byte
  vector or a whole 128-byte k-tile (the direct-to-LDS path, whose padding
  taps read zeros from the buffer range check; 256 x 64 tiles up to 64
  output channels, 128 x 128 above), 1x1 and 5x5 filters, ragged
  output-channel and pixel counts, whole tiles through the LDS epilogue;
* 64 -> 64 channels at stride 1 (the slab kernel: the whole filter and the
  image rows of a band of output rows in LDS) over padding, dilation,
  R != S, 1x1, 16 taps, bands of several rows with a last band of fewer,
  and the shapes that fall back to the implicit GEMM (5x5: the filter does
  not fit beside a slab; rows wider than 512 pixels);
* every kernel forced through tla_conv2d_fprop_variant on a subset, bit for
  bit where it applies and refused where it does not;
* random inputs with GELU within the tolerance, C aliasing y;
* the measured layer (32 x 56 x 56 x 64, 3x3) compared in full, and the
  32 x 28 x 28 x 256 layer on sampled outputs.
Tolerance: |y - ref| <= tol*(1 + |ref|), tol 1e-2.
"""
import numpy as np
import pytest
import torch

import tiled_layout_algebra_amd as tla
import workloads as W
from oracle import conv as oc
from oracle import gemm as og
from tests.gpu_util import to_dev, to_host

pytestmark = pytest.mark.gpu


def _oracle(case, inp):
    return oc.conv2d(inp["x"], inp["w"], case.N, case.H, case.W, case.C, case.K, case.R,
                     case.S, case.stride, case.pad, case.dil, case.dtype, Cres=inp["C"],
                     bias=inp["bias"], bias_type=case.dtype, alpha=case.alpha, beta=case.beta,
                     act=case.act)


def _run(case, inp, alias=False, variant=None):
    P, Q = case.out_hw()
    x, w = to_dev(inp["x"]), to_dev(inp["w"])
    c = to_dev(inp["C"]) if inp["C"] is not None else None
    b = to_dev(inp["bias"]) if inp["bias"] is not None else None
    y = c if alias else torch.full((case.N * P * Q * case.K,), 0x5A5A, dtype=torch.int16,
                                  device="cuda")
    tla.conv2d_fprop(x, w, y, case.N, case.H, case.W, case.C, case.K, case.R, case.S,
                     case.dtype, case.stride, case.pad, case.dil, C_res=c, bias=b,
                     bias_type=case.dtype, alpha=case.alpha, beta=case.beta, act=case.act,
                     variant=variant)
    torch.cuda.synchronize()
    return to_host(y, np.dtype(np.uint16)).reshape(case.N * P * Q, case.K)


GEOMETRIES = [  # N, H, W, C, K, R, S, stride, pad, dil
    (2, 9, 11, 16, 24, 3, 3, (1, 1), (1, 1), (1, 1)),
    (1, 10, 7, 3, 5, 3, 2, (2, 1), (1, 0), (1, 2)),
    (3, 8, 8, 8, 130, 1, 1, (1, 1), (0, 0), (1, 1)),
    (1, 17, 13, 24, 40, 5, 5, (2, 2), (2, 2), (1, 1)),
    (2, 12, 12, 32, 64, 3, 3, (1, 1), (2, 2), (2, 2)),
    (1, 6, 20, 40, 7, 2, 4, (3, 2), (0, 1), (1, 1)),
    # channel counts that are multiples of 64 take the direct-to-LDS path
    (2, 9, 11, 64, 24, 3, 3, (1, 1), (1, 1), (1, 1)),
    (1, 10, 7, 128, 72, 3, 2, (2, 1), (1, 0), (1, 2)),
    (3, 6, 6, 64, 130, 1, 1, (1, 1), (0, 0), (1, 1)),
    (1, 17, 13, 64, 40, 5, 5, (2, 2), (2, 2), (1, 1)),
    (2, 5, 7, 192, 33, 3, 3, (1, 2), (3, 3), (2, 1)),
    # 64 output channels: whole 256 x 64 tiles (and a ragged last one);
    # 128 output channels: whole 128 x 128 tiles -- the LDS epilogue with C
    (4, 16, 16, 64, 64, 3, 3, (1, 1), (1, 1), (1, 1)),
    (3, 9, 10, 64, 64, 3, 3, (1, 1), (1, 1), (1, 1)),
    (2, 8, 16, 128, 128, 3, 3, (1, 1), (1, 1), (1, 1)),
    # 64 -> 64 channels at stride 1 (the measured layer's channel counts):
    # no padding, dilation 2, R != S, 1x1, 5x5, wide and very wide rows;
    # 128 input channels with whole 256 x 64 tiles
    (2, 13, 7, 64, 64, 3, 3, (1, 1), (0, 0), (1, 1)),
    (1, 11, 12, 64, 64, 3, 3, (1, 1), (2, 2), (2, 2)),
    (3, 30, 17, 64, 64, 3, 1, (1, 1), (1, 0), (1, 1)),
    (1, 6, 40, 64, 64, 1, 1, (1, 1), (0, 0), (1, 1)),
    (1, 8, 200, 64, 64, 3, 3, (1, 1), (1, 1), (1, 1)),
    (1, 12, 12, 64, 64, 5, 5, (1, 1), (2, 2), (1, 1)),
    (1, 3, 600, 64, 64, 3, 3, (1, 1), (1, 1), (1, 1)),
    (4, 16, 16, 128, 64, 3, 3, (1, 1), (1, 1), (1, 1)),
    # slab bands of two (three) output rows with a last band of one (two);
    # 3x5 and 4x4 filters (16 taps: 128 KiB of filter beside the slab)
    (10, 27, 27, 64, 64, 3, 3, (1, 1), (1, 1), (1, 1)),
    (40, 14, 14, 64, 64, 3, 3, (1, 1), (1, 1), (1, 1)),
    # more than 256 bands of one row: bands of several rows, the last shorter
    (24, 48, 48, 64, 64, 3, 3, (1, 1), (1, 1), (1, 1)),
    (2, 7, 9, 64, 64, 3, 5, (1, 1), (1, 2), (1, 1)),
    (1, 6, 9, 64, 64, 4, 4, (1, 1), (3, 3), (2, 1)),
    # coordinates near 2^20 (padding, stride and dilation): taps on both sides
    # of the image, tap byte offsets that pass 2^32 on the direct-to-LDS path
    (2, 5, 32, 64, 24, 3, 1, (2**20 + 3, 1), (2**20, 0), (2**19, 1)),
    (2, 5, 32, 16, 24, 3, 1, (2**20 + 3, 1), (2**20, 0), (2**19, 1)),
]


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
@pytest.mark.parametrize("geom", GEOMETRIES)
def test_integer_inputs_bit_exact(geom, dtype):
    N, H, Wd, C, K, R, S, st, pd, dl = geom
    case = W.ConvCase(name="exact", N=N, H=H, W=Wd, C=C, K=K, R=R, S=S, stride=st, pad=pd,
                      dil=dl, dtype=dtype, alpha=1.5, beta=0.5, act=W.ACT_RELU, has_c=True,
                      has_bias=True, seed=N * 1000 + H * 10 + C, dist="int3", dist_bias="eighths")
    inp = W.conv_inputs(case)
    got = _run(case, inp)
    want = W.encode(_oracle(case, inp), dtype).reshape(got.shape)
    bad = np.argwhere(got != want)
    assert bad.size == 0, "%s: %d mismatches, first at %s" % (geom, len(bad), bad[0])


FORCED = [  # N, H, W, C, K, R, S, stride, pad, dil
    (4, 16, 16, 64, 64, 3, 3, (1, 1), (1, 1), (1, 1)),
    (10, 27, 27, 64, 64, 3, 3, (1, 1), (1, 1), (1, 1)),
    (1, 11, 12, 64, 64, 3, 3, (1, 1), (2, 2), (2, 2)),
    (2, 7, 9, 64, 64, 3, 5, (1, 1), (1, 2), (1, 1)),
    (1, 6, 40, 64, 64, 1, 1, (1, 1), (0, 0), (1, 1)),
    (2, 9, 11, 64, 24, 3, 3, (1, 1), (1, 1), (1, 1)),
    (1, 10, 7, 128, 72, 3, 2, (2, 1), (1, 0), (1, 2)),
    (2, 9, 11, 16, 24, 3, 3, (1, 1), (1, 1), (1, 1)),
]


def _variant_applies(v, geom):
    N, H, Wd, C, K, R, S, st, pd, dl = geom
    if v == 0:
        return C == 64 and K == 64 and st == (1, 1)
    if v == 1:
        return C % 64 == 0
    return True


@pytest.mark.parametrize("variant", range(tla.CONV_VARIANTS))
@pytest.mark.parametrize("geom", FORCED)
def test_forced_variants_bit_exact(geom, variant):
    """Each kernel run through tla_conv2d_fprop_variant on the integer set:
    bit-exact where it applies, TLA_ERR_UNSUPPORTED (and y untouched)
    where it does not."""
    N, H, Wd, C, K, R, S, st, pd, dl = geom
    case = W.ConvCase(name="forced", N=N, H=H, W=Wd, C=C, K=K, R=R, S=S, stride=st, pad=pd,
                      dil=dl, dtype=W.BF16, alpha=1.5, beta=0.5, act=W.ACT_RELU, has_c=True,
                      has_bias=True, seed=N * 1000 + H * 10 + C + variant, dist="int3",
                      dist_bias="eighths")
    inp = W.conv_inputs(case)
    if not _variant_applies(variant, geom):
        with pytest.raises(RuntimeError, match="UNSUPPORTED"):
            _run(case, inp, variant=variant)
        return
    got = _run(case, inp, variant=variant)
    want = W.encode(_oracle(case, inp), case.dtype).reshape(got.shape)
    bad = np.argwhere(got != want)
    assert bad.size == 0, "%s v%d: %d mismatches, first at %s" % (geom, variant, len(bad), bad[0])


def _tolerance(case, got, ref):
    ok, worst = og.within_tolerance(og.decode(case.dtype, got), ref, case.tol)
    assert ok, "worst |y-ref|/(1+|ref|) = %g" % worst


def test_random_inputs_gelu_and_c_aliasing_y():
    case = W.ConvCase(name="rand", N=2, H=15, W=14, C=48, K=72, R=3, S=3, stride=(1, 2),
                      pad=(1, 1), dtype=W.BF16, alpha=0.75, beta=1.0, act=W.ACT_GELU,
                      has_c=True, has_bias=True, seed=31)
    inp = W.conv_inputs(case)
    ref = _oracle(case, inp)
    _tolerance(case, _run(case, inp), ref)
    _tolerance(case, _run(case, inp, alias=True), ref)


def test_64_channels_random_gelu_and_c_aliasing_y():
    case = W.ConvCase(name="rand64", N=2, H=15, W=14, C=64, K=64, R=3, S=3, pad=(1, 1),
                      dtype=W.BF16, alpha=0.75, beta=1.0, act=W.ACT_GELU, has_c=True,
                      has_bias=True, seed=32)
    inp = W.conv_inputs(case)
    ref = _oracle(case, inp)
    _tolerance(case, _run(case, inp), ref)
    _tolerance(case, _run(case, inp, alias=True), ref)


def test_measured_layer_full():
    case = W.CONV_F16_56
    inp = W.conv_inputs(case)
    _tolerance(case, _run(case, inp), _oracle(case, inp))


def test_wide_layer_sampled():
    """32 x 28 x 28 x 256 -> 256 (3x3, pad 1, bias, ReLU), the 128 x 128 tile
    path at full size: every tile-boundary row and column plus random points
    against the oracle's per-point mode."""
    case = W.ConvCase(name="conv_f16_n32_28x28x256_k256_3x3", N=32, H=28, W=28, C=256, K=256,
                      R=3, S=3, pad=(1, 1), dtype=W.F16, act=W.ACT_RELU, has_bias=True, seed=6)
    inp = W.conv_inputs(case)
    got = _run(case, inp)
    M = got.shape[0]
    rng = np.random.default_rng(11)
    edges_m = np.unique(np.clip(np.concatenate([np.arange(0, M, 128), np.arange(127, M, 128)]),
                                0, M - 1))
    edges_k = np.array([0, 63, 64, 127, 128, 255])
    ms = np.concatenate([np.repeat(edges_m, edges_k.size), rng.integers(0, M, 4096)])
    ks = np.concatenate([np.tile(edges_k, edges_m.size), rng.integers(0, case.K, 4096)])
    ref = oc.conv2d_points(ms, ks, inp["x"], inp["w"], case.N, case.H, case.W, case.C, case.K,
                           case.R, case.S, case.stride, case.pad, case.dil, case.dtype,
                           bias=inp["bias"], bias_type=case.dtype, alpha=case.alpha,
                           beta=case.beta, act=case.act)
    ok, worst = og.within_tolerance(og.decode(case.dtype, got[ms, ks]), ref, case.tol)
    assert ok, "worst |y-ref|/(1+|ref|) = %g" % worst


@pytest.mark.parametrize("variant", [0, 1])
def test_64_channels_fp32_bias_and_c(variant):
    """An fp32 bias (not y's type) sends the slab kernel's and the implicit
    GEMM's epilogues down the per-element path; integer inputs, bit-exact,
    with C and a band whose last tile is partial."""
    case = W.ConvCase(name="f32bias", N=3, H=9, W=10, C=64, K=64, R=3, S=3, pad=(1, 1),
                      dtype=W.F16, alpha=0.5, beta=1.5, act=W.ACT_RELU, has_c=True,
                      has_bias=False, seed=41, dist="int3")
    inp = W.conv_inputs(case)
    rng = np.random.default_rng(42)
    inp["bias"] = W.encode(rng.integers(-8, 9, size=case.K) / 8.0, W.F32)
    P, Q = case.out_hw()
    x, w, c = to_dev(inp["x"]), to_dev(inp["w"]), to_dev(inp["C"])
    b = to_dev(inp["bias"])
    y = torch.full((case.N * P * Q * case.K,), 0x5A5A, dtype=torch.int16, device="cuda")
    tla.conv2d_fprop(x, w, y, case.N, case.H, case.W, case.C, case.K, case.R, case.S,
                     case.dtype, case.stride, case.pad, case.dil, C_res=c, bias=b,
                     bias_type=W.F32, alpha=case.alpha, beta=case.beta, act=case.act,
                     variant=variant)
    torch.cuda.synchronize()
    got = to_host(y, np.dtype(np.uint16)).reshape(case.N * P * Q, case.K)
    ref = oc.conv2d(inp["x"], inp["w"], case.N, case.H, case.W, case.C, case.K, case.R, case.S,
                    case.stride, case.pad, case.dil, case.dtype, Cres=inp["C"], bias=inp["bias"],
                    bias_type=W.F32, alpha=case.alpha, beta=case.beta, act=case.act)
    want = W.encode(ref, case.dtype).reshape(got.shape)
    bad = np.argwhere(got != want)
    assert bad.size == 0, "v%d: %d mismatches, first at %s" % (variant, len(bad), bad[0])
