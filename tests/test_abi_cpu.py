"""The C ABI without a GPU: the library loads and exports every function
include/tla.h declares; argument errors come back as status codes before
any device work; the host-side descriptor builders (logical/tiled divide,
thread map) agree with the oracle's definitions."""
import ctypes
import os
import re

import pytest

import tiled_layout_algebra_amd as tla
from oracle import layout as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tla.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tla_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = tla.lib()
    names = _declared()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(tla.EXPORTED) == names
    assert tla.version() == 1
    for code, name in [(0, "TLA_OK"), (-1, "TLA_ERR_INVALID_ARG"), (-2, "TLA_ERR_UNSUPPORTED"),
                       (-3, "TLA_ERR_OVERLAP"), (-4, "TLA_ERR_HIP")]:
        assert tla.status_string(code) == name


FAKE = 1 << 20  # an aligned address that is never dereferenced on these paths


def _args(**kw):
    base = dict(M=64, N=64, K=64, A=FAKE, a_type=tla.BF16, a_order=tla.ROW_MAJOR, lda=64,
                B=FAKE, b_type=tla.BF16, b_order=tla.COL_MAJOR, ldb=64,
                C=None, c_type=tla.BF16, c_order=tla.ROW_MAJOR, ldc=64,
                D=FAKE, d_type=tla.BF16, d_order=tla.ROW_MAJOR, ldd=64,
                bias=None, bias_type=tla.BF16, act=tla.ACT_NONE,
                alpha=1.0, beta=0.0, scale_a=1.0, scale_b=1.0)
    base.update(kw)
    return tla.GemmArgs(**base)


def _variant(a):
    buf = ctypes.create_string_buffer(64)
    rc = tla.lib().tla_gemm_variant(ctypes.byref(a), buf, 64)
    return rc, buf.value.decode()


@pytest.mark.parametrize("kw,status", [
    (dict(M=-1), tla.ERR_INVALID_ARG),
    (dict(K=-5), tla.ERR_INVALID_ARG),
    (dict(a_order=7), tla.ERR_INVALID_ARG),
    (dict(act=9), tla.ERR_INVALID_ARG),
    (dict(b_type=tla.F16), tla.ERR_UNSUPPORTED),
    (dict(a_type=tla.F32, b_type=tla.F32), tla.ERR_UNSUPPORTED),
    (dict(d_type=tla.E4M3), tla.ERR_UNSUPPORTED),
    (dict(beta=0.5), tla.ERR_INVALID_ARG),                 # C missing
    (dict(beta=0.5, C=FAKE, c_type=tla.E4M3), tla.ERR_UNSUPPORTED),
    (dict(bias=FAKE, bias_type=tla.E4M3), tla.ERR_UNSUPPORTED),
    (dict(D=None), tla.ERR_INVALID_ARG),
    (dict(A=None), tla.ERR_INVALID_ARG),
    (dict(lda=63), tla.ERR_INVALID_ARG),                   # row-major A needs lda >= K
    (dict(a_order=tla.COL_MAJOR, lda=63), tla.ERR_INVALID_ARG),
    (dict(ldb=10), tla.ERR_INVALID_ARG),
    (dict(ldd=3), tla.ERR_INVALID_ARG),
    (dict(beta=1.0, C=FAKE, ldc=8), tla.ERR_INVALID_ARG),
    (dict(beta=1.0, C=FAKE, c_order=tla.COL_MAJOR), tla.ERR_INVALID_ARG),  # aliases D, other order
])
def test_gemm_argument_errors(kw, status):
    a = _args(**kw)
    assert tla.gemm_epilogue_args(a, None) == status
    assert _variant(a)[0] == status


def test_gemm_null_args_and_noops():
    assert tla.lib().tla_gemm_epilogue(None, None) == tla.ERR_INVALID_ARG
    # M == 0 / N == 0 are no-ops even with NULL pointers
    assert tla.gemm_epilogue_args(_args(M=0, A=None, B=None, D=None), None) == tla.OK
    assert tla.gemm_epilogue_args(_args(N=0, A=None, B=None, D=None), None) == tla.OK
    assert _variant(_args(M=0))[1] == "noop"
    # K == 0 needs no A/B and no lda/ldb
    assert _variant(_args(K=0, A=None, B=None, lda=0, ldb=0)) == (0, "gemm_general_128x128")


def test_gemm_variant_choice():
    # aligned K-contiguous operands with K a multiple of the slab width: fast
    assert _variant(_args(M=4096, N=4096, K=4096, lda=4096, ldb=4096, ldd=4096))[1] == "gemm_pingpong_256x256"
    assert _variant(_args(M=256, N=256, K=256, lda=256, ldb=256, ldd=256))[1] == "gemm_fast_128x128"
    e4 = dict(a_type=tla.E4M3, b_type=tla.E4M3, M=8192, N=8192, K=8192, lda=8192, ldb=8192, ldd=8192)
    assert _variant(_args(**e4))[1] == "gemm_pingpong_256x256"
    assert _variant(_args(**dict(e4, M=1024, N=1024)))[1] == "gemm_fast_128x128"
    # fp8 slabs are 128 elements wide: with K = 64 only the two-group kernel
    # (range-checked copies) stays fast, so small e4m3 problems go general
    assert _variant(_args(**dict(e4, K=64, lda=64, ldb=64)))[1] == "gemm_pingpong_256x256"
    assert _variant(_args(**dict(e4, M=1024, N=1024, K=64, lda=64, ldb=64)))[1] == "gemm_general_128x128"
    assert _variant(_args(**dict(e4, K=72, lda=80, ldb=80)))[1] == "gemm_general_128x128"  # K % 16
    # N-contiguous 16-bit B with aligned rows: the 128 x 128 transpose-read
    # kernel below 128 tiles of 256 x 256, the two-group kernel's
    # transpose-read form from there on (the fast layout's rule)
    assert _variant(_args(b_order=tla.ROW_MAJOR))[1] == "gemm_fast_128x128"
    big_nn = dict(M=4096, N=4096, K=4096, lda=4096, ldb=4096, ldd=4096, b_order=tla.ROW_MAJOR)
    assert _variant(_args(**big_nn))[1] == "gemm_pingpong_256x256"
    assert _variant(_args(**dict(big_nn, M=3072, N=3072, ldb=3072, ldd=3072)))[1] == "gemm_pingpong_256x256"
    assert _variant(_args(**dict(big_nn, M=2048, N=2048, ldb=2048, ldd=2048)))[1] == "gemm_fast_128x128"
    assert _variant(_args(**dict(big_nn, M=2048 - 256)))[1] == "gemm_fast_128x128"  # 112 tiles
    assert _variant(_args(**dict(big_nn, M=2048)))[1] == "gemm_pingpong_256x256"  # 128
    # ... but not for e4m3, N not a multiple of 8, unaligned B rows or K off
    # the 16-byte chunk
    assert _variant(_args(**dict(e4, b_order=tla.ROW_MAJOR)))[1] == "gemm_general_128x128"
    assert _variant(_args(b_order=tla.ROW_MAJOR, N=60, ldd=60, ldb=60))[1] == "gemm_general_128x128"
    assert _variant(_args(b_order=tla.ROW_MAJOR, ldb=67))[1] == "gemm_general_128x128"
    assert _variant(_args(b_order=tla.ROW_MAJOR, K=92, lda=96))[1] == "gemm_general_128x128"
    # 16-bit K a multiple of 8 but not of the 64-element slab: still fast
    assert _variant(_args(b_order=tla.ROW_MAJOR, K=96, lda=96))[1] == "gemm_fast_128x128"
    assert _variant(_args(K=96, lda=96, ldb=96))[1] == "gemm_fast_128x128"
    big_k = dict(M=4096, N=4096, K=4000, lda=4096, ldb=4096, ldd=4096)
    assert _variant(_args(**big_k))[1] == "gemm_pingpong_256x256"
    # column-major 16-bit A with aligned columns, M a multiple of 8: the
    # transpose-read forms, by the fast layout's rule, either B layout
    at = dict(a_order=tla.COL_MAJOR, M=4096, N=4096, K=4096, lda=4096, ldb=4096, ldd=4096)
    assert _variant(_args(**at))[1] == "gemm_pingpong_256x256"
    assert _variant(_args(**dict(at, b_order=tla.ROW_MAJOR)))[1] == "gemm_pingpong_256x256"
    assert _variant(_args(**dict(at, M=1024, N=1024, lda=1024, ldd=1024)))[1] == "gemm_fast_128x128"
    assert _variant(_args(**dict(at, M=4092, ldd=4096)))[1] == "gemm_general_128x128"  # M % 8
    assert _variant(_args(**dict(at, lda=4100)))[1] == "gemm_general_128x128"  # column pitch
    assert _variant(_args(**dict(at, a_type=tla.E4M3, b_type=tla.E4M3)))[1] == "gemm_general_128x128"
    # odd pitches, misaligned bases, K off the chunk: general
    assert _variant(_args(lda=65))[1] == "gemm_general_128x128"
    assert _variant(_args(A=FAKE + 2))[1] == "gemm_general_128x128"
    assert _variant(_args(K=63, lda=64, ldb=64))[1] == "gemm_general_128x128"


def test_transpose_argument_errors():
    f = tla.lib().tla_tiled_transpose
    assert f(FAKE, 8, FAKE * 4, 8, -1, 8, 4, None) == tla.ERR_INVALID_ARG
    assert f(FAKE, 8, FAKE * 4, 8, 8, 8, 3, None) == tla.ERR_UNSUPPORTED
    assert f(FAKE, 8, FAKE * 4, 8, 0, 8, 4, None) == tla.OK          # empty
    assert f(None, 8, FAKE * 4, 8, 8, 8, 4, None) == tla.ERR_INVALID_ARG
    assert f(FAKE, 7, FAKE * 4, 8, 8, 8, 4, None) == tla.ERR_INVALID_ARG  # ld_src < N
    assert f(FAKE, 8, FAKE * 4, 7, 8, 8, 4, None) == tla.ERR_INVALID_ARG  # ld_dst < M
    assert f(FAKE + 2, 8, FAKE * 4, 8, 8, 8, 4, None) == tla.ERR_INVALID_ARG  # misaligned
    assert f(FAKE, 8, FAKE + 64, 8, 8, 8, 4, None) == tla.ERR_OVERLAP
    assert f(FAKE + 64, 8, FAKE, 8, 8, 8, 4, None) == tla.ERR_OVERLAP


def test_copy_argument_errors():
    f = tla.lib().tla_tiled_copy
    assert f(FAKE, 8, FAKE * 4, 8, -1, 8, 4, None) == tla.ERR_INVALID_ARG
    assert f(FAKE, 8, FAKE * 4, 8, 8, 8, 3, None) == tla.ERR_UNSUPPORTED
    assert f(FAKE, 8, FAKE * 4, 8, 0, 8, 4, None) == tla.OK          # empty
    assert f(None, 8, FAKE * 4, 8, 8, 8, 4, None) == tla.ERR_INVALID_ARG
    assert f(FAKE, 7, FAKE * 4, 8, 8, 8, 4, None) == tla.ERR_INVALID_ARG  # ld_src < N
    assert f(FAKE, 8, FAKE * 4, 7, 8, 8, 4, None) == tla.ERR_INVALID_ARG  # ld_dst < N
    assert f(FAKE + 2, 8, FAKE * 4, 8, 8, 8, 4, None) == tla.ERR_INVALID_ARG  # misaligned
    assert f(FAKE, 8, FAKE + 64, 8, 8, 8, 4, None) == tla.ERR_OVERLAP


def _eval_desc(d):
    shape, stride = tla.layout_tuple(d)
    return L.Layout(shape, stride)


def test_layout_size_and_descriptor_round_trip():
    d = tla.make_layout(((4, 8), (2, 2, 2)), ((32, 1), (16, 8, 128)))
    assert tla.layout_size(d) == 256
    assert tla.layout_tuple(d) == (((4, 8), (2, 2, 2)), ((32, 1), (16, 8, 128)))
    bad = tla.make_layout((4, 0), (1, 4))
    with pytest.raises(tla.TlaError):
        tla.layout_size(bad)


@pytest.mark.parametrize("shape,stride,tile", [
    ((1024,), (1,), (128,)),
    ((10, 7), (7, 1), (4, 3)),
    ((96, 64), (64, 1), (32, 32)),
    ((5, 6, 7), (1, 5, 30), (2, 3, 4)),
    ((16384, 16384), (16384, 1), (32, 32)),
])
def test_divide_descriptors_match_oracle(shape, stride, tile):
    d = tla.make_layout(shape, stride)
    ld = tla.logical_divide(d, tile)
    td = tla.tiled_divide(d, tile)
    o_ld = L.logical_divide(L.Layout(shape, stride), tile)
    o_td = L.tiled_divide(L.Layout(shape, stride), tile)
    ev_ld, ev_td = _eval_desc(ld), _eval_desc(td)
    # same leaves in the same order (a one-leaf mode prints as an int)
    assert L.flatten(ev_ld.shape) == L.flatten(o_ld.shape)
    assert L.flatten(ev_td.shape) == L.flatten(o_td.shape)
    n = o_ld.size()
    idxs = range(n) if n <= 5000 else range(0, n, n // 4999)
    for i in idxs:
        assert ev_ld(i) == o_ld(L.idx2crd(i, o_ld.shape))
        assert ev_td(i) == o_td(L.idx2crd(i, o_td.shape))


def test_divide_errors():
    d = tla.make_layout(((2, 2), 4), ((1, 2), 4))  # nested: not flat
    with pytest.raises(tla.TlaError):
        tla.logical_divide(d, (2, 2))
    with pytest.raises(tla.TlaError):
        tla.logical_divide(tla.make_layout((8,), (1,)), (0,))
    with pytest.raises(tla.TlaError):
        tla.logical_divide(tla.make_layout((8, 8), (8, 1)), (2,))


@pytest.mark.parametrize("R,C,T,V,I,contig", [
    (64, 64, 128, 4, 8, 1), (64, 64, 128, 4, 8, 0), (256, 8, 256, 1, 8, 1),
    (128, 8, 256, 1, 4, 0), (32, 32, 256, 1, 4, 1), (16, 16, 64, 4, 1, 1),
])
def test_thread_map_descriptor_matches_oracle(R, C, T, V, I, contig):
    d = tla.thread_map(R, C, T, V, I, contig)
    tm = L.StripMinedThreadMap(R, C, T, V, I, contig)
    ev = _eval_desc(d)
    assert ev.shape == tm.tv_layout().shape and ev.stride == tm.tv_layout().stride
    assert ev.table() == tm.table()


@pytest.mark.parametrize("args", [
    (64, 64, 128, 4, 4, 1),   # tile equation violated
    (64, 60, 120, 8, 4, 1),   # V does not divide C
    (64, 64, 128, 4, 8, 2),   # bad contiguous dim
    (0, 64, 128, 4, 8, 1),
])
def test_thread_map_errors(args):
    with pytest.raises(tla.TlaError):
        tla.thread_map(*args)
    assert tla.lib().tla_thread_map_eval(*args, 64, 64, FAKE, None, None) == tla.ERR_INVALID_ARG


def test_layout_eval_argument_errors():
    f = tla.lib().tla_layout_eval
    outer = tla.make_layout((4, 8), (8, 1))
    inner = tla.make_layout((8, 4), (4, 1))
    assert f(ctypes.byref(outer), None, FAKE, 31, None) == tla.ERR_INVALID_ARG   # n != size
    assert f(ctypes.byref(outer), None, None, 32, None) == tla.ERR_INVALID_ARG   # out NULL
    big = tla.make_layout((8, 8), (8, 1))                                        # reaches 63 >= 32
    assert f(ctypes.byref(outer), ctypes.byref(big), FAKE, 64, None) == tla.ERR_INVALID_ARG
    neg = tla.make_layout((4,), (-1,))
    assert f(ctypes.byref(outer), ctypes.byref(neg), FAKE, 4, None) == tla.ERR_INVALID_ARG
    assert f(ctypes.byref(outer), ctypes.byref(inner), FAKE, 31, None) == tla.ERR_INVALID_ARG
    assert f(None, None, FAKE, 1, None) == tla.ERR_INVALID_ARG


def test_run_variant_argument_errors():
    """Variant ids outside [0, TLA_GEMM_VARIANTS) are argument errors, and a
    fast variant on a problem without the fast layout is refused -- both
    before any device work."""
    a = _args()
    for bad in (-1, tla.GEMM_VARIANTS, 99):
        assert tla.lib().tla_gemm_run_variant(ctypes.byref(a), bad, None) == tla.ERR_INVALID_ARG
    nn = _args(b_order=tla.ROW_MAJOR, ldb=67)   # B rows not 16-byte aligned
    for v in (0, 1, 3):
        assert tla.lib().tla_gemm_run_variant(ctypes.byref(nn), v, None) == tla.ERR_UNSUPPORTED
    # aligned N-contiguous B: the single-group 256 x 256 kernel has no such form
    nn = _args(b_order=tla.ROW_MAJOR, ldb=64)
    assert tla.lib().tla_gemm_run_variant(ctypes.byref(nn), 3, None) == tla.ERR_UNSUPPORTED
    # column-major A: the single-group 256 x 256 kernel has no such form
    at = _args(a_order=tla.COL_MAJOR)
    assert tla.lib().tla_gemm_run_variant(ctypes.byref(at), 3, None) == tla.ERR_UNSUPPORTED
    # e4m3 with K off the 128-byte slab: the 128 x 128 and 256 x 256 kernels
    # copy whole slabs without a range check
    e4 = _args(a_type=tla.E4M3, b_type=tla.E4M3, K=80, lda=80, ldb=80)
    for v in (1, 3):
        assert tla.lib().tla_gemm_run_variant(ctypes.byref(e4), v, None) == tla.ERR_UNSUPPORTED


def _conv(**kw):
    base = dict(N=1, H=8, W=8, C=16, K=16, R=3, S=3, stride_h=1, stride_w=1, pad_h=1, pad_w=1,
                dil_h=1, dil_w=1, x=FAKE, w=FAKE, C_res=None, y=FAKE, type=tla.F16, bias=None,
                bias_type=tla.F16, act=tla.ACT_NONE, alpha=1.0, beta=0.0)
    base.update(kw)
    return tla.ConvArgs(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(N=-1), tla.ERR_INVALID_ARG), (dict(C=0), tla.ERR_INVALID_ARG),
    (dict(stride_h=0), tla.ERR_INVALID_ARG), (dict(dil_w=0), tla.ERR_INVALID_ARG),
    (dict(pad_h=-1), tla.ERR_INVALID_ARG), (dict(act=9), tla.ERR_INVALID_ARG),
    (dict(type=tla.E4M3), tla.ERR_UNSUPPORTED), (dict(x=None), tla.ERR_INVALID_ARG),
    (dict(beta=0.5), tla.ERR_INVALID_ARG),                       # beta != 0 without C
    (dict(pad_h=1 << 29, stride_h=1 << 30), tla.ERR_INVALID_ARG),  # padded extent >= 2^30
    (dict(W=(1 << 30) - 2, pad_w=1, N=0), tla.ERR_INVALID_ARG),
    (dict(N=0), tla.OK), (dict(H=2, R=5, pad_h=0), tla.OK),     # empty output: no-op
])
def test_conv_argument_errors(kw, status):
    a = _conv(**kw)
    assert tla.lib().tla_conv2d_fprop(ctypes.byref(a), None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(N=-1), tla.ERR_INVALID_ARG), (dict(type=tla.E4M3), tla.ERR_UNSUPPORTED),
    (dict(beta=0.5), tla.ERR_INVALID_ARG), (dict(N=0), tla.OK),
])
def test_conv_variant_validates_like_the_dispatching_call(kw, status):
    a = _conv(**kw)
    for v in range(tla.CONV_VARIANTS):
        assert tla.lib().tla_conv2d_fprop_variant(ctypes.byref(a), v, None) == status


def test_conv_variant_refusals():
    """Variant ids outside [0, TLA_CONV_VARIANTS) are argument errors; the
    slab kernel is refused outside 64 -> 64 channels at stride 1, and the
    direct-to-LDS implicit GEMM when C is not a multiple of 64 -- all before
    any device work."""
    a = _conv()
    for bad in (-1, tla.CONV_VARIANTS, 7):
        assert tla.lib().tla_conv2d_fprop_variant(ctypes.byref(a), bad, None) == tla.ERR_INVALID_ARG
    for kw in (dict(), dict(C=64, K=32), dict(C=128, K=64), dict(C=64, K=64, stride_h=2),
               dict(C=64, K=64, x=FAKE + 8)):
        assert tla.lib().tla_conv2d_fprop_variant(ctypes.byref(_conv(**kw)), 0, None) == \
            tla.ERR_UNSUPPORTED, kw
    for kw in (dict(), dict(C=96), dict(C=64, x=FAKE + 8)):
        assert tla.lib().tla_conv2d_fprop_variant(ctypes.byref(_conv(**kw)), 1, None) == \
            tla.ERR_UNSUPPORTED, kw
