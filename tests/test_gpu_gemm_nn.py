"""GEMM parity with an N-contiguous B (a row-major K x N matrix) on the fast
128 x 128 kernel and the two-group 256 x 256 kernel, whose B fragments come
through LDS transpose reads (ds_read_b64_tr_b16), through the C ABI against
the oracle:

* integer-valued inputs, bit for bit, over both 16-bit types, the whole
  epilogue (alpha, beta*C, bias, ReLU), ragged M and N (N a multiple of 8,
  down to one 16-byte chunk), K from one k-tile up, and pitched operands
  with NaN padding;
* the kernel choice: variant 1 below 128 tiles of 256 x 256, variant 0
  (its own transpose-read form) from there on, either forcible, variant 3
  refused, the general kernel forcible;
* the general kernel's own k-rows-of-n slab for pitches and bases off
  16-byte alignment: N and K ragged down to one element, misaligned bases;
* random inputs at 2048 x 2048 x 1024 and 4096 x 4096 x 512 within the
  tolerance.
Tolerance: |D - ref| <= tol*(1 + |ref|), tol 1e-2.
"""
import numpy as np
import pytest

import tiled_layout_algebra_amd as tla
import workloads as W
from oracle import gemm as og
from tests import gpu_util as G

pytestmark = pytest.mark.gpu
SENT = 0x5A5A

SHAPES = [(64, 8, 64), (128, 128, 128), (300, 136, 192), (257, 520, 448), (129, 264, 64),
          (1000, 1032, 1024)]


def _case(M, N, K, a_type, seed, **kw):
    return W.GemmCase(name="nn", M=M, N=N, K=K, a_type=a_type, b_type=a_type, d_type=a_type,
                      a_order=W.ROW, b_order=W.ROW, alpha=1.5, beta=0.5, act=W.ACT_RELU,
                      has_c=True, has_bias=True, seed=seed, dist_a="int3", dist_b="int3",
                      dist_c="int3", dist_bias="eighths", **kw)


def _exact(case, inp, variant=None):
    D = G.run_gemm(case, inp, sentinel=SENT, variant=variant)
    assert G.padding_untouched(case, D, SENT)
    want = W.encode(G.oracle_ref(case, inp), case.d_type).reshape(case.M, case.N)
    got = W.d_logical(case, D)
    bad = np.argwhere(got != want)
    assert bad.size == 0, "%s: %d mismatches, first at %s" % (
        (case.M, case.N, case.K), len(bad), bad[0])


@pytest.mark.parametrize("a_type", [W.F16, W.BF16])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_row_major_b_bit_exact(M, N, K, a_type):
    case = _case(M, N, K, a_type, seed=M * 7 + N + K)
    assert G.variant(case) == "gemm_fast_128x128"
    _exact(case, W.gemm_inputs(case))


@pytest.mark.parametrize("a_type", [W.F16, W.BF16])
def test_row_major_b_pitched_nan_padding(a_type):
    case = _case(300, 136, 192, a_type, seed=5)
    case.lda += 8
    case.ldb += 24   # rows stay 16-byte aligned: the transpose-read path
    case.ldc += 5
    case.ldd += 8
    assert G.variant(case) == "gemm_fast_128x128"
    _exact(case, W.gemm_inputs(case))  # NaN padding would poison D


def test_row_major_b_unaligned_pitch_takes_general_path():
    case = _case(300, 136, 192, W.BF16, seed=6)
    case.ldb += 3
    assert G.variant(case) == "gemm_general_128x128"
    _exact(case, W.gemm_inputs(case))


GENERAL_SHAPES = [(1, 1, 1), (37, 7, 5), (64, 13, 64), (130, 129, 77), (300, 261, 200),
                  (257, 1031, 131), (96, 4097, 40)]


@pytest.mark.parametrize("a_type", [W.F16, W.BF16])
@pytest.mark.parametrize("M,N,K", GENERAL_SHAPES)
def test_general_kernel_row_major_b_bit_exact(M, N, K, a_type):
    """Odd pitches for A, B, C and D and bases one element off alignment:
    the general kernel with B's slab as k rows of n (chunks crossing N
    element by element, rows past K zero)."""
    case = _case(M, N, K, a_type, seed=M * 3 + N + K)
    case.lda += 1
    case.ldb += 1
    case.ldc += 3
    case.ldd += 1
    assert G.variant(case) == "gemm_general_128x128"
    inp = W.gemm_inputs(case)
    D = G.run_gemm(case, inp, sentinel=SENT, pad_front=1)
    assert G.padding_untouched(case, D, SENT)
    want = W.encode(G.oracle_ref(case, inp), case.d_type).reshape(case.M, case.N)
    got = W.d_logical(case, D)
    bad = np.argwhere(got != want)
    assert bad.size == 0, "%s: %d mismatches, first at %s" % ((M, N, K), len(bad), bad[0])


@pytest.mark.parametrize("a_type", [W.F16, W.BF16])
def test_row_major_b_forced_variants(a_type):
    case = _case(300, 520, 384, a_type, seed=7)
    inp = W.gemm_inputs(case)
    for v in (0, 1, 2):
        _exact(case, inp, variant=v)
    with pytest.raises(tla.TlaError, match="UNSUPPORTED"):
        G.run_gemm(case, inp, sentinel=SENT, variant=3)


@pytest.mark.parametrize("M,N,K", [(256, 256, 64), (513, 776, 320), (1000, 1032, 1024)])
def test_row_major_b_two_group_kernel_bit_exact(M, N, K):
    case = _case(M, N, K, W.BF16, seed=M + N + K)
    _exact(case, W.gemm_inputs(case), variant=0)


def test_row_major_b_random_4096_two_group_kernel():
    case = W.GemmCase(name="nn_rand_big", M=4096, N=4096, K=512, a_type=W.BF16, b_type=W.BF16,
                      d_type=W.BF16, a_order=W.ROW, b_order=W.ROW, alpha=1.5, beta=0.5,
                      act=W.ACT_RELU, has_c=True, has_bias=True, seed=9)
    assert G.variant(case) == "gemm_pingpong_256x256"
    inp = W.gemm_inputs(case)
    D = G.run_gemm(case, inp, sentinel=SENT)
    assert G.padding_untouched(case, D, SENT)
    got = og.decode(case.d_type, W.d_logical(case, D).copy())
    ok, worst = og.within_tolerance(got, G.oracle_ref(case, inp), case.tol)
    assert ok, "worst |D-ref|/(1+|ref|) = %g" % worst


def test_row_major_b_random_2048():
    case = W.GemmCase(name="nn_rand", M=2048, N=2048, K=1024, a_type=W.BF16, b_type=W.BF16,
                      d_type=W.BF16, a_order=W.ROW, b_order=W.ROW, alpha=1.0, beta=1.0,
                      act=W.ACT_GELU, has_c=True, has_bias=True, seed=8)
    assert G.variant(case) == "gemm_fast_128x128"
    inp = W.gemm_inputs(case)
    D = G.run_gemm(case, inp, sentinel=SENT)
    assert G.padding_untouched(case, D, SENT)
    got = og.decode(case.d_type, W.d_logical(case, D).copy())
    ok, worst = og.within_tolerance(got, G.oracle_ref(case, inp), case.tol)
    assert ok, "worst |D-ref|/(1+|ref|) = %g" % worst
