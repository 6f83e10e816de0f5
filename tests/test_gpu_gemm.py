"""GEMM + epilogue parity: the HIP path through the C ABI against the
oracle on the same seeded inputs.

* integer-valued inputs: every partial sum is exact in fp32, so D must equal
  the oracle's exact result rounded to D's type, bit for bit;
* the measured workloads at full size, every output compared (a sampled
  pre-check of the tile-boundary rows and columns runs first), and at
  reduced sizes;
* edge cases: K = 0, ragged edges on every side, pitched operands with NaN
  padding, sentinel-filled output padding, misaligned bases, C aliasing D,
  column-major C and D, fp32 C and bias.
Tolerance: |D - ref| <= tol*(1 + |ref|), tol 1e-2 (fp16/bf16), 5e-2 (fp8).
"""
import dataclasses
import itertools

import numpy as np
import pytest

import workloads as W
from oracle import gemm as og
from tests import gpu_util as G

pytestmark = pytest.mark.gpu
SENT = {W.F16: 0x5A5A, W.BF16: 0x5A5A}


def _logical(case, D):
    return og.decode(case.d_type, W.d_logical(case, D).copy())


def _check_full(case, inp, **kw):
    D = G.run_gemm(case, inp, sentinel=SENT[case.d_type], **kw)
    assert G.padding_untouched(case, D, SENT[case.d_type])
    got = _logical(case, D)
    ref = G.oracle_ref(case, inp)
    ok, worst = og.within_tolerance(got, ref, case.tol)
    assert ok, "%s: worst |D-ref|/(1+|ref|) = %g > %g" % (case.name, worst, case.tol)
    return worst


def _sample(case, rng, tile=256):
    rows = {0, 1, case.M - 1}
    cols = {0, 1, case.N - 1}
    for t in range(tile, case.M, tile):
        rows |= {t - 1, t}
    for t in range(tile, case.N, tile):
        cols |= {t - 1, t}
    rows |= set(rng.integers(0, case.M, 16).tolist())
    cols |= set(rng.integers(0, case.N, 8).tolist())
    rows, cols = sorted(r for r in rows if r < case.M), sorted(c for c in cols if c < case.N)
    ms = [m for m in rows for _ in range(case.N)]
    ns = [n for _ in rows for n in range(case.N)]
    ms += [m for _ in cols for m in range(case.M)]
    ns += [n for n in cols for _ in range(case.M)]
    ms += rng.integers(0, case.M, 4096).tolist()
    ns += rng.integers(0, case.N, 4096).tolist()
    return np.array(ms, dtype=np.int64), np.array(ns, dtype=np.int64)


def _check_sampled(case, inp, seed=0):
    D = G.run_gemm(case, inp, sentinel=SENT[case.d_type])
    assert G.padding_untouched(case, D, SENT[case.d_type])
    got = _logical(case, D)
    ms, ns = _sample(case, np.random.default_rng(seed))
    ref = G.oracle_points(case, inp, ms, ns)
    ok, worst = og.within_tolerance(got[ms, ns], ref, case.tol)
    assert ok, "%s: worst |D-ref|/(1+|ref|) = %g > %g" % (case.name, worst, case.tol)
    assert not np.isnan(got).any()
    return worst


# ------------------------------------------------------------ bit-exact set

EXACT_SIZES = [(1, 1, 1), (2, 3, 5), (13, 17, 31), (33, 65, 64), (65, 33, 17), (64, 64, 64),
               (128, 128, 128), (131, 67, 200), (256, 256, 256)]
ORDERS = list(itertools.product([W.ROW, W.COL], repeat=2))


@pytest.mark.parametrize("a_type,d_type", [(W.F16, W.F16), (W.BF16, W.BF16), (W.E4M3, W.BF16)])
@pytest.mark.parametrize("M,N,K", EXACT_SIZES)
def test_integer_inputs_bit_exact(M, N, K, a_type, d_type):
    for (a_order, b_order), act in zip(ORDERS, [W.ACT_NONE, W.ACT_RELU, W.ACT_NONE, W.ACT_RELU]):
        case = W.GemmCase(name="exact", M=M, N=N, K=K, a_type=a_type, b_type=a_type,
                          d_type=d_type, a_order=a_order, b_order=b_order, alpha=1.5, beta=0.5,
                          act=act, has_c=True, has_bias=True, seed=M * 1000 + N + K,
                          dist_a="int3", dist_b="int3", dist_c="int3", dist_bias="eighths")
        inp = W.gemm_inputs(case)
        D = G.run_gemm(case, inp, sentinel=SENT[d_type])
        ref = G.oracle_ref(case, inp)
        want = W.encode(ref, d_type).reshape(M, N)
        got = W.d_logical(case, D)
        bad = np.argwhere(got != want)
        assert bad.size == 0, "%s orders %s: %d mismatches, first at %s (variant %s)" % (
            (M, N, K), (a_order, b_order), len(bad), bad[0], G.variant(case))


def test_exact_set_covers_both_paths():
    seen = set()
    for (M, N, K) in EXACT_SIZES:
        for a_type in (W.F16, W.E4M3):
            case = W.GemmCase(name="v", M=M, N=N, K=K, a_type=a_type, b_type=a_type,
                              d_type=W.BF16)
            seen.add(G.variant(case))
    assert {"gemm_fast_128x128", "gemm_general_128x128"} <= seen


# --------------------------------------------------- measured workloads

def test_f16_256_full():
    case = W.GEMM_F16_256
    assert G.variant(case) == "gemm_fast_128x128"
    _check_full(case, W.gemm_inputs(case))


def test_bf16_epilogue_reduced_full():
    case = dataclasses.replace(W.GEMM_BF16_4096, M=512, N=768, K=1024, lda=0, ldb=0, ldc=0, ldd=0)
    case.__post_init__()
    _check_full(case, W.gemm_inputs(case))


def test_bf16_fast256_ragged_edges():
    # 8 x 16 tiles of 256 take the two-group 256x256 kernel; M and N end
    # mid-tile (M = 7*256 + 208: the last tile's rows end inside a 32-row
    # copy block, whose missing rows load as zeros)
    case = dataclasses.replace(W.GEMM_BF16_4096, M=2000, N=4000, K=256, lda=0, ldb=0, ldc=0, ldd=0)
    case.__post_init__()
    assert G.variant(case) == "gemm_pingpong_256x256"
    _check_full(case, W.gemm_inputs(case))


@pytest.fixture(scope="module")
def bf16_4096_inputs():
    return W.gemm_inputs(W.GEMM_BF16_4096)


@pytest.fixture(scope="module")
def e4m3_8192_inputs():
    return W.gemm_inputs(W.GEMM_E4M3_8192)


def test_bf16_4096_full_size_sampled(bf16_4096_inputs):
    """Fast pre-check: every tile-boundary row and column plus random points."""
    case = W.GEMM_BF16_4096
    assert G.variant(case) == "gemm_pingpong_256x256"
    _check_sampled(case, bf16_4096_inputs)


def test_bf16_4096_full_size_every_output(bf16_4096_inputs):
    """The verdict at full size: all 4096 x 4096 outputs against the whole
    oracle GEMM, within 1e-2 (1 + |ref|), no NaN, D's padding untouched."""
    case = W.GEMM_BF16_4096
    assert G.variant(case) == "gemm_pingpong_256x256"
    _check_full(case, bf16_4096_inputs)


def test_f16_ragged_reduced_full():
    case = dataclasses.replace(W.GEMM_F16_RAGGED, M=301, N=409, K=77, lda=0, ldb=0, ldc=0, ldd=0)
    case.__post_init__()
    _check_full(case, W.gemm_inputs(case))


def test_f16_ragged_full_size():
    case = W.GEMM_F16_RAGGED
    assert G.variant(case) == "gemm_general_128x128"
    _check_full(case, W.gemm_inputs(case))


def test_e4m3_gelu_reduced_full():
    case = dataclasses.replace(W.GEMM_E4M3_8192, M=1024, N=768, K=1024, lda=0, ldb=0, ldc=0, ldd=0)
    case.__post_init__()
    assert G.variant(case) == "gemm_fast_128x128"
    _check_full(case, W.gemm_inputs(case))


def test_e4m3_general_path_ragged_k():
    case = dataclasses.replace(W.GEMM_E4M3_8192, M=300, N=200, K=200, lda=0, ldb=0, ldc=0, ldd=0)
    case.__post_init__()
    assert G.variant(case) == "gemm_general_128x128"
    _check_full(case, W.gemm_inputs(case))


def test_e4m3_8192_full_size_sampled(e4m3_8192_inputs):
    """Fast pre-check: every tile-boundary row and column plus random points."""
    case = W.GEMM_E4M3_8192
    _check_sampled(case, e4m3_8192_inputs)


def test_e4m3_8192_full_size_every_output(e4m3_8192_inputs):
    """The verdict at full size: all 8192 x 8192 outputs against the whole
    oracle GEMM, within 5e-2 (1 + |ref|), no NaN, D's padding untouched."""
    _check_full(W.GEMM_E4M3_8192, e4m3_8192_inputs)


# ------------------------------------------------------------- edge cases

def _small(**kw):
    base = dict(name="edge", M=70, N=90, K=100, a_type=W.BF16, b_type=W.BF16, d_type=W.BF16,
                alpha=1.25, beta=0.75, has_c=True, has_bias=True, act=W.ACT_GELU, seed=5)
    base.update(kw)
    return W.GemmCase(**base)


@pytest.mark.parametrize("a_order,b_order", ORDERS)
@pytest.mark.parametrize("a_type", [W.F16, W.BF16, W.E4M3])
def test_pitched_operands_nan_padding(a_order, b_order, a_type):
    case = _small(a_order=a_order, b_order=b_order, a_type=a_type, b_type=a_type,
                  d_type=W.F16 if a_type == W.F16 else W.BF16)
    case.lda += 8
    case.ldb += 3
    case.ldc += 5
    case.ldd += 7
    _check_full(case, W.gemm_inputs(case))  # NaN padding would poison D


def test_fast_path_pitched():
    case = _small(M=256, N=384, K=256, act=W.ACT_RELU)
    case.lda, case.ldb, case.ldc, case.ldd = 256 + 64, 256 + 8, 384 + 4, 384 + 12
    assert G.variant(case) == "gemm_fast_128x128"
    _check_full(case, W.gemm_inputs(case))


def test_k_zero():
    case = _small(K=0, act=W.ACT_RELU)
    case.lda = case.ldb = 1
    inp = W.gemm_inputs(case)
    inp["A"] = inp["B"] = None
    _check_full(case, inp)


def test_misaligned_bases_take_general_path():
    case = _small(M=128, N=128, K=128)
    _check_full(case, W.gemm_inputs(case), pad_front=1)


@pytest.mark.parametrize("a_order,b_order", ORDERS)
@pytest.mark.parametrize("a_type,pad", [(W.F16, 1), (W.BF16, 3), (W.E4M3, 1), (W.E4M3, 2),
                                        (W.E4M3, 3)])
def test_realigned_loads_bit_exact(a_order, b_order, a_type, pad):
    """Bases shifted off alignment by `pad` elements (1 to 3 bytes for e4m3)
    and odd pitches: the general kernel's whole-chunk loads from dword-aligned
    pairs, funnel-shifted, for every byte offset of a row start; integer
    inputs, so D is exact."""
    M, N, K = 150, 140, 203
    d_type = W.F16 if a_type == W.F16 else W.BF16
    case = W.GemmCase(name="realign", M=M, N=N, K=K, a_type=a_type, b_type=a_type,
                      d_type=d_type, a_order=a_order, b_order=b_order, alpha=1.5, beta=0.5,
                      act=W.ACT_RELU, has_c=True, has_bias=True, seed=31 + pad,
                      dist_a="int3", dist_b="int3", dist_c="int3", dist_bias="eighths")
    case.lda += 1
    case.ldb += 3
    case.ldd += 1
    assert G.variant(case) == "gemm_general_128x128"
    inp = W.gemm_inputs(case)
    D = G.run_gemm(case, inp, sentinel=SENT[d_type], pad_front=pad)
    assert G.padding_untouched(case, D, SENT[d_type])
    want = W.encode(G.oracle_ref(case, inp), d_type).reshape(M, N)
    assert np.array_equal(W.d_logical(case, D), want)


@pytest.mark.parametrize("b_order", [W.ROW, W.COL])
@pytest.mark.parametrize("a_type", [W.F16, W.BF16])
@pytest.mark.parametrize("M,N,K", [(300, 264, 200), (7, 40, 131), (1031, 257, 777)])
def test_column_major_a_bit_exact(M, N, K, a_type, b_order):
    """A column-major (M-contiguous) with a pitch past M: the general
    kernel holds it as k rows of m, the tiles that cross M reading on past
    it into NaN-filled pitch padding (rows of D past M are never stored);
    integer inputs, so D is exact."""
    case = W.GemmCase(name="acol", M=M, N=N, K=K, a_type=a_type, b_type=a_type, d_type=a_type,
                      a_order=W.COL, b_order=b_order, alpha=1.5, beta=0.5, act=W.ACT_RELU,
                      has_c=True, has_bias=True, seed=M + N + K, dist_a="int3", dist_b="int3",
                      dist_c="int3", dist_bias="eighths")
    case.lda += 5
    case.ldb += 3
    assert G.variant(case) == "gemm_general_128x128"
    inp = W.gemm_inputs(case)
    D = G.run_gemm(case, inp, sentinel=SENT[a_type])
    assert G.padding_untouched(case, D, SENT[a_type])
    want = W.encode(G.oracle_ref(case, inp), a_type).reshape(M, N)
    assert np.array_equal(W.d_logical(case, D), want)


@pytest.mark.parametrize("a_order,b_order", [(W.COL, W.COL), (W.ROW, W.ROW), (W.COL, W.ROW)])
@pytest.mark.parametrize("M,N,K,pad", [(300, 264, 200, 16), (7, 40, 131, 0), (1031, 257, 777, 32),
                                       (1024, 1024, 1024, 0)])
def test_e4m3_runs_along_m_or_n_bit_exact(M, N, K, pad, a_order, b_order):
    """e4m3 with A column-major and/or B row-major, every run along M or N
    16-byte aligned (pitch: the extent rounded up to 16, plus pad): the
    general kernel loads those runs whole and transposes them in registers
    into its rows-of-k slab.  Ragged M, N and K cross the tile edges, the
    pitch padding holds NaN; integer inputs, so D is exact."""
    case = W.GemmCase(name="e4runs", M=M, N=N, K=K, a_type=W.E4M3, b_type=W.E4M3,
                      d_type=W.BF16, a_order=a_order, b_order=b_order, alpha=1.5, beta=0.5,
                      act=W.ACT_RELU, has_c=True, has_bias=True, seed=M + N + K + pad,
                      dist_a="int3", dist_b="int3", dist_c="int3", dist_bias="eighths")
    if a_order == W.COL:
        case.lda = -(-M // 16) * 16 + pad
    if b_order == W.ROW:
        case.ldb = -(-N // 16) * 16 + pad
    assert G.variant(case) == "gemm_general_128x128"
    inp = W.gemm_inputs(case)
    D = G.run_gemm(case, inp, sentinel=SENT[W.BF16])
    assert G.padding_untouched(case, D, SENT[W.BF16])
    want = W.encode(G.oracle_ref(case, inp), W.BF16).reshape(M, N)
    assert np.array_equal(W.d_logical(case, D), want)


@pytest.mark.parametrize("b_order", [W.ROW, W.COL])
@pytest.mark.parametrize("a_type", [W.F16, W.BF16])
@pytest.mark.parametrize("M,N,K", [(296, 264, 200), (8, 40, 64), (1024, 520, 1000)])
def test_column_major_a_fast_kernel_bit_exact(M, N, K, a_type, b_order):
    """A column-major with 16-byte aligned columns and M a multiple of 8: the
    128 x 128 kernel holds A as k rows of m (direct copies, transpose reads);
    rows of k past K lie past the copy's record count, tiles past M read the
    last 8 columns; NaN pitch padding on every operand; integer inputs, so D
    is exact."""
    case = W.GemmCase(name="acol_fast", M=M, N=N, K=K, a_type=a_type, b_type=a_type,
                      d_type=a_type, a_order=W.COL, b_order=b_order, alpha=1.5, beta=0.5,
                      act=W.ACT_RELU, has_c=True, has_bias=True, seed=M + N + K + 1,
                      dist_a="int3", dist_b="int3", dist_c="int3", dist_bias="eighths")
    case.lda += 8
    case.ldb += 8 if b_order == W.COL else 16
    assert G.variant(case) == "gemm_fast_128x128"
    inp = W.gemm_inputs(case)
    D = G.run_gemm(case, inp, sentinel=SENT[a_type])
    assert G.padding_untouched(case, D, SENT[a_type])
    want = W.encode(G.oracle_ref(case, inp), a_type).reshape(M, N)
    assert np.array_equal(W.d_logical(case, D), want)


@pytest.mark.parametrize("b_order", [W.ROW, W.COL])
@pytest.mark.parametrize("M,N,K", [(296, 264, 200), (520, 776, 1000)])
def test_column_major_a_two_group_kernel_bit_exact(M, N, K, b_order):
    """The two-group kernel's k-rows-of-m form for a column-major A (forced;
    the dispatch takes it from 128 tiles of 256 x 256)."""
    case = W.GemmCase(name="acol_pp", M=M, N=N, K=K, a_type=W.BF16, b_type=W.BF16,
                      d_type=W.BF16, a_order=W.COL, b_order=b_order, alpha=1.5, beta=0.5,
                      act=W.ACT_RELU, has_c=True, has_bias=True, seed=M + N + K + 2,
                      dist_a="int3", dist_b="int3", dist_c="int3", dist_bias="eighths")
    case.lda += 8
    case.ldb += 8 if b_order == W.COL else 16
    inp = W.gemm_inputs(case)
    D = G.run_gemm(case, inp, sentinel=SENT[W.BF16], variant=0)
    assert G.padding_untouched(case, D, SENT[W.BF16])
    want = W.encode(G.oracle_ref(case, inp), W.BF16).reshape(M, N)
    assert np.array_equal(W.d_logical(case, D), want)


def test_column_major_a_random_4096_auto():
    case = _small(M=4096, N=4096, K=1024, a_order=W.COL, b_order=W.ROW, act=W.ACT_RELU,
                  seed=25)
    assert G.variant(case) == "gemm_pingpong_256x256"
    _check_sampled(case, W.gemm_inputs(case), seed=6)


def test_column_major_a_fast_kernel_random_2048():
    case = _small(M=2048, N=2048, K=1024, a_order=W.COL, act=W.ACT_GELU, seed=24)
    assert G.variant(case) == "gemm_fast_128x128"
    _check_full(case, W.gemm_inputs(case))


@pytest.mark.parametrize("b_order", [W.ROW, W.COL])
@pytest.mark.parametrize("a_type", [W.F16, W.BF16])
@pytest.mark.parametrize("M,N,K", [(130, 201, 96), (70, 4223, 64), (257, 69, 40), (65, 4129, 16)])
def test_odd_pitch_epilogue_edges_bit_exact(M, N, K, a_type, b_order):
    """C and D at odd pitches with a bias: wave tiles that end inside M, or
    inside N with at least half their columns in D, take the any-pitch LDS
    epilogue (row-predicated stores, the chunk that crosses N element by
    element, bias groups past N clamped), narrower ones the per-group path;
    integer inputs, so D is exact and D's padding keeps its sentinel."""
    case = W.GemmCase(name="epi_edges", M=M, N=N, K=K, a_type=a_type, b_type=a_type,
                      d_type=a_type, b_order=b_order, alpha=1.5, beta=0.5, act=W.ACT_RELU,
                      has_c=True, has_bias=True, seed=M + 2 * N + K, dist_a="int3",
                      dist_b="int3", dist_c="int3", dist_bias="eighths")
    case.lda += 1
    case.ldc += 3
    case.ldd += 5
    assert G.variant(case) == "gemm_general_128x128"
    inp = W.gemm_inputs(case)
    D = G.run_gemm(case, inp, sentinel=SENT[a_type])
    assert G.padding_untouched(case, D, SENT[a_type])
    want = W.encode(G.oracle_ref(case, inp), a_type).reshape(M, N)
    assert np.array_equal(W.d_logical(case, D), want)


@pytest.mark.parametrize("variant", [0, 1, 3])
@pytest.mark.parametrize("a_type", [W.F16, W.BF16])
@pytest.mark.parametrize("K,pad", [(8, 0), (72, 8), (200, 0), (1000, 24)])
def test_fast_kernels_ragged_k_bit_exact(K, pad, a_type, variant):
    """16-bit K a multiple of 8 but not of the 64-element slab, on the
    direct-copy kernels: the last k-tile's chunks past K read zeros through
    the buffer range check.  With pad > 0 those chunks are the NaN-filled
    pitch padding, with pad = 0 the next row's data; either would show in D."""
    M, N = 300, 520
    case = W.GemmCase(name="ragged_k", M=M, N=N, K=K, a_type=a_type, b_type=a_type,
                      d_type=a_type, alpha=1.5, beta=0.5, act=W.ACT_RELU, has_c=True,
                      has_bias=True, seed=K + variant, dist_a="int3", dist_b="int3",
                      dist_c="int3", dist_bias="eighths")
    case.lda += pad
    case.ldb += pad
    assert G.variant(case) in ("gemm_fast_128x128", "gemm_pingpong_256x256")
    inp = W.gemm_inputs(case)
    D = G.run_gemm(case, inp, sentinel=SENT[a_type], variant=variant)
    assert G.padding_untouched(case, D, SENT[a_type])
    want = W.encode(G.oracle_ref(case, inp), a_type).reshape(M, N)
    assert np.array_equal(W.d_logical(case, D), want)


@pytest.mark.parametrize("variant", [0, 1])
@pytest.mark.parametrize("K", [8, 200, 1000])
def test_row_major_b_ragged_k_bit_exact(K, variant):
    """N-contiguous B with K a multiple of 8 but not of 64: B's rows past K
    lie past its record count, A's chunks past K read from past every
    record."""
    M, N = 300, 520
    case = W.GemmCase(name="ragged_k_nn", M=M, N=N, K=K, a_type=W.BF16, b_type=W.BF16,
                      d_type=W.BF16, b_order=W.ROW, alpha=1.5, beta=0.5, act=W.ACT_RELU,
                      has_c=True, has_bias=True, seed=K + 7 * variant, dist_a="int3",
                      dist_b="int3", dist_c="int3", dist_bias="eighths")
    case.lda += 8
    case.ldb += 16
    assert G.variant(case) == "gemm_fast_128x128"
    inp = W.gemm_inputs(case)
    D = G.run_gemm(case, inp, sentinel=SENT[W.BF16], variant=variant)
    assert G.padding_untouched(case, D, SENT[W.BF16])
    want = W.encode(G.oracle_ref(case, inp), W.BF16).reshape(M, N)
    assert np.array_equal(W.d_logical(case, D), want)


@pytest.mark.parametrize("M,N,K", [(300, 520, 144), (4096, 2048, 80)])
def test_e4m3_ragged_k_two_group_bit_exact(M, N, K):
    """e4m3 with K a multiple of 16 but not of the 128-element slab: the
    two-group kernel (chosen from 128 tiles of 256 x 256, forced below) reads
    zeros past K through its range-checked copies; the pitches carry NaN
    padding right past K."""
    case = W.GemmCase(name="e4_ragged_k", M=M, N=N, K=K, a_type=W.E4M3, b_type=W.E4M3,
                      d_type=W.BF16, alpha=1.5, beta=0.5, act=W.ACT_RELU, has_c=True,
                      has_bias=True, seed=K + M, dist_a="int3", dist_b="int3",
                      dist_c="int3", dist_bias="eighths")
    case.lda += 16
    case.ldb += 16
    big = (M // 256) * (N // 256) >= 128
    assert G.variant(case) == ("gemm_pingpong_256x256" if big else "gemm_general_128x128")
    inp = W.gemm_inputs(case)
    D = G.run_gemm(case, inp, sentinel=SENT[W.BF16], variant=None if big else 0)
    assert G.padding_untouched(case, D, SENT[W.BF16])
    want = W.encode(G.oracle_ref(case, inp), W.BF16).reshape(M, N)
    assert np.array_equal(W.d_logical(case, D), want)


def test_ragged_k_random_4096_auto():
    """bf16 4096 x 4096 x 4000 (K ends inside the last 64-element slab) on
    the automatically chosen two-group kernel, random inputs, sampled
    against the oracle."""
    case = _small(M=4096, N=4096, K=4000, act=W.ACT_RELU, seed=23)
    assert G.variant(case) == "gemm_pingpong_256x256"
    _check_sampled(case, W.gemm_inputs(case), seed=5)


def test_c_aliases_d():
    case = _small(M=200, N=136, K=64)
    inp = W.gemm_inputs(case)
    D = G.run_gemm(case, inp, d_is_c=True)
    got = _logical(case, D)
    ok, worst = og.within_tolerance(got, G.oracle_ref(case, inp), case.tol)
    assert ok, worst


@pytest.mark.parametrize("c_order,d_order", [(W.COL, W.ROW), (W.ROW, W.COL), (W.COL, W.COL)])
def test_column_major_c_and_d(c_order, d_order):
    case = _small(c_order=c_order, d_order=d_order)
    case.ldc = case.M if c_order == W.COL else case.N
    case.ldd = (case.M if d_order == W.COL else case.N) + 2
    _check_full(case, W.gemm_inputs(case))


def test_fp32_c_and_bias():
    case = _small(M=256, N=256, K=128, c_type=W.F32, bias_type=W.F32, act=W.ACT_NONE)
    _check_full(case, W.gemm_inputs(case))


def test_beta_zero_without_c():
    case = _small(beta=0.0, has_c=False)
    _check_full(case, W.gemm_inputs(case))


def test_repeatable():
    case = _small(M=512, N=512, K=512, act=W.ACT_NONE)
    inp = W.gemm_inputs(case)
    assert np.array_equal(G.run_gemm(case, inp), G.run_gemm(case, inp))


# ----------------------------------------------- pitched operands at scale

def test_fast_path_pitched_at_scale():
    """4096 x 4096 x 1024 bf16 with every pitch past its extent (NaN in the
    operand padding, a sentinel in D's): the 256x256 fast kernel and the
    whole-row LDS epilogue read and write through the pitch."""
    case = _small(M=4096, N=4096, K=1024, act=W.ACT_RELU, seed=21)
    case.lda, case.ldb, case.ldc, case.ldd = 1024 + 64, 1024 + 8, 4096 + 8, 4096 + 24
    assert G.variant(case) == "gemm_pingpong_256x256"
    _check_sampled(case, W.gemm_inputs(case), seed=3)


def test_general_path_pitched_at_scale():
    """3000 x 2500 x 700 fp16, B row-major (N contiguous), odd
    pitches everywhere: the register-staged general path at scale."""
    case = _small(M=3000, N=2500, K=700, a_type=W.F16, b_type=W.F16, d_type=W.F16,
                  b_order=W.ROW, act=W.ACT_GELU, seed=22)
    case.lda, case.ldb, case.ldc, case.ldd = 700 + 3, 2500 + 5, 2500 + 1, 2500 + 7
    assert G.variant(case) == "gemm_general_128x128"
    _check_sampled(case, W.gemm_inputs(case), seed=4)


# ------------------------------------------------- tile-configuration dispatch

@pytest.mark.parametrize("variant", [0, 1, 2, 3])
@pytest.mark.parametrize("a_type,d_type", [(W.BF16, W.BF16), (W.F16, W.F16), (W.E4M3, W.BF16)])
def test_forced_variants_bit_exact(variant, a_type, d_type):
    """Every compiled variant, forced through tla_gemm_run_variant on the
    same integer-valued problem (exact in fp32), gives D bit for bit; the
    M/N extents are ragged for all three tilings."""
    M, N, K = 300, 520, 384
    case = W.GemmCase(name="forced", M=M, N=N, K=K, a_type=a_type, b_type=a_type,
                      d_type=d_type, alpha=1.5, beta=0.5, act=W.ACT_RELU, has_c=True,
                      has_bias=True, seed=91, dist_a="int3", dist_b="int3", dist_c="int3",
                      dist_bias="eighths")
    inp = W.gemm_inputs(case)
    D = G.run_gemm(case, inp, sentinel=SENT[d_type], variant=variant)
    assert G.padding_untouched(case, D, SENT[d_type])
    want = W.encode(G.oracle_ref(case, inp), d_type).reshape(M, N)
    assert np.array_equal(W.d_logical(case, D), want)


@pytest.mark.parametrize("variant", [0, 1, 2, 3])
def test_forced_variants_random_inputs(variant):
    case = _small(M=640, N=768, K=512, act=W.ACT_GELU, seed=92)
    _check_full(case, W.gemm_inputs(case), variant=variant)


def _ulp(v, d_type):
    """Spacing of D's type at |v| (the least subnormal at 0)."""
    v = np.abs(v)
    if d_type == W.F16:
        return np.spacing(v.astype(np.float16)).astype(np.float64)
    _, e = np.frexp(np.maximum(v, 2.0 ** -126))
    return np.ldexp(1.0, e - 8)


@pytest.mark.parametrize("variant", [0, 1, 2, 3])
@pytest.mark.parametrize("d_type,c_type", [(W.BF16, W.BF16), (W.F16, W.F16), (W.BF16, W.F32)])
def test_gelu_activation_accuracy(variant, d_type, c_type):
    """D = GELU(C) (A = 0, beta = 1) over y in [-9, 9] on every variant and
    both epilogue forms (16-bit C through the tile epilogue, fp32 C through
    the per-group one): within half an output ulp of the exact y * Phi(y)
    plus 4e-7 (1 + |y|) of fp32 evaluation error."""
    M, N, K = 512, 512, 128
    a_type = W.F16 if d_type == W.F16 else W.BF16
    case = W.GemmCase(name="gelu", M=M, N=N, K=K, a_type=a_type, b_type=a_type, d_type=d_type,
                      c_type=c_type, alpha=1.0, beta=1.0, act=W.ACT_GELU, has_c=True, seed=93)
    inp = W.gemm_inputs(case)
    inp["A"] = np.zeros_like(inp["A"])
    inp["B"] = np.zeros_like(inp["B"])
    inp["C"] = W.encode(np.linspace(-9.0, 9.0, M * N), c_type).reshape(-1)
    y = og.decode(c_type, inp["C"].copy()).reshape(M, N)
    D = G.run_gemm(case, inp, sentinel=SENT[d_type], variant=variant)
    got = _logical(case, D)
    ref = G.oracle_ref(case, inp)
    bound = 0.5 * _ulp(np.maximum(np.abs(got), np.abs(ref)), d_type) + 4e-7 * (1 + np.abs(y))
    err = np.abs(got - ref)
    assert not np.isnan(got).any()
    assert (err <= bound).all(), "worst excess %g at y = %g" % (
        (err - bound).max(), y.flat[np.argmax(err - bound)])


def test_forced_fast_variant_refuses_general_layout():
    import tiled_layout_algebra_amd as tla
    case = _small(b_order=W.ROW)  # B N-contiguous: no fast layout
    for variant in (0, 1, 3):
        with pytest.raises(tla.TlaError) as e:
            G.run_gemm(case, W.gemm_inputs(case), sentinel=SENT[case.d_type], variant=variant)
        assert e.value.status == tla.ERR_UNSUPPORTED


def test_variant_info_reports_the_compiled_kernels():
    import tiled_layout_algebra_amd as tla
    for a_type in (W.BF16, W.F16, W.E4M3):
        infos = [tla.gemm_variant_info(v, a_type) for v in range(tla.GEMM_VARIANTS)]
        assert [i["name"] for i in infos] == ["gemm_pingpong_256x256", "gemm_fast_128x128",
                                              "gemm_general_128x128", "gemm_fast_256x256"]
        assert infos[0]["threads"] == 512 and infos[0]["blocks_per_cu"] == 1
        for i in infos:
            assert i["threads"] in (256, 512) and i["lds_bytes"] > 0 and i["blocks_per_cu"] >= 1
            assert i["lds_bytes"] * i["blocks_per_cu"] <= 160 * 1024
        assert infos[0]["block_m"] == 256 and infos[2]["block_n"] == 128
        assert infos[3]["block_m"] == 256


# ------------------------------------------------- two-group 256x256 kernel

@pytest.mark.parametrize("k_tiles", [1, 2, 3, 4])
@pytest.mark.parametrize("a_type,d_type", [(W.BF16, W.BF16), (W.F16, W.F16), (W.E4M3, W.BF16)])
def test_pingpong_few_k_tiles_bit_exact(k_tiles, a_type, d_type):
    """The two-group kernel's prologue and last phases: 1 to 4 k-tiles of
    128 bytes, ragged M and N (the last row block ends inside a 32-row copy
    block), integer inputs (exact in fp32), forced variant 0."""
    K = k_tiles * 128 // W.ITEMSIZE[a_type]
    M, N = 300, 520
    case = W.GemmCase(name="pp_k", M=M, N=N, K=K, a_type=a_type, b_type=a_type, d_type=d_type,
                      alpha=1.5, beta=0.5, act=W.ACT_RELU, has_c=True, has_bias=True,
                      seed=400 + k_tiles, dist_a="int3", dist_b="int3", dist_c="int3",
                      dist_bias="eighths")
    inp = W.gemm_inputs(case)
    D = G.run_gemm(case, inp, sentinel=SENT[d_type], variant=0)
    assert G.padding_untouched(case, D, SENT[d_type])
    want = W.encode(G.oracle_ref(case, inp), d_type).reshape(M, N)
    assert np.array_equal(W.d_logical(case, D), want)


def test_pingpong_e4m3_ragged_full():
    """e4m3 on the two-group kernel with both extents ragged and a pitched D
    (13 x 11 tiles of 256; rows and columns end mid-tile), every output
    against the oracle within 5e-2 (1 + |ref|)."""
    case = dataclasses.replace(W.GEMM_E4M3_8192, M=3100, N=2600, K=1024, lda=0, ldb=0, ldc=0,
                               ldd=0)
    case.__post_init__()
    case.ldd += 24
    assert G.variant(case) == "gemm_pingpong_256x256"
    _check_full(case, W.gemm_inputs(case))
