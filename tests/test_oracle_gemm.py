"""Pins of the GEMM + epilogue oracle and the transpose oracle: textbook
routines (numpy.matmul in float64, scipy's normal CDF), special cases,
exact invariants of the epilogue terms, and bit identities of the
transpose.  CPU only."""
import itertools

import numpy as np
import pytest
from scipy.special import ndtr

import workloads as W
from oracle import gemm as og


def _logical(bits, dtype, rows, cols, order, ld):
    vals = og.decode(dtype, bits)
    if order == W.ROW:
        return vals.reshape(rows, ld)[:, :cols]
    return vals.reshape(cols, ld)[:, :rows].T


def _case(M, N, K, a_order, b_order, dtype=W.F16, pad=3, seed=0, **kw):
    lda = (K if a_order == W.ROW else M) + pad
    ldb = (N if b_order == W.ROW else K) + pad
    return W.GemmCase(name="t", M=M, N=N, K=K, a_type=dtype, b_type=dtype, d_type=W.F16,
                      a_order=a_order, b_order=b_order, lda=lda, ldb=ldb,
                      ldc=N + pad, seed=seed, **kw)


def _run(case, inp, nthreads=None, **over):
    p = dict(M=case.M, N=case.N, K=case.K, A=inp["A"], a_type=case.a_type,
             a_order=case.a_order, lda=case.lda, B=inp["B"], b_type=case.b_type,
             b_order=case.b_order, ldb=case.ldb, C=inp["C"], c_type=case.c_type,
             c_order=case.c_order, ldc=case.ldc, bias=inp["bias"], bias_type=case.bias_type,
             alpha=case.alpha, beta=case.beta, scale_a=case.scale_a, scale_b=case.scale_b,
             act=case.act, nthreads=nthreads)
    p.update(over)
    return og.gemm(**p)


@pytest.mark.parametrize("a_order,b_order", list(itertools.product([W.ROW, W.COL], repeat=2)))
@pytest.mark.parametrize("dtype", [W.F16, W.BF16, W.E4M3])
def test_oracle_equals_numpy_matmul(a_order, b_order, dtype):
    # alpha=1, beta=0, no bias/act reduces the oracle to a plain matmul; the
    # padding is NaN, so reading it would poison the result
    case = _case(37, 29, 53, a_order, b_order, dtype=dtype, seed=dtype * 10 + a_order * 2 + b_order)
    inp = W.gemm_inputs(case)
    ref = _run(case, inp)
    A = _logical(inp["A"], dtype, case.M, case.K, a_order, case.lda)
    B = _logical(inp["B"], dtype, case.K, case.N, b_order, case.ldb)
    want = np.matmul(A, B)
    assert np.all(np.isfinite(ref))
    np.testing.assert_allclose(ref, want, rtol=1e-12, atol=1e-12)


def test_oracle_c_column_major_and_transposed_roles():
    # C stored column-major is read as C(m, n), not C(n, m)
    case = _case(9, 13, 5, W.ROW, W.COL, has_c=True, beta=1.0)
    case.c_order, case.ldc = W.COL, case.M + 2
    inp = W.gemm_inputs(case)
    ref = _run(case, inp)
    A = _logical(inp["A"], W.F16, case.M, case.K, W.ROW, case.lda)
    B = _logical(inp["B"], W.F16, case.K, case.N, W.COL, case.ldb)
    C = _logical(inp["C"], W.F16, case.M, case.N, W.COL, case.ldc)
    np.testing.assert_allclose(ref, A @ B + C, rtol=1e-12, atol=1e-12)


def test_epilogue_terms_are_exact_increments():
    case = _case(17, 11, 19, W.ROW, W.COL, has_c=True, has_bias=True, beta=0.5)
    inp = W.gemm_inputs(case)
    base = _run(case, inp, C=None, beta=0.0, bias=None)
    C = _logical(inp["C"], W.F16, case.M, case.N, W.ROW, case.ldc)
    bias = og.decode(W.F16, inp["bias"])
    # alpha scales by an exact power of two
    assert np.array_equal(_run(case, inp, C=None, beta=0.0, bias=None, alpha=2.0), 2.0 * base)
    # scale_a * scale_b fold into alpha (0.5 * 4 = 2)
    assert np.array_equal(_run(case, inp, C=None, beta=0.0, bias=None, scale_a=0.5, scale_b=4.0),
                          2.0 * base)
    # beta*C adds exactly beta*C(m,n)
    with_c = _run(case, inp, bias=None, beta=0.5)
    np.testing.assert_array_equal(with_c - base, (base + 0.5 * C) - base)
    # bias adds bias[n] to every row
    with_b = _run(case, inp, C=None, beta=0.0)
    np.testing.assert_array_equal(with_b, base + bias[None, :])
    # beta == 0 never reads C (NaN C must not leak)
    nan_c = np.full_like(inp["C"], W.NAN_BITS[W.F16])
    assert np.array_equal(_run(case, inp, C=nan_c, beta=0.0, bias=None), base)


def test_k_zero_is_beta_c_plus_bias():
    case = _case(7, 9, 0, W.ROW, W.COL, has_c=True, has_bias=True, beta=1.5, act=W.ACT_RELU)
    case.lda, case.ldb = 1, 1
    inp = W.gemm_inputs(case)
    inp["A"], inp["B"] = None, None
    ref = _run(case, inp)
    C = _logical(inp["C"], W.F16, case.M, case.N, W.ROW, case.ldc)
    bias = og.decode(W.F16, inp["bias"])
    assert np.array_equal(ref, np.maximum(1.5 * C + bias[None, :], 0.0))


def test_relu_and_gelu_against_library():
    case = _case(23, 31, 41, W.ROW, W.COL, seed=9)
    inp = W.gemm_inputs(case)
    none = _run(case, inp, act=W.ACT_NONE)
    assert (none < 0).any() and (none > 0).any()
    assert np.array_equal(_run(case, inp, act=W.ACT_RELU), np.where(none > 0, none, 0.0))
    gelu = _run(case, inp, act=W.ACT_GELU)
    np.testing.assert_allclose(gelu, none * ndtr(none), rtol=1e-13, atol=1e-15)


def test_gelu_identities():
    # GELU(0) = 0, GELU(x) - GELU(-x) = x, GELU -> x at +inf and -> 0 at -inf,
    # checked through 1x1x1 GEMMs with A = x, B = 1
    xs = np.array([0.0, 0.25, 1.0, 2.5, 7.0, 40.0])
    for x in xs:
        def g(v):
            A = W.encode(np.array([[v]]), W.F32).reshape(-1)
            B = W.encode(np.array([[1.0]]), W.F32).reshape(-1)
            return og.gemm(1, 1, 1, A, W.F32, W.ROW, 1, B, W.F32, W.ROW, 1, act=W.ACT_GELU)[0, 0]
        xv = float(np.float32(x))
        assert abs((g(xv) - g(-xv)) - xv) <= 1e-15 * max(1.0, xv)
        if x == 0:
            assert g(0.0) == 0.0
        if x >= 7.0:
            assert abs(g(xv) - xv) < 1e-10 * xv and abs(g(-xv)) < 1e-10


def test_points_and_thread_count_agree_with_full():
    case = _case(45, 38, 29, W.ROW, W.ROW, has_c=True, has_bias=True, beta=0.5,
                 act=W.ACT_GELU, alpha=1.5)
    inp = W.gemm_inputs(case)
    full1 = _run(case, inp, nthreads=1)
    full8 = _run(case, inp, nthreads=8)
    assert np.array_equal(full1, full8)
    rng = np.random.default_rng(0)
    ms = rng.integers(0, case.M, 300)
    ns = rng.integers(0, case.N, 300)
    pts = og.gemm_points(ms, ns, case.M, case.N, case.K, inp["A"], case.a_type, case.a_order,
                         case.lda, inp["B"], case.b_type, case.b_order, case.ldb, C=inp["C"],
                         c_type=case.c_type, c_order=case.c_order, ldc=case.ldc,
                         bias=inp["bias"], bias_type=case.bias_type, alpha=case.alpha,
                         beta=case.beta, act=case.act)
    assert np.array_equal(pts, full1[ms, ns])


def test_integer_inputs_give_exact_sums():
    # integer operands in [-3,3]: the binary64 sum is the exact integer
    case = _case(13, 17, 65, W.COL, W.ROW, dtype=W.E4M3)
    case.dist_a = case.dist_b = "int3"
    inp = W.gemm_inputs(case)
    ref = _run(case, inp)
    A = _logical(inp["A"], W.E4M3, case.M, case.K, W.COL, case.lda).astype(np.int64)
    B = _logical(inp["B"], W.E4M3, case.K, case.N, W.ROW, case.ldb).astype(np.int64)
    assert np.array_equal(ref, (A @ B).astype(np.float64))


def test_bad_arguments_are_rejected():
    A = np.zeros(4, np.uint16)
    with pytest.raises(ValueError):
        og.gemm(2, 2, 2, A, W.F16, W.ROW, 2, A, W.F16, W.ROW, 2, beta=1.0)  # C missing
    with pytest.raises(ValueError):
        og.gemm(-1, 2, 2, A, W.F16, W.ROW, 2, A, W.F16, W.ROW, 2)


# ------------------------------------------------------------ transpose (P9)

@pytest.mark.parametrize("M,N,pad_s,pad_d", [(1, 1, 0, 0), (33, 65, 0, 0), (64, 48, 3, 5), (5, 1, 1, 0)])
@pytest.mark.parametrize("eb", [1, 2, 4, 8])
def test_transpose_oracle(M, N, pad_s, pad_d, eb):
    case = W.TransposeCase(name="t", M=M, N=N, ld_src=N + pad_s, ld_dst=M + pad_d,
                           elem_bytes=eb, seed=M * 7 + N)
    src = W.transpose_input(case)
    dst = og.transpose(src, M, N, case.ld_src, case.ld_dst)
    S = src.reshape(M, case.ld_src)[:, :N]
    D = dst.reshape(N, case.ld_dst)[:, :M]
    assert np.array_equal(D, S.T)       # numpy's transpose, bit for bit
    assert (dst.reshape(N, case.ld_dst)[:, M:] == 0).all()  # padding untouched
    # applying the transpose to the result gives back the source
    back = og.transpose(dst, N, M, case.ld_dst, case.ld_src)
    assert np.array_equal(back.reshape(M, case.ld_src)[:, :N], S)
    assert np.array_equal(np.sort(D, axis=None), np.sort(S, axis=None))


def test_transpose_keeps_nan_payloads_and_subnormals():
    src = np.array([0x7FC00001, 0x7F800001, 0xFFFFFFFF, 0x00000001, 0x80000001, 0x007FFFFF],
                   dtype=np.uint32)
    dst = og.transpose(src, 2, 3, 3, 2)
    assert np.array_equal(dst, src.reshape(2, 3).T.reshape(-1))


# --------------------------------------------------- pitched 2-D copy (P9)

@pytest.mark.parametrize("M,N,pad_s,pad_d", [(1, 1, 0, 0), (33, 65, 0, 0), (64, 48, 3, 5), (5, 1, 1, 0)])
@pytest.mark.parametrize("eb", [1, 2, 4, 8])
def test_copy2d_oracle(M, N, pad_s, pad_d, eb):
    case = W.TransposeCase(name="c", M=M, N=N, ld_src=N + pad_s, ld_dst=N + pad_d,
                           elem_bytes=eb, seed=M * 5 + N)
    src = W.transpose_input(case)
    dst = og.copy2d(src, M, N, case.ld_src, case.ld_dst)
    S = src.reshape(M, case.ld_src)[:, :N]
    D = dst.reshape(M, case.ld_dst)
    assert np.array_equal(D[:, :N], S)               # numpy slicing, bit for bit
    assert (D[:, N:] == 0).all()                     # padding untouched
    # the copy is the identity layout's case of the transpose: transposing
    # twice through the oracle gives the same bits
    t = og.transpose(src, M, N, case.ld_src, M)
    tt = og.transpose(t, N, M, M, case.ld_dst)
    assert np.array_equal(tt.reshape(M, case.ld_dst)[:, :N], D[:, :N])


def test_copy2d_rejects_bad_pitch():
    with pytest.raises(ValueError):
        og.copy2d(np.zeros(8, np.uint32), 2, 4, 4, 3)
