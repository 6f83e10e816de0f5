"""Pitched 2-D copy parity (the identity-layout case of the layout-driven
copy): the HIP path through the C ABI against the oracle's copy, bit for
bit -- ragged and pitched shapes for every element size, misaligned bases
(element-wise path), the full 16384 x 16384 fp32 workload, destination
padding left untouched."""
import numpy as np
import pytest
import torch

import tiled_layout_algebra_amd as tla
import workloads as W
from oracle import gemm as og
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

_DT = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}
SENT = 0xA5


def _src(case):
    if case.elem_bytes == 16:  # two random 8-byte halves per element
        half = W.TransposeCase(name=case.name, M=case.M, N=2 * case.N, ld_src=2 * case.ld_src,
                               elem_bytes=8, seed=case.seed)
        return W.transpose_input(half)
    return W.transpose_input(case)


def _check(case, pad_front=0):
    eb = case.elem_bytes
    dt = _DT[min(eb, 8)]
    per = eb // np.dtype(dt).itemsize
    src = _src(case)
    n_dst = (case.M - 1) * case.ld_dst + case.N
    dst0 = np.full(n_dst * per, np.array(SENT * 0x0101010101010101 & np.iinfo(dt).max, dtype=dt))
    s, d = G.to_dev(src, pad_front), G.to_dev(dst0, pad_front)
    tla.tiled_copy(s, case.ld_src, d, case.ld_dst, case.M, case.N, eb)
    torch.cuda.synchronize()
    got = G.to_host(d, np.dtype(dt))
    vt = np.dtype((np.void, eb))
    want = dst0.copy().view(vt)
    og.copy2d(np.ascontiguousarray(src).view(vt), case.M, case.N, case.ld_src, case.ld_dst,
              dst=want)
    assert np.array_equal(got, want.view(dt))  # bits, and the padding kept


SHAPES = [(1, 1, 0, 0), (3, 5, 0, 0), (33, 65, 0, 0), (100, 37, 3, 1), (64, 256, 0, 0),
          (260, 516, 0, 0), (64, 48, 4, 8), (129, 1031, 7, 5)]


@pytest.mark.parametrize("eb", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("M,N,ps,pd", SHAPES)
def test_copy_bit_exact(M, N, ps, pd, eb):
    _check(W.TransposeCase(name="c", M=M, N=N, ld_src=N + ps, ld_dst=N + pd, elem_bytes=eb,
                           seed=M * 17 + N))


@pytest.mark.parametrize("eb", [2, 4, 8])
def test_copy_misaligned_bases(eb):
    # one element in front: rows are no longer 16-byte aligned
    _check(W.TransposeCase(name="c", M=70, N=260, ld_src=260, ld_dst=264, elem_bytes=eb,
                           seed=3), pad_front=1)


@pytest.mark.parametrize("eb,pad_front", [(4, 0), (4, 1)])
def test_copy_more_rows_than_one_grid_column(eb, pad_front):
    """131075 rows: the rows go out in launches of at most 65535 (the grid's
    y limit), with the 16-byte path and the element-wise one."""
    _check(W.TransposeCase(name="c", M=131075, N=12, ld_src=16, ld_dst=20, elem_bytes=eb,
                           seed=5), pad_front=pad_front)


def test_copy_full_size_fp32_bits():
    tc = W.TRANSPOSE_F32_16384
    case = W.TransposeCase(name="copy", M=tc.M, N=tc.N, ld_src=tc.N, ld_dst=tc.N, seed=tc.seed)
    src = W.transpose_input(case)
    s = G.to_dev(src)
    d = torch.empty_like(s)
    tla.tiled_copy(s, case.N, d, case.N, case.M, case.N, 4)
    torch.cuda.synchronize()
    assert np.array_equal(G.to_host(d, np.dtype(np.uint32)), src)


def test_copy_argument_errors():
    x = torch.zeros(64, dtype=torch.int32, device="cuda")
    with pytest.raises(tla.TlaError) as e:
        tla.tiled_copy(x, 8, x[4:], 8, 4, 8, 4)     # overlapping ranges
    assert e.value.status == tla.ERR_OVERLAP
    with pytest.raises(tla.TlaError):
        tla.tiled_copy(x, 4, x, 8, 2, 8, 4)         # ld_src < N
