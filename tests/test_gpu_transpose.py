"""Transpose parity: the HIP path through the C ABI against the oracle's
bit-copy transpose, bit for bit -- small, ragged and pitched shapes for
every element size, the full 16384 x 16384 fp32 workload, destination
padding left untouched, and run-to-run determinism."""
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


def _run(case, src_bits, pad_front=0):
    eb = case.elem_bytes
    dt = _DT[min(eb, 8)]
    per = eb // np.dtype(dt).itemsize
    n_dst = (case.N - 1) * case.ld_dst + case.M if case.M and case.N else 0
    dst0 = np.full(max(n_dst, 1) * per, np.array(SENT * 0x0101010101010101 & np.iinfo(dt).max, dtype=dt))
    s = G.to_dev(src_bits, pad_front)
    d = G.to_dev(dst0, pad_front)
    tla.tiled_transpose(s, case.ld_src, d, case.ld_dst, case.M, case.N, eb)
    torch.cuda.synchronize()
    return G.to_host(d, np.dtype(dt)), dst0


def _oracle(case, src_bits, dst0):
    eb = case.elem_bytes
    vt = np.dtype((np.void, eb))
    src = np.ascontiguousarray(src_bits).view(vt)
    dst = dst0.copy().view(vt)
    og.transpose(src, case.M, case.N, case.ld_src, case.ld_dst, dst=dst)
    return dst.view(dst0.dtype)


SHAPES = [(1, 1, 0, 0), (3, 5, 0, 0), (32, 32, 0, 0), (33, 65, 0, 0), (100, 37, 3, 1),
          (64, 64, 0, 0), (128, 256, 0, 0), (256, 1024, 0, 0), (260, 516, 0, 0),
          (64, 48, 4, 8), (63, 64, 0, 0), (129, 131, 7, 5), (4, 4, 0, 0), (256, 64, 0, 0),
          (516, 260, 0, 0), (300, 68, 8, 4), (1028, 196, 4, 12)]


@pytest.mark.parametrize("eb", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("M,N,ps,pd", SHAPES)
def test_transpose_bit_exact(M, N, ps, pd, eb):
    case = W.TransposeCase(name="t", M=M, N=N, ld_src=N + ps, ld_dst=M + pd, elem_bytes=eb,
                           seed=M * 131 + N)
    src = _src(case)
    got, dst0 = _run(case, src)
    want = _oracle(case, src, dst0)
    assert np.array_equal(got, want)   # includes the untouched destination padding


def test_transpose_misaligned_rows_use_general_path():
    case = W.TransposeCase(name="t", M=64, N=64, ld_src=66, ld_dst=65, elem_bytes=4, seed=9)
    src = _src(case)
    got, dst0 = _run(case, src, pad_front=1)
    assert np.array_equal(got, _oracle(case, src, dst0))


def test_transpose_full_size_fp32_bits():
    case = W.TRANSPOSE_F32_16384
    src = W.transpose_input(case)
    s = G.to_dev(src)
    d = torch.empty_like(s)
    tla.tiled_transpose(s, case.ld_src, d, case.ld_dst, case.M, case.N, 4)
    torch.cuda.synchronize()
    got = G.to_host(d, np.dtype(np.uint32))
    want = og.transpose(src, case.M, case.N, case.ld_src, case.ld_dst)
    assert np.array_equal(got, want)
    # NaN payloads and subnormals survive: count both kinds in the result
    exp = (got >> 23) & 0xFF
    assert ((exp == 0xFF) & ((got & 0x7FFFFF) != 0)).sum() > 0
    assert ((exp == 0) & ((got & 0x7FFFFF) != 0)).sum() > 0
    # twice is the identity; same result on a second run
    d2 = torch.empty_like(s)
    tla.tiled_transpose(d, case.ld_dst, d2, case.ld_src, case.N, case.M, 4)
    d3 = torch.empty_like(s)
    tla.tiled_transpose(s, case.ld_src, d3, case.ld_dst, case.M, case.N, 4)
    torch.cuda.synchronize()
    assert torch.equal(d2, s)
    assert torch.equal(d3, d)


@pytest.mark.parametrize("ps,pd,eb", [(4, 12, 4), (3, 5, 4), (8, 16, 2)])
def test_transpose_pitched_at_scale(ps, pd, eb):
    """8192 x 4096 with row pitches past the extents (the pitch taken from the
    layout, walk-through section 6.3): 16-byte aligned pitches take the fast
    path, odd ones the general one; every element and every padding element
    of the destination is compared."""
    case = W.TransposeCase(name="t", M=8192, N=4096, ld_src=4096 + ps, ld_dst=8192 + pd,
                           elem_bytes=eb, seed=77 + ps)
    src = _src(case)
    got, dst0 = _run(case, src)
    assert np.array_equal(got, _oracle(case, src, dst0))
