"""Pins of the oracle's storage-format decoders: every code of fp16, bf16
and e4m3 against the closed form of the format and against the library
conversions (numpy float16, torch bfloat16 / float8_e4m3fn).  CPU only."""
import math

import numpy as np
import pytest
import torch

from oracle import gemm as og


def _closed_form(code, ebits, mbits, bias, has_inf):
    s = -1.0 if (code >> (ebits + mbits)) & 1 else 1.0
    e = (code >> mbits) & ((1 << ebits) - 1)
    f = code & ((1 << mbits) - 1)
    emax = (1 << ebits) - 1
    if e == emax and has_inf:
        return s * math.inf if f == 0 else math.nan
    if e == 0:
        return s * f * 2.0 ** (1 - bias - mbits)
    return s * (1.0 + f / 2.0 ** mbits) * 2.0 ** (e - bias)


def _same(a, b):
    return (math.isnan(a) and math.isnan(b)) or a == b


def test_fp16_all_codes():
    codes = np.arange(1 << 16, dtype=np.uint16)
    got = og.decode(og.F16, codes)
    lib = codes.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(lib))
    ok = ~np.isnan(lib)
    assert np.array_equal(got[ok], lib[ok])
    for c in [0x0000, 0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0x7C00, 0xFC00, 0x8001, 0xC000]:
        assert _same(got[c], _closed_form(c, 5, 10, 15, True))
    assert got[0x3C00] == 1.0 and got[0x7BFF] == 65504.0 and got[0x0001] == 2.0 ** -24


def test_bf16_all_codes():
    codes = np.arange(1 << 16, dtype=np.uint16)
    got = og.decode(og.BF16, codes)
    lib = torch.from_numpy(codes.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(lib))
    ok = ~np.isnan(lib)
    assert np.array_equal(got[ok], lib[ok])
    for c in [0x0001, 0x007F, 0x0080, 0x3F80, 0x7F7F, 0x7F80, 0xFF80, 0xBF80]:
        assert _same(got[c], _closed_form(c, 8, 7, 127, True))
    # subnormals are kept, not flushed
    assert got[0x0001] == 2.0 ** -133


def test_e4m3_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    got = og.decode(og.E4M3, codes)
    lib = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(lib))
    ok = ~np.isnan(lib)
    assert np.array_equal(got[ok], lib[ok])
    # OCP E4M3FN: no infinity, only S.1111.111 is NaN, max 448, min subnormal 2^-9
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert np.isnan(got).sum() == 2
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0
    assert got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6
    for c in range(256):
        if c & 0x7F != 0x7F:
            assert got[c] == _closed_form(c, 4, 3, 7, False)


def test_fp32_decoder_sample():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 1 << 32, size=200000, dtype=np.uint64).astype(np.uint32)
    codes[:6] = [0, 1, 0x007FFFFF, 0x00800000, 0x7F800000, 0xFF800000]
    got = og.decode(og.F32, codes)
    lib = codes.view(np.float32).astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(lib))
    ok = ~np.isnan(lib)
    assert np.array_equal(got[ok], lib[ok])
    assert got[1] == 2.0 ** -149


@pytest.mark.parametrize("dtype", [og.F16, og.BF16, og.E4M3])
def test_encoder_round_trips(dtype):
    # the input encoder (workloads) rounds to nearest even; decoding what it
    # produced and re-encoding is the identity on finite codes
    import workloads as W
    rng = np.random.default_rng(1)
    x = rng.uniform(-400, 400, size=20000)
    bits = W.encode(x, dtype)
    vals = og.decode(dtype, bits)
    assert np.array_equal(W.encode(vals, dtype), bits)
    # nearest: no other representable value is closer than the decoded one
    grid = np.unique(og.decode(dtype, np.arange(1 << (8 * W.ITEMSIZE[dtype]),
                                                dtype=W.STORAGE[dtype])))
    grid = grid[np.isfinite(grid)]
    x32 = x.astype(np.float32).astype(np.float64)
    pos = np.searchsorted(grid, x32)
    lo = grid[np.clip(pos - 1, 0, len(grid) - 1)]
    hi = grid[np.clip(pos, 0, len(grid) - 1)]
    best = np.minimum(np.abs(x32 - lo), np.abs(x32 - hi))
    assert np.all(np.abs(vals - x32) <= best)
