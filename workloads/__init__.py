"""Seeded synthetic inputs for the GEMM + epilogue, transpose and thread-map
workloads.

This module only draws random numbers and stores them in the operands'
storage formats; it holds none of the GEMM, epilogue or layout arithmetic.
It is the one module both the oracle-side checks and the GPU path read, so
both see exactly the same bits.

Recipe (the same for every workload):
  * generator ``numpy.random.default_rng(seed)`` (PCG64);
  * draw order A, B, C, bias, each drawn as the logical matrix in C order
    (row index slowest) whatever its storage order;
  * values drawn in float64, rounded to float32, then rounded
    round-to-nearest-even into the storage format by library conversions
    (numpy float16; torch bfloat16 and float8_e4m3fn on the CPU);
  * e4m3 values are clamped to [-448, 448] before rounding (the format has
    no infinity);
  * padding between the logical extent and the leading dimension is filled
    with a caller-chosen bit pattern (NaN by default) so that any read of
    it poisons a result.

Storage type codes: 0 fp16, 1 bf16, 2 e4m3 (OCP E4M3FN), 3 fp32.
Orders: 0 row-major, 1 column-major.
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

F16, BF16, E4M3, F32 = 0, 1, 2, 3
ROW, COL = 0, 1
ACT_NONE, ACT_RELU, ACT_GELU = 0, 1, 2

STORAGE = {F16: np.uint16, BF16: np.uint16, E4M3: np.uint8, F32: np.uint32}
ITEMSIZE = {F16: 2, BF16: 2, E4M3: 1, F32: 4}
NAN_BITS = {F16: 0x7E00, BF16: 0x7FC0, E4M3: 0x7F, F32: 0x7FC00000}
DTYPE_NAME = {F16: "f16", BF16: "bf16", E4M3: "e4m3", F32: "f32"}


# --------------------------------------------------------------- encoders

def encode(x: np.ndarray, dtype: int) -> np.ndarray:
    """float64 values -> float32 -> storage bits of ``dtype`` (RNE)."""
    f32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == F32:
        return f32.view(np.uint32)
    if dtype == F16:
        return f32.astype(np.float16).view(np.uint16)
    import torch
    t = torch.from_numpy(np.ascontiguousarray(f32))
    if dtype == BF16:
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype == E4M3:
        t = t.clamp(-448.0, 448.0)
        return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    raise ValueError("unknown dtype %r" % dtype)


def draw(rng: np.random.Generator, shape, dist: str) -> np.ndarray:
    """float64 draws.  ``dist``: 'u1' U[-1,1], 'u01' U[-0.1,0.1],
    'n05' N(0,1)*0.5, 'int3' integers in [-3,3], 'z/<s>' N(0,1)/s,
    'eighths' integers/8 in [-2,2]."""
    if dist == "u1":
        return rng.uniform(-1.0, 1.0, size=shape)
    if dist == "u01":
        return rng.uniform(-0.1, 0.1, size=shape)
    if dist == "n05":
        return rng.standard_normal(size=shape) * 0.5
    if dist == "int3":
        return rng.integers(-3, 4, size=shape).astype(np.float64)
    if dist == "eighths":
        return rng.integers(-16, 17, size=shape).astype(np.float64) / 8.0
    if dist.startswith("z/"):
        return rng.standard_normal(size=shape) / float(dist[2:])
    raise ValueError("unknown distribution %r" % dist)


def storage_len(rows: int, cols: int, order: int, ld: int) -> int:
    """Elements a rows x cols matrix with leading dimension ld occupies."""
    if rows == 0 or cols == 0:
        return 0
    return rows * ld if order == ROW else ld * cols


def place(logical_bits: np.ndarray, order: int, ld: int, dtype: int,
          pad_bits: Optional[int] = None) -> np.ndarray:
    """Store a logical (rows, cols) array of storage bits with leading
    dimension ``ld``; padding gets ``pad_bits`` (NaN pattern by default)."""
    rows, cols = logical_bits.shape
    if pad_bits is None:
        pad_bits = NAN_BITS[dtype]
    n = storage_len(rows, cols, order, ld)
    buf = np.full(n, pad_bits, dtype=STORAGE[dtype])
    if n:
        if order == ROW:
            if ld < cols:
                raise ValueError("ld < cols")
            buf.reshape(rows, ld)[:, :cols] = logical_bits
        else:
            if ld < rows:
                raise ValueError("ld < rows")
            buf.reshape(cols, ld)[:, :rows] = logical_bits.T
    return buf


def matrix(rng, rows, cols, order, ld, dtype, dist, pad_bits=None) -> np.ndarray:
    """Draw, encode and place one operand; returns the flat storage array."""
    vals = draw(rng, (rows, cols), dist)
    bits = encode(vals, dtype).reshape(rows, cols)
    return place(bits, order, ld, dtype, pad_bits)


# -------------------------------------------------------------- GEMM cases

@dataclass
class GemmCase:
    """One GEMM problem: D = act(alpha*sa*sb*A.B + beta*C + bias)."""
    name: str
    M: int
    N: int
    K: int
    a_type: int
    b_type: int
    d_type: int
    a_order: int = ROW
    b_order: int = COL
    c_order: int = ROW
    d_order: int = ROW
    lda: int = 0
    ldb: int = 0
    ldc: int = 0
    ldd: int = 0
    alpha: float = 1.0
    beta: float = 0.0
    scale_a: float = 1.0
    scale_b: float = 1.0
    act: int = ACT_NONE
    has_c: bool = False
    has_bias: bool = False
    seed: int = 0
    dist_a: str = "u1"
    dist_b: str = "u1"
    dist_c: str = "u1"
    dist_bias: str = "u01"
    c_type: int = -1       # defaults to d_type
    bias_type: int = -1    # defaults to d_type
    tol: float = 1e-2
    extra: dict = field(default_factory=dict)

    def __post_init__(self):
        if self.c_type < 0:
            self.c_type = self.d_type
        if self.bias_type < 0:
            self.bias_type = self.d_type
        if not self.lda:
            self.lda = self.K if self.a_order == ROW else self.M
        if not self.ldb:
            self.ldb = self.N if self.b_order == ROW else self.K
        if not self.ldc:
            self.ldc = self.N if self.c_order == ROW else self.M
        if not self.ldd:
            self.ldd = self.N if self.d_order == ROW else self.M

    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K


def gemm_inputs(case: GemmCase, pad_bits=None):
    """Seeded operands of ``case`` as flat storage arrays:
    dict(A=..., B=..., C=... or None, bias=... or None)."""
    rng = np.random.default_rng(case.seed)
    A = matrix(rng, case.M, case.K, case.a_order, case.lda, case.a_type, case.dist_a, pad_bits)
    B = matrix(rng, case.K, case.N, case.b_order, case.ldb, case.b_type, case.dist_b, pad_bits)
    C = None
    if case.has_c:
        C = matrix(rng, case.M, case.N, case.c_order, case.ldc, case.c_type, case.dist_c, pad_bits)
    bias = None
    if case.has_bias:
        bias = encode(draw(rng, (case.N,), case.dist_bias), case.bias_type).reshape(-1)
    return dict(A=A, B=B, C=C, bias=bias)


def d_storage(case: GemmCase, sentinel: Optional[int] = None) -> np.ndarray:
    """Output buffer of ``case`` pre-filled with a sentinel bit pattern."""
    n = storage_len(case.M, case.N, case.d_order, case.ldd)
    if sentinel is None:
        sentinel = {F16: 0x5A5A, BF16: 0x5A5A, E4M3: 0x5A, F32: 0x5A5A5A5A}[case.d_type]
    return np.full(n, sentinel, dtype=STORAGE[case.d_type])


def d_logical(case: GemmCase, flat: np.ndarray) -> np.ndarray:
    """The logical (M, N) view of an output storage array."""
    if case.d_order == ROW:
        return flat.reshape(case.M, case.ldd)[:, :case.N]
    return flat.reshape(case.N, case.ldd)[:, :case.M].T


# The five workloads.  Names describe the work; sizes and recipes follow the
# problem statement this library is measured on.
GEMM_F16_256 = GemmCase(
    name="gemm_f16_256x256x256_tn", M=256, N=256, K=256,
    a_type=F16, b_type=F16, d_type=F16, a_order=ROW, b_order=COL,
    seed=0, dist_a="u1", dist_b="u1", tol=1e-2)

GEMM_BF16_4096 = GemmCase(
    name="gemm_bf16_4096x4096x4096_tn_relu", M=4096, N=4096, K=4096,
    a_type=BF16, b_type=BF16, d_type=BF16, a_order=ROW, b_order=COL,
    alpha=1.5, beta=0.5, act=ACT_RELU, has_c=True, has_bias=True,
    seed=1, dist_a="u1", dist_b="u1", dist_c="u1", dist_bias="u01", tol=1e-2)

GEMM_F16_RAGGED = GemmCase(
    name="gemm_f16_3001x4097x777_nn", M=3001, N=4097, K=777,
    a_type=F16, b_type=F16, d_type=F16, a_order=ROW, b_order=ROW,
    alpha=1.0, beta=1.0, has_c=True, seed=2,
    dist_a="n05", dist_b="n05", dist_c="n05", tol=1e-2)

GEMM_E4M3_8192 = GemmCase(
    name="gemm_e4m3_8192x8192x8192_tn_gelu", M=8192, N=8192, K=8192,
    a_type=E4M3, b_type=E4M3, d_type=BF16, a_order=ROW, b_order=COL,
    alpha=1.0, scale_a=0.02, scale_b=0.03, act=ACT_GELU, has_bias=True,
    seed=4, dist_a="z/0.02", dist_b="z/0.03", dist_bias="u01", tol=5e-2)

GEMM_CASES = [GEMM_F16_256, GEMM_BF16_4096, GEMM_F16_RAGGED, GEMM_E4M3_8192]


@dataclass
class TransposeCase:
    name: str
    M: int
    N: int
    ld_src: int = 0
    ld_dst: int = 0
    elem_bytes: int = 4
    seed: int = 3

    def __post_init__(self):
        self.ld_src = self.ld_src or self.N
        self.ld_dst = self.ld_dst or self.M

    def bytes_moved(self) -> int:
        return 2 * self.M * self.N * self.elem_bytes


TRANSPOSE_F32_16384 = TransposeCase(name="transpose_f32_16384x16384", M=16384, N=16384)

_BITS_DTYPE = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}


def transpose_input(case: TransposeCase, pad_bits: int = 0x7FC00001) -> np.ndarray:
    """Row-major source: every bit pattern equally likely (so NaN payloads
    and subnormals occur), padding columns filled with ``pad_bits``."""
    rng = np.random.default_rng(case.seed)
    dt = _BITS_DTYPE[case.elem_bytes]
    info = np.iinfo(dt)
    vals = rng.integers(0, int(info.max) + 1, size=(case.M, case.N), dtype=dt)
    if case.ld_src == case.N:
        return vals.reshape(-1)
    buf = np.full((case.M, case.ld_src), pad_bits & int(info.max), dtype=dt)
    buf[:, :case.N] = vals
    return buf.reshape(-1)


@dataclass
class ThreadMapCase:
    name: str
    R: int
    C: int
    T: int
    V: int
    I: int
    contiguous_dim: int = 1


THREAD_MAP_64x64 = ThreadMapCase(name="thread_map_64x64_t128_v4_i8", R=64, C=64, T=128, V=4, I=8)


# ------------------------------------------------------------ convolution

@dataclass
class ConvCase:
    """A forward convolution: x N x H x W x C (NHWC), w K x R x S x C (KRSC),
    output N x P x Q x K (NPQK), all of one 16-bit type."""
    name: str
    N: int
    H: int
    W: int
    C: int
    K: int
    R: int
    S: int
    stride: tuple = (1, 1)
    pad: tuple = (0, 0)
    dil: tuple = (1, 1)
    dtype: int = F16
    alpha: float = 1.0
    beta: float = 0.0
    act: int = ACT_NONE
    has_c: bool = False
    has_bias: bool = False
    seed: int = 0
    dist: str = "u1"          # x, w and C
    dist_bias: str = "u01"
    tol: float = 1e-2

    def out_hw(self):
        def one(extent, f, s, p, d):
            span = extent + 2 * p - d * (f - 1) - 1
            return 0 if span < 0 else span // s + 1
        return (one(self.H, self.R, self.stride[0], self.pad[0], self.dil[0]),
                one(self.W, self.S, self.stride[1], self.pad[1], self.dil[1]))


def conv_inputs(case: ConvCase) -> dict:
    """Seeded raw-bit inputs, drawn in the order x, w, C, bias."""
    rng = np.random.default_rng(case.seed)
    P, Q = case.out_hw()
    x = encode(draw(rng, (case.N, case.H, case.W, case.C), case.dist), case.dtype)
    w = encode(draw(rng, (case.K, case.R, case.S, case.C), case.dist), case.dtype)
    c = encode(draw(rng, (case.N * P * Q, case.K), case.dist), case.dtype) if case.has_c else None
    b = encode(draw(rng, (case.K,), case.dist_bias), case.dtype) if case.has_bias else None
    return {"x": x, "w": w, "C": c, "bias": b}


# A 3x3, stride-1, padded layer of 56 x 56 x 64 images (batch 32), fp16,
# with bias and ReLU: an implicit GEMM of M = 100352, N = 64, K = 576.
CONV_F16_56 = ConvCase(name="conv_f16_n32_56x56x64_k64_3x3", N=32, H=56, W=56, C=64, K=64, R=3,
                       S=3, pad=(1, 1), dtype=F16, act=ACT_RELU, has_bias=True, seed=5)
