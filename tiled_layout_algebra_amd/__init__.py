"""Python binding of libtla.so (include/tla.h): argument marshalling only.

Every function has the name of the C entry point without its ``tla_``
prefix and forwards to it; all computation happens in the HIP library.
Device buffers are torch CUDA tensors (any dtype: the library reads raw
bits; sizes and leading dimensions are passed explicitly, in elements of the
storage type).  ``stream`` defaults to torch's current stream on the
tensors' device.

There is no fallback: if ``libtla.so`` has not been built this module
raises on first use.  Build it with ``python -m tiled_layout_algebra_amd.build``.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtla.so")

# enums of tla.h
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_OVERLAP, ERR_HIP = 0, -1, -2, -3, -4
F16, BF16, E4M3, F32 = 0, 1, 2, 3
ROW_MAJOR, COL_MAJOR = 0, 1
ACT_NONE, ACT_RELU, ACT_GELU = 0, 1, 2
MAX_MODES, MAX_LEAVES = 8, 16

EXPORTED = [
    "tla_gemm_epilogue", "tla_gemm_variant", "tla_gemm_run_variant", "tla_gemm_variant_info",
    "tla_conv2d_fprop", "tla_conv2d_fprop_variant",
    "tla_tiled_transpose", "tla_tiled_copy", "tla_layout_size",
    "tla_layout_eval", "tla_logical_divide", "tla_tiled_divide", "tla_thread_map",
    "tla_thread_map_eval", "tla_logical_product", "tla_coalesce", "tla_composition",
    "tla_logical_divide_modes", "tla_thread_map_ex", "tla_thread_map_eval_ex",
    "tla_status_string", "tla_version",
]


class GemmArgs(ctypes.Structure):
    _fields_ = [
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("A", ctypes.c_void_p), ("a_type", ctypes.c_int32), ("a_order", ctypes.c_int32),
        ("lda", ctypes.c_int64),
        ("B", ctypes.c_void_p), ("b_type", ctypes.c_int32), ("b_order", ctypes.c_int32),
        ("ldb", ctypes.c_int64),
        ("C", ctypes.c_void_p), ("c_type", ctypes.c_int32), ("c_order", ctypes.c_int32),
        ("ldc", ctypes.c_int64),
        ("D", ctypes.c_void_p), ("d_type", ctypes.c_int32), ("d_order", ctypes.c_int32),
        ("ldd", ctypes.c_int64),
        ("bias", ctypes.c_void_p), ("bias_type", ctypes.c_int32),
        ("act", ctypes.c_int32),
        ("alpha", ctypes.c_float), ("beta", ctypes.c_float),
        ("scale_a", ctypes.c_float), ("scale_b", ctypes.c_float),
    ]


class LayoutDesc(ctypes.Structure):
    _fields_ = [
        ("n_modes", ctypes.c_int32),
        ("leaves", ctypes.c_int32 * MAX_MODES),
        ("shape", ctypes.c_int64 * MAX_LEAVES),
        ("stride", ctypes.c_int64 * MAX_LEAVES),
    ]


class TlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s: %s (%d)" % (where, status_string(status), status))
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libtla.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libtla.so is not built (%s); run "
                              "`python -m tiled_layout_algebra_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        LP = ctypes.POINTER(LayoutDesc)
        L.tla_gemm_epilogue.argtypes = [ctypes.POINTER(GemmArgs), P]
        L.tla_gemm_variant.argtypes = [ctypes.POINTER(GemmArgs), ctypes.c_char_p, I32]
        L.tla_gemm_run_variant.argtypes = [ctypes.POINTER(GemmArgs), I32, P]
        L.tla_conv2d_fprop.argtypes = [ctypes.POINTER(ConvArgs), P]
        L.tla_conv2d_fprop_variant.argtypes = [ctypes.POINTER(ConvArgs), I32, P]
        L.tla_gemm_variant_info.argtypes = [I32, I32, ctypes.POINTER(GemmKernelInfo)]
        L.tla_tiled_transpose.argtypes = [P, I64, P, I64, I64, I64, I32, P]
        L.tla_tiled_copy.argtypes = [P, I64, P, I64, I64, I64, I32, P]
        L.tla_layout_size.argtypes = [LP, ctypes.POINTER(I64)]
        L.tla_layout_eval.argtypes = [LP, LP, P, I64, P]
        L.tla_logical_divide.argtypes = [LP, ctypes.POINTER(I64), I32, LP]
        L.tla_tiled_divide.argtypes = [LP, ctypes.POINTER(I64), I32, LP]
        L.tla_thread_map.argtypes = [I64, I64, I32, I32, I32, I32, LP]
        L.tla_thread_map_eval.argtypes = [I64, I64, I32, I32, I32, I32, I64, I64, P, P, P]
        L.tla_logical_product.argtypes = [LP, LP, LP]
        L.tla_coalesce.argtypes = [LP, LP]
        L.tla_composition.argtypes = [LP, LP, LP]
        L.tla_logical_divide_modes.argtypes = [LP, ctypes.POINTER(I64), I32, LP]
        L.tla_thread_map_ex.argtypes = [I64, I64, I32, I32, I32, I32, I32, LP]
        L.tla_thread_map_eval_ex.argtypes = [I64, I64, I32, I32, I32, I32, I32, I32, I64, I64,
                                             P, P, P]
        L.tla_status_string.argtypes = [ctypes.c_int]
        L.tla_status_string.restype = ctypes.c_char_p
        for name in EXPORTED:
            if name != "tla_status_string":
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().tla_status_string(int(status)).decode()


def version() -> int:
    return lib().tla_version()


def _check(rc: int, where: str):
    if rc != OK:
        raise TlaError(rc, where)


def _dev(t, what):
    """Device address of a CUDA tensor (None -> NULL).  Host tensors are
    refused: a host address must never reach a kernel."""
    if t is None:
        return None
    if not getattr(t, "is_cuda", False):
        raise ValueError("%s must be a CUDA tensor" % what)
    return t.data_ptr()


def _stream(stream, *tensors):
    if stream is not None:
        return int(stream)
    import torch
    dev = next((t.device for t in tensors if t is not None), None)
    return torch.cuda.current_stream(dev).cuda_stream


# ------------------------------------------------------------------- GEMM

def _gemm_args(M, N, K, A, a_type, a_order, lda, B, b_type, b_order, ldb, D, d_type,
               d_order, ldd, C=None, c_type=None, c_order=ROW_MAJOR, ldc=0, bias=None,
               bias_type=None, alpha=1.0, beta=0.0, scale_a=1.0, scale_b=1.0, act=ACT_NONE):
    return GemmArgs(
        M, N, K, _dev(A, "A"), a_type, a_order, lda, _dev(B, "B"), b_type, b_order, ldb,
        _dev(C, "C"), d_type if c_type is None else c_type, c_order, ldc,
        _dev(D, "D"), d_type, d_order, ldd,
        _dev(bias, "bias"), d_type if bias_type is None else bias_type, act,
        alpha, beta, scale_a, scale_b)


def gemm_epilogue(M, N, K, A, a_type, a_order, lda, B, b_type, b_order, ldb, D, d_type,
                  d_order, ldd, C=None, c_type=None, c_order=ROW_MAJOR, ldc=0, bias=None,
                  bias_type=None, alpha=1.0, beta=0.0, scale_a=1.0, scale_b=1.0,
                  act=ACT_NONE, stream=None, variant=None):
    """D = act(alpha*scale_a*scale_b*A.B + beta*C + bias) (tla_gemm_epilogue);
    with `variant` (0 .. GEMM_VARIANTS-1) that kernel variant is forced
    (tla_gemm_run_variant)."""
    args = _gemm_args(M, N, K, A, a_type, a_order, lda, B, b_type, b_order, ldb, D, d_type,
                      d_order, ldd, C, c_type, c_order, ldc, bias, bias_type, alpha, beta,
                      scale_a, scale_b, act)
    if variant is None:
        _check(lib().tla_gemm_epilogue(ctypes.byref(args), _stream(stream, A, B, D)),
               "tla_gemm_epilogue")
    else:
        _check(lib().tla_gemm_run_variant(ctypes.byref(args), variant, _stream(stream, A, B, D)),
               "tla_gemm_run_variant")


class ConvArgs(ctypes.Structure):
    _fields_ = [
        ("N", ctypes.c_int64), ("H", ctypes.c_int64), ("W", ctypes.c_int64),
        ("C", ctypes.c_int64), ("K", ctypes.c_int64), ("R", ctypes.c_int64),
        ("S", ctypes.c_int64),
        ("stride_h", ctypes.c_int32), ("stride_w", ctypes.c_int32),
        ("pad_h", ctypes.c_int32), ("pad_w", ctypes.c_int32),
        ("dil_h", ctypes.c_int32), ("dil_w", ctypes.c_int32),
        ("x", ctypes.c_void_p), ("w", ctypes.c_void_p), ("C_res", ctypes.c_void_p),
        ("y", ctypes.c_void_p), ("type", ctypes.c_int32),
        ("bias", ctypes.c_void_p), ("bias_type", ctypes.c_int32), ("act", ctypes.c_int32),
        ("alpha", ctypes.c_float), ("beta", ctypes.c_float),
    ]


def conv2d_args(x, w, y, N, H, W, C, K, R, S, dtype, stride=(1, 1), pad=(0, 0), dil=(1, 1),
                C_res=None, bias=None, bias_type=None, alpha=1.0, beta=0.0, act=ACT_NONE):
    """The tla_conv2d_args of a convolution (see conv2d_fprop)."""
    return ConvArgs(N, H, W, C, K, R, S, stride[0], stride[1], pad[0], pad[1], dil[0], dil[1],
                    _dev(x, "x"), _dev(w, "w"), _dev(C_res, "C_res"), _dev(y, "y"), dtype,
                    _dev(bias, "bias"), bias_type if bias_type is not None else dtype, act,
                    alpha, beta)


def conv2d_fprop(x, w, y, N, H, W, C, K, R, S, dtype, stride=(1, 1), pad=(0, 0), dil=(1, 1),
                 C_res=None, bias=None, bias_type=None, alpha=1.0, beta=0.0, act=ACT_NONE,
                 stream=None, variant=None):
    """y = act(alpha * conv(x, w) + beta * C_res + bias) (tla_conv2d_fprop, or
    tla_conv2d_fprop_variant when `variant` is given): x NHWC, w KRSC, y and
    C_res NPQK, CUDA tensors of raw 16-bit storage."""
    a = conv2d_args(x, w, y, N, H, W, C, K, R, S, dtype, stride, pad, dil, C_res, bias,
                    bias_type, alpha, beta, act)
    s = _stream(stream, x, w, y)
    if variant is None:
        _check(lib().tla_conv2d_fprop(ctypes.byref(a), s), "tla_conv2d_fprop")
    else:
        _check(lib().tla_conv2d_fprop_variant(ctypes.byref(a), variant, s),
               "tla_conv2d_fprop_variant")


def conv2d_fprop_args(args: ConvArgs, stream, variant=None) -> int:
    """Raw call with prepared ConvArgs; returns the status (no raise)."""
    if variant is None:
        return lib().tla_conv2d_fprop(ctypes.byref(args), stream)
    return lib().tla_conv2d_fprop_variant(ctypes.byref(args), variant, stream)


CONV_VARIANTS = 3
CONV_VARIANT_NAMES = ("conv_slab", "conv_implicit_fast", "conv_implicit_general")


GEMM_VARIANTS = 4


class GemmKernelInfo(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("block_m", ctypes.c_int32),
                ("block_n", ctypes.c_int32), ("threads", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32), ("vgprs", ctypes.c_int32),
                ("blocks_per_cu", ctypes.c_int32)]


def gemm_variant_info(variant: int, a_type: int) -> dict:
    """Compiled-kernel facts of a variant on the current device (needs a GPU)."""
    out = GemmKernelInfo()
    _check(lib().tla_gemm_variant_info(variant, a_type, ctypes.byref(out)),
           "tla_gemm_variant_info")
    return dict(name=out.name.decode(), block_m=out.block_m, block_n=out.block_n,
                threads=out.threads, lds_bytes=out.lds_bytes, vgprs=out.vgprs,
                blocks_per_cu=out.blocks_per_cu)


def gemm_epilogue_args(args: GemmArgs, stream) -> int:
    """Raw call with a prepared GemmArgs; returns the status (no raise)."""
    return lib().tla_gemm_epilogue(ctypes.byref(args), stream)


def gemm_variant(*args, **kw) -> str:
    """Name of the kernel variant gemm_epilogue would launch (host only)."""
    kw.pop("stream", None)
    a = _gemm_args(*args, **kw)
    buf = ctypes.create_string_buffer(64)
    _check(lib().tla_gemm_variant(ctypes.byref(a), buf, 64), "tla_gemm_variant")
    return buf.value.decode()


# -------------------------------------------------------------- transpose

def tiled_transpose(src, ld_src, dst, ld_dst, M, N, elem_bytes, stream=None):
    """dst[m + n*ld_dst] = src[m*ld_src + n], raw bits (tla_tiled_transpose)."""
    _check(lib().tla_tiled_transpose(_dev(src, "src"), ld_src, _dev(dst, "dst"), ld_dst, M, N,
                                     elem_bytes, _stream(stream, src, dst)),
           "tla_tiled_transpose")


def tiled_copy(src, ld_src, dst, ld_dst, M, N, elem_bytes, stream=None):
    """dst[m*ld_dst + n] = src[m*ld_src + n], raw bits (tla_tiled_copy)."""
    _check(lib().tla_tiled_copy(_dev(src, "src"), ld_src, _dev(dst, "dst"), ld_dst, M, N,
                                elem_bytes, _stream(stream, src, dst)), "tla_tiled_copy")


# ---------------------------------------------------------------- layouts

def make_layout(shape, stride) -> LayoutDesc:
    """Descriptor of a layout with at most one level of nesting: shape and
    stride are tuples whose entries are ints or tuples of ints."""
    if isinstance(shape, int):
        shape, stride = (shape,), (stride,)
    d = LayoutDesc()
    d.n_modes = len(shape)
    k = 0
    for i, (s, st) in enumerate(zip(shape, stride)):
        ss = s if isinstance(s, tuple) else (s,)
        dd = st if isinstance(st, tuple) else (st,)
        d.leaves[i] = len(ss)
        for x, y in zip(ss, dd):
            d.shape[k], d.stride[k] = x, y
            k += 1
    return d


def layout_tuple(d: LayoutDesc):
    """(shape, stride) nested tuples of a descriptor."""
    shape, stride, k = [], [], 0
    for i in range(d.n_modes):
        n = d.leaves[i]
        s = tuple(d.shape[k:k + n])
        t = tuple(d.stride[k:k + n])
        shape.append(s[0] if n == 1 else s)
        stride.append(t[0] if n == 1 else t)
        k += n
    return tuple(shape), tuple(stride)


def layout_size(d: LayoutDesc) -> int:
    out = ctypes.c_int64()
    _check(lib().tla_layout_size(ctypes.byref(d), ctypes.byref(out)), "tla_layout_size")
    return out.value


def layout_eval(outer: LayoutDesc, inner, out, n, stream=None):
    """out[i] = outer(i) or outer(inner(i)), i < n; out is an int64 CUDA tensor."""
    _check(lib().tla_layout_eval(ctypes.byref(outer),
                                 None if inner is None else ctypes.byref(inner),
                                 _dev(out, "out"), n, _stream(stream, out)),
           "tla_layout_eval")


def _divide(fn, d, tile):
    tile = list(tile)
    arr = (ctypes.c_int64 * len(tile))(*tile)
    out = LayoutDesc()
    _check(fn(ctypes.byref(d), arr, len(tile), ctypes.byref(out)), fn.__name__)
    return out


def logical_divide(d: LayoutDesc, tile) -> LayoutDesc:
    return _divide(lib().tla_logical_divide, d, tile)


def tiled_divide(d: LayoutDesc, tile) -> LayoutDesc:
    return _divide(lib().tla_tiled_divide, d, tile)


def logical_divide_modes(d: LayoutDesc, tile) -> LayoutDesc:
    """Every mode (nested ones too) split into (inside, index) top-level modes."""
    return _divide(lib().tla_logical_divide_modes, d, tile)


def logical_product(a: LayoutDesc, b: LayoutDesc) -> LayoutDesc:
    out = LayoutDesc()
    _check(lib().tla_logical_product(ctypes.byref(a), ctypes.byref(b), ctypes.byref(out)),
           "tla_logical_product")
    return out


def coalesce(d: LayoutDesc) -> LayoutDesc:
    out = LayoutDesc()
    _check(lib().tla_coalesce(ctypes.byref(d), ctypes.byref(out)), "tla_coalesce")
    return out


def composition(a: LayoutDesc, b: LayoutDesc) -> LayoutDesc:
    """Closed-form a o b; TlaError with status UNSUPPORTED when it has none."""
    out = LayoutDesc()
    _check(lib().tla_composition(ctypes.byref(a), ctypes.byref(b), ctypes.byref(out)),
           "tla_composition")
    return out


def thread_map(R, C, T, V, I, contiguous_dim=1) -> LayoutDesc:
    out = LayoutDesc()
    _check(lib().tla_thread_map(R, C, T, V, I, contiguous_dim, ctypes.byref(out)),
           "tla_thread_map")
    return out


def thread_map_ex(R, C, T, V, I, contiguous_dim=1, threads_per_row=0) -> LayoutDesc:
    out = LayoutDesc()
    _check(lib().tla_thread_map_ex(R, C, T, V, I, contiguous_dim, threads_per_row,
                                   ctypes.byref(out)), "tla_thread_map_ex")
    return out


def thread_map_eval_ex(R, C, T, V, I, contiguous_dim, threads_per_row, swizzle_shift, rows_valid,
                       cols_valid, out_index, out_valid=None, stream=None):
    _check(lib().tla_thread_map_eval_ex(R, C, T, V, I, contiguous_dim, threads_per_row,
                                        swizzle_shift, rows_valid, cols_valid,
                                        _dev(out_index, "out_index"), _dev(out_valid, "out_valid"),
                                        _stream(stream, out_index)),
           "tla_thread_map_eval_ex")


def thread_map_eval(R, C, T, V, I, contiguous_dim, rows_valid, cols_valid, out_index,
                    out_valid=None, stream=None):
    _check(lib().tla_thread_map_eval(R, C, T, V, I, contiguous_dim, rows_valid, cols_valid,
                                     _dev(out_index, "out_index"),
                                     _dev(out_valid, "out_valid"),
                                     _stream(stream, out_index)),
           "tla_thread_map_eval")
