"""Helpers shared by the GPU parity tests: host <-> device copies of raw
storage bits, and one call of each entry point through the binding."""
import numpy as np
import torch

import tiled_layout_algebra_amd as tla
import workloads as W
from oracle import gemm as og
from workloads.device import to_dev, to_host  # noqa: F401  (re-exported for the tests)


def run_gemm(case: W.GemmCase, inp: dict, sentinel=None, pad_front=0, d_is_c=False, variant=None):
    """One tla_gemm_epilogue call; returns the D storage array (host)."""
    dA = to_dev(inp["A"], pad_front) if inp["A"] is not None else None
    dB = to_dev(inp["B"], pad_front) if inp["B"] is not None else None
    dC = to_dev(inp["C"], pad_front) if inp["C"] is not None else None
    dbias = to_dev(inp["bias"], pad_front) if inp["bias"] is not None else None
    if d_is_c:
        dD = dC
    else:
        dD = to_dev(W.d_storage(case, sentinel), pad_front)
    tla.gemm_epilogue(case.M, case.N, case.K, dA, case.a_type, case.a_order, case.lda,
                      dB, case.b_type, case.b_order, case.ldb, dD, case.d_type, case.d_order,
                      case.ldd, C=dC, c_type=case.c_type, c_order=case.c_order, ldc=case.ldc,
                      bias=dbias, bias_type=case.bias_type, alpha=case.alpha, beta=case.beta,
                      scale_a=case.scale_a, scale_b=case.scale_b, act=case.act, variant=variant)
    torch.cuda.synchronize()
    return to_host(dD, W.STORAGE[case.d_type])


def variant(case: W.GemmCase) -> str:
    """The kernel variant the library picks for `case` (host-side query);
    distinct 256-byte-aligned dummies stand in for the buffers."""
    fA, fB, fC, fD, fb = (torch.empty(64, device="cuda") for _ in range(5))
    return tla.gemm_variant(case.M, case.N, case.K, fA, case.a_type, case.a_order, case.lda,
                            fB, case.b_type, case.b_order, case.ldb, fD, case.d_type,
                            case.d_order, case.ldd, C=fC if case.has_c else None,
                            c_type=case.c_type, c_order=case.c_order, ldc=case.ldc,
                            bias=fb if case.has_bias else None, bias_type=case.bias_type,
                            alpha=case.alpha, beta=case.beta, scale_a=case.scale_a,
                            scale_b=case.scale_b, act=case.act)


def oracle_kwargs(case: W.GemmCase, inp: dict) -> dict:
    return dict(M=case.M, N=case.N, K=case.K, A=inp["A"], a_type=case.a_type,
                a_order=case.a_order, lda=case.lda, B=inp["B"], b_type=case.b_type,
                b_order=case.b_order, ldb=case.ldb, C=inp["C"], c_type=case.c_type,
                c_order=case.c_order, ldc=case.ldc, bias=inp["bias"],
                bias_type=case.bias_type, alpha=case.alpha, beta=case.beta,
                scale_a=case.scale_a, scale_b=case.scale_b, act=case.act)


def oracle_ref(case, inp):
    return og.gemm(**oracle_kwargs(case, inp))


def oracle_points(case, inp, ms, ns):
    return og.gemm_points(ms, ns, **oracle_kwargs(case, inp))


def padding_untouched(case: W.GemmCase, D_flat: np.ndarray, sentinel: int) -> bool:
    """Every element of D's storage outside the logical M x N is the sentinel."""
    if D_flat.size == 0:
        return True
    mask = np.ones(D_flat.size, dtype=bool)
    if case.d_order == W.ROW:
        mask.reshape(case.M, case.ldd)[:, :case.N] = False
    else:
        mask.reshape(case.N, case.ldd)[:, :case.M] = False
    return bool((D_flat[mask] == sentinel).all())
