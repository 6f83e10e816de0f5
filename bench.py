"""Throughput of the hot path on one MI355X.

One step = one pass of every hot-path operation over resident synthetic
inputs, enqueued on torch's current stream:
  1. tla_gemm_epilogue   bf16 4096^3, D = ReLU(1.5*A.B + 0.5*C + bias), fp32 acc
  2. tla_tiled_transpose fp32 16384 x 16384, row-major -> column-major
  3. tla_thread_map_eval the 64x64 / 128-thread / width-4 / 8-iteration map

Prints ONE JSON line.  `value` is the GEMM's TFLOP/s (2*M*N*K useful flops
per launch over its average launch time, measured with HIP events recorded
on the launch stream); the transpose's GB/s (algorithmic bytes: one read and
one write of the matrix) is reported beside it, each with its roofline.
After the step loop the e4m3 8192^3 + GELU GEMM ("fp8", against the fp8
peak), the fp16 256^3 GEMM ("f16_256") and a row-major to row-major copy of
the transpose's matrix (transpose.copy_ceiling: the same bytes with
unit-stride runs on both sides) are timed on their own.
`cpu_baseline` times the oracle on a bounded row sample of the bf16 GEMM
(and of the fp8 GEMM and the transpose, inside their entries).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --sweep [--steps K] [--warmup W]   # GEMM variant x shape table
    python bench.py --variants [--steps K] [--warmup W]  # big GEMMs, each fast variant
"""
import argparse
import itertools
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "bf16 GEMM+epilogue TFLOP/s @4096³ (% MFMA peak); transpose GB/s (% HBM peak)"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 flop/clk x 2.4 GHz, dense (fp16 the same)
PEAK_FP8_TFLOPS = 5033.2    # twice the 16-bit rate, dense
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the engine clock ramps over the first few tens of milliseconds of load:
    # 5 warm-up steps timed the GEMM at 119.7 us, 50 at 112.9, 200 at 111.5
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the separately timed fp8 8192^3 and fp16 256^3 GEMMs")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--variants", action="store_true",
                    help="instead of the JSON line: run the bf16 4096^3 and e4m3 8192^3 "
                         "workloads with every fast GEMM variant forced (a short program "
                         "for profiler counter passes) and print one line per variant")
    ap.add_argument("--pad", type=int, default=0,
                    help="with --variants: extra elements on every leading dimension")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the JSON line: time every compiled GEMM variant on a "
                         "set of shapes and print a table with each kernel's occupancy")
    return ap.parse_args()


SWEEP_SHAPES = [(1024, 1024, 1024), (2048, 2048, 2048), (4096, 4096, 4096), (8192, 8192, 2048)]


def sweep(steps, warmup):
    """Tile-configuration sweep: every variant x shape x operand type, plain
    D = A.B (bf16 D), inputs U[-1,1] seeded; occupancy from the runtime."""
    import torch
    import tiled_layout_algebra_amd as tla
    import workloads as W
    from workloads.device import to_dev

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    peaks = {W.BF16: PEAK_BF16_TFLOPS, W.E4M3: 2 * PEAK_BF16_TFLOPS}
    lines = ["| type | variant | tile | threads | LDS KiB | regs/lane | WGs/CU | waves/SIMD "
             "| M×N×K | tiles | µs | TFLOP/s | % peak | auto |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for a_type, tname in ((W.BF16, "bf16"), (W.E4M3, "e4m3")):
        infos = [tla.gemm_variant_info(v, a_type) for v in range(tla.GEMM_VARIANTS)]
        for M, N, K in SWEEP_SHAPES:
            case = W.GemmCase(name="sweep", M=M, N=N, K=K, a_type=a_type, b_type=a_type,
                              d_type=W.BF16, seed=7)
            inp = W.gemm_inputs(case)
            dA, dB = to_dev(inp["A"]), to_dev(inp["B"])
            dD = torch.empty(M * N, dtype=torch.int16, device="cuda")
            call = (M, N, K, dA, a_type, case.a_order, case.lda, dB, a_type, case.b_order,
                    case.ldb, dD, W.BF16, case.d_order, case.ldd)
            auto = tla.gemm_variant(*call)
            for v, info in enumerate(infos):
                def run():
                    tla.gemm_epilogue(*call, stream=stream.cuda_stream, variant=v)
                for _ in range(warmup):
                    run()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record(stream)
                for _ in range(steps):
                    run()
                e1.record(stream)
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1e3 / steps
                tf = 2.0 * M * N * K / (us * 1e-6) / 1e12
                bm = info["block_m"]
                tiles = -(-M // bm) * -(-N // bm)
                waves = info["blocks_per_cu"] * info["threads"] / 64 / 4
                lines.append("| %s | %s | %d×%d | %d | %d | %d | %d | %g | %d×%d×%d | %d | %.1f "
                             "| %.0f | %.1f | %s |" % (
                                 tname, info["name"], bm, bm, info["threads"],
                                 info["lds_bytes"] // 1024, info["vgprs"], info["blocks_per_cu"],
                                 waves, M, N, K, tiles, us, tf, 100 * tf / peaks[a_type],
                                 "←" if info["name"] == auto else ""))
                print(lines[-1], file=sys.stderr, flush=True)
            del dA, dB, dD
    # a row-major (N-contiguous) B or a column-major (M-contiguous) A: the
    # variants that accept them (e4m3: the general kernel only)
    lines += ["", "| operand layouts | variant | M×N×K | µs | TFLOP/s | % peak | auto |",
              "|---|---|---|---|---|---|---|"]
    layouts = ((W.BF16, W.ROW, W.ROW, "bf16 NN", (0, 1, 2)),
               (W.BF16, W.COL, W.COL, "bf16 A col, B col", (0, 1, 2)),
               (W.BF16, W.COL, W.ROW, "bf16 A col, B row", (0, 1, 2)),
               (W.E4M3, W.ROW, W.ROW, "e4m3 NN", (2,)),
               (W.E4M3, W.COL, W.COL, "e4m3 A col, B col", (2,)))
    for (a_type, a_order, b_order, label, variants), (M, N, K) in itertools.product(
            layouts, SWEEP_SHAPES):
        case = W.GemmCase(name="sweep_nn", M=M, N=N, K=K, a_type=a_type, b_type=a_type,
                          d_type=W.BF16, a_order=a_order, b_order=b_order, seed=7)
        inp = W.gemm_inputs(case)
        dA, dB = to_dev(inp["A"]), to_dev(inp["B"])
        dD = torch.empty(M * N, dtype=torch.int16, device="cuda")
        call = (M, N, K, dA, a_type, case.a_order, case.lda, dB, a_type, case.b_order,
                case.ldb, dD, W.BF16, case.d_order, case.ldd)
        auto = tla.gemm_variant(*call)
        for v in variants:
            def run():
                tla.gemm_epilogue(*call, stream=stream.cuda_stream, variant=v)
            for _ in range(warmup):
                run()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(steps):
                run()
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / steps
            tf = 2.0 * M * N * K / (us * 1e-6) / 1e12
            name = tla.gemm_variant_info(v, a_type)["name"]
            lines.append("| %s | %s | %d×%d×%d | %.1f | %.0f | %.1f | %s |" % (
                label, name, M, N, K, us, tf, 100 * tf / peaks[a_type], "←" if name == auto else ""))
            print(lines[-1], file=sys.stderr, flush=True)
        del dA, dB, dD
    # pitches off 16-byte alignment (every leading dimension one element past
    # its extent) and the ragged fp16 workload: the general kernel's cases
    lines += ["", "| odd pitches | layout | M×N×K | µs | TFLOP/s | % peak | variant |",
              "|---|---|---|---|---|---|---|"]
    odd = []
    for a_type, b_order in ((W.BF16, W.COL), (W.BF16, W.ROW), (W.E4M3, W.COL)):
        c = W.GemmCase(name="sweep_odd", M=4096, N=4096, K=4096, a_type=a_type, b_type=a_type,
                       d_type=W.BF16, b_order=b_order, seed=5)
        c.lda += 1
        c.ldb += 1
        c.ldd += 1
        odd.append(c)
    odd.append(W.GEMM_F16_RAGGED)
    for case in odd:
        inp = W.gemm_inputs(case)
        dA, dB = to_dev(inp["A"]), to_dev(inp["B"])
        dC = to_dev(inp["C"]) if inp["C"] is not None else None
        dD = torch.empty(case.M * case.ldd, dtype=torch.int16, device="cuda")
        run = gemm_call(tla, case, dA, dB, dD, dC, None, stream)
        for _ in range(warmup):
            run()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        tf = case.flops() / (us * 1e-6) / 1e12
        peak = PEAK_FP8_TFLOPS if case.a_type == W.E4M3 else PEAK_BF16_TFLOPS
        layout = "%s, A %s, B %s, lda %d, ldb %d%s" % (
            {W.BF16: "bf16", W.F16: "fp16", W.E4M3: "e4m3"}[case.a_type],
            "row" if case.a_order == W.ROW else "col", "row" if case.b_order == W.ROW else "col",
            case.lda, case.ldb, ", C ldc %d, beta %g" % (case.ldc, case.beta) if case.has_c else "")
        lines.append("| %s | %s | %d×%d×%d | %.1f | %.0f | %.1f | %s |" % (
            case.name, layout, case.M, case.N, case.K, us, tf, 100 * tf / peak,
            tla.gemm_variant(case.M, case.N, case.K, dA, case.a_type, case.a_order, case.lda, dB,
                             case.b_type, case.b_order, case.ldb, dD, case.d_type, case.d_order,
                             case.ldd, C=dC, c_type=case.c_type, ldc=case.ldc,
                             alpha=case.alpha, beta=case.beta)))
        print(lines[-1], file=sys.stderr, flush=True)
        del dA, dB, dC, dD
    # convolution: every kernel that applies, forced through
    # tla_conv2d_fprop_variant with prepared arguments (a launch costs the
    # host a few microseconds, less than any of these kernels)
    lines += ["", "| convolution | N×H×W×C → K, R×S, stride, pad | GEMM M×N×K | kernel | µs "
              "| TFLOP/s | % peak | auto |", "|---|---|---|---|---|---|---|---|"]
    for case in (W.CONV_F16_56,
                 W.ConvCase(name="conv_f16_n32_56x56x64_k64_1x1", N=32, H=56, W=56, C=64,
                            K=64, R=1, S=1, pad=(0, 0), dtype=W.F16, act=W.ACT_RELU,
                            has_bias=True, seed=8),
                 W.ConvCase(name="conv_f16_n32_56x56x128_k64_3x3", N=32, H=56, W=56, C=128,
                            K=64, R=3, S=3, pad=(1, 1), dtype=W.F16, act=W.ACT_RELU,
                            has_bias=True, seed=7),
                 W.ConvCase(name="conv_f16_n32_28x28x256_k256_3x3", N=32, H=28, W=28, C=256,
                            K=256, R=3, S=3, pad=(1, 1), dtype=W.F16, act=W.ACT_RELU,
                            has_bias=True, seed=6)):
        inp = W.conv_inputs(case)
        P, Q = case.out_hw()
        x, w, b = to_dev(inp["x"]), to_dev(inp["w"]), to_dev(inp["bias"])
        y = torch.empty(case.N * P * Q * case.K, dtype=torch.int16, device="cuda")
        args = tla.conv2d_args(x, w, y, case.N, case.H, case.W, case.C, case.K, case.R, case.S,
                               case.dtype, case.stride, case.pad, case.dil, bias=b,
                               bias_type=case.dtype, act=case.act)
        M, Kg = case.N * P * Q, case.R * case.S * case.C
        auto_done = False
        for v in range(tla.CONV_VARIANTS):
            if tla.conv2d_fprop_args(args, stream.cuda_stream, v) != tla.OK:
                continue  # this kernel does not apply to the layer
            for _ in range(warmup):
                tla.conv2d_fprop_args(args, stream.cuda_stream, v)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(steps):
                tla.conv2d_fprop_args(args, stream.cuda_stream, v)
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / steps
            tf = 2.0 * M * case.K * Kg / (us * 1e-6) / 1e12
            lines.append("| %s | %d×%d×%d×%d → %d, %d×%d, %s, %s | %d×%d×%d | %s | %.1f | %.0f "
                         "| %.1f | %s |" % (
                             case.name, case.N, case.H, case.W, case.C, case.K, case.R, case.S,
                             case.stride, case.pad, M, case.K, Kg, tla.CONV_VARIANT_NAMES[v], us,
                             tf, 100 * tf / PEAK_BF16_TFLOPS, "" if auto_done else "←"))
            auto_done = True
            print(lines[-1], file=sys.stderr, flush=True)
    print("\n".join(lines), flush=True)


CSRC = os.path.join(ROOT, "tiled_layout_algebra_amd", "csrc")
_HEADERS = ["tla/layout.hpp", "tla/copy.hpp", "tla/mfma.hpp", "kernels.hpp"]
# the sources each measured kernel is built from, besides _HEADERS
GEMM_SOURCES = "gemm_pingpong.hip+gemm_common.hpp"
GENERAL_SOURCES = "gemm_general.hip+gemm_common.hpp"
TRANSPOSE_SOURCES = "transpose.hip"


def source_sha(kernel_files):
    """First 16 hex digits of sha256 over a kernel's sources ('+'-separated
    names under csrc/) followed by the shared headers, with comments and
    blank lines taken out: an edit to comments alone keeps the hash."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in kernel_files.split("+") + _HEADERS:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        for line in text.splitlines():
            line = line.split("//", 1)[0].rstrip()
            if line:
                h.update(line.encode() + b"\n")
    return h.hexdigest()[:16]


def kernel_counters(label, kernel_files):
    """Counter results recorded in profiles/kernel_counters.txt for the kernel
    `label`, if its sources are unchanged since the counters were taken:
    dict(clock_ghz, mfma_busy, lds_conflict_rate, traffic); else None."""
    path = os.path.join(ROOT, "profiles", "kernel_counters.txt")
    if not os.path.exists(path):
        return None
    sha = source_sha(kernel_files)
    for line in open(path):
        f = line.split()
        if len(f) == 7 and not line.startswith("#") and f[0] == label and f[1] == sha:
            conf = float(f[4])
            return {"clock_ghz": float(f[2]), "mfma_busy": float(f[3]),
                    "lds_conflict_rate": None if conf != conf else conf,
                    "traffic": int(f[5]) + int(f[6])}
    return None


def roofline(achieved, peak, bound, unit, t, counters):
    """The roofline object of one kernel: achieved vs the nameplate peak, the
    launch times, and the counter results when they match the sources."""
    r = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4), "traffic": counters["traffic"] if counters else None,
         "kernel_us": round(t.mean() * 1e6, 2), "kernel_us_min": round(t.min() * 1e6, 2)}
    if counters:
        clk = counters["clock_ghz"]
        # the engine clock the counters saw during this kernel, and the
        # fraction of the peak at that clock (nameplate: 2.4 GHz)
        r["clock_ghz"] = clk
        r["frac_at_clock"] = round(achieved / (peak * clk / 2.4), 4)
        if bound == "mfma":
            r["mfma_busy"] = counters["mfma_busy"]
            r["lds_conflict_rate"] = counters["lds_conflict_rate"]
    return r


def cpu_baseline(case, inp, target_s):
    """The oracle (unchanged) on the first R rows of the GEMM: R is grown
    until one run takes about target_s seconds; returns its TFLOP/s."""
    from oracle import gemm as og
    threads = min(og.host_threads(), 16)
    rows = 4
    while True:
        kw = dict(M=rows, N=case.N, K=case.K, A=inp["A"][: rows * case.lda], a_type=case.a_type,
                  a_order=case.a_order, lda=case.lda, B=inp["B"], b_type=case.b_type,
                  b_order=case.b_order, ldb=case.ldb,
                  C=None if inp["C"] is None else inp["C"][: rows * case.ldc],
                  c_type=case.c_type, c_order=case.c_order,
                  ldc=case.ldc, bias=inp["bias"], bias_type=case.bias_type, alpha=case.alpha,
                  beta=case.beta, act=case.act, nthreads=threads)
        t0 = time.perf_counter()
        og.gemm(**kw)
        dt = time.perf_counter() - t0
        if dt >= target_s * 0.5 or rows >= case.M:
            break
        rows = min(case.M, max(rows * 2, int(rows * target_s / max(dt, 1e-3))))
    flops = 2.0 * rows * case.N * case.K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "first %d of %d output rows of %s (all %d columns, full K); %.1f s"
                      % (rows, case.M, case.name, case.N, dt)}


def cpu_baseline_transpose(tc, src, target_s):
    """The oracle's bit-copy transpose (one host thread) on the first R source
    rows of the matrix, R grown until one run takes about target_s seconds;
    returns its GB/s of algorithmic bytes (one read and one write)."""
    from oracle import gemm as og
    rows = 64
    while True:
        sub = src[: rows * tc.ld_src]
        t0 = time.perf_counter()
        og.transpose(sub, rows, tc.N, tc.ld_src, rows)
        dt = time.perf_counter() - t0
        if dt >= target_s * 0.5 or rows >= tc.M:
            break
        rows = min(tc.M, max(rows * 2, int(rows * target_s / max(dt, 1e-3))))
    return {"value": 2.0 * rows * tc.N * tc.elem_bytes / dt / 1e9, "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": "first %d of %d source rows of the fp32 %dx%d transpose; %.1f s"
                      % (rows, tc.M, tc.M, tc.N, dt)}


def time_launches(fn, stream, warmup, steps):
    """Per-launch seconds of `fn` from HIP events recorded on `stream` around
    each launch, after `warmup` untimed launches."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for e0, e1 in ev:
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return np.array([e0.elapsed_time(e1) for e0, e1 in ev]) * 1e-3


def gemm_call(tla, case, dA, dB, dD, dC, dbias, stream):
    def run():
        tla.gemm_epilogue(case.M, case.N, case.K, dA, case.a_type, case.a_order, case.lda, dB,
                          case.b_type, case.b_order, case.ldb, dD, case.d_type, case.d_order,
                          case.ldd, C=dC, c_type=case.c_type, c_order=case.c_order, ldc=case.ldc,
                          bias=dbias, bias_type=case.bias_type, alpha=case.alpha, beta=case.beta,
                          scale_a=case.scale_a, scale_b=case.scale_b, act=case.act,
                          stream=stream.cuda_stream)
    return run


def extra_gemm(tla, W, case, peak, stream, warmup, steps, cpu_s, label=None, sources=None):
    """One of the other measured GEMMs, timed on its own after the step loop:
    TFLOP/s against `peak`, and (cpu_s > 0) the oracle on a row sample;
    `label` names the kernel's row in profiles/kernel_counters.txt."""
    import torch
    from workloads.device import to_dev
    inp = W.gemm_inputs(case)
    dA, dB = to_dev(inp["A"]), to_dev(inp["B"])
    dC = to_dev(inp["C"]) if inp["C"] is not None else None
    dbias = to_dev(inp["bias"]) if inp["bias"] is not None else None
    dD = torch.empty(case.M * case.ldd, dtype=torch.int16, device="cuda")
    run = gemm_call(tla, case, dA, dB, dD, dC, dbias, stream)
    t = time_launches(run, stream, warmup, steps)
    tf = case.flops() / t.mean() / 1e12
    out = {"workload": case.name, "variant": tla.gemm_variant(
               case.M, case.N, case.K, dA, case.a_type, case.a_order, case.lda, dB, case.b_type,
               case.b_order, case.ldb, dD, case.d_type, case.d_order, case.ldd, C=dC,
               c_type=case.c_type, ldc=case.ldc, bias=dbias, bias_type=case.bias_type,
               alpha=case.alpha, beta=case.beta, scale_a=case.scale_a, scale_b=case.scale_b,
               act=case.act),
           "value": round(tf, 2), "unit": "TFLOP/s",
           "roofline": roofline(tf, peak, "mfma", "TFLOP/s", t,
                                kernel_counters(label, sources) if label else None)}
    if cpu_s > 0:
        out["cpu_baseline"] = cpu_baseline(case, inp, cpu_s)
    del dA, dB, dC, dbias, dD
    return out


def variants(steps, warmup, pad=0):
    """The two large measured GEMMs with each fast variant forced: per-launch
    µs from HIP events, one line per (workload, variant).  pad > 0 adds that
    many elements to every leading dimension (same math, other addresses)."""
    import dataclasses
    import torch
    import tiled_layout_algebra_amd as tla
    import workloads as W
    from workloads.device import to_dev
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    for case, peak in ((W.GEMM_BF16_4096, PEAK_BF16_TFLOPS), (W.GEMM_E4M3_8192, PEAK_FP8_TFLOPS)):
        if pad:
            case = dataclasses.replace(case, name=case.name + "_pad%d" % pad, lda=case.lda + pad,
                                       ldb=case.ldb + pad, ldc=case.ldc + pad if case.has_c else 0,
                                       ldd=case.ldd + pad)
        inp = W.gemm_inputs(case)
        dA, dB = to_dev(inp["A"]), to_dev(inp["B"])
        dC = to_dev(inp["C"]) if inp["C"] is not None else None
        dbias = to_dev(inp["bias"]) if inp["bias"] is not None else None
        dD = torch.empty(case.M * case.ldd, dtype=torch.int16, device="cuda")
        # three rounds, variants alternating, so clock drift hits all alike
        times = {}
        for rnd in range(3):
            for v in (0, 3, 1):
                def run():
                    tla.gemm_epilogue(case.M, case.N, case.K, dA, case.a_type, case.a_order,
                                      case.lda, dB, case.b_type, case.b_order, case.ldb, dD,
                                      case.d_type, case.d_order, case.ldd, C=dC,
                                      c_type=case.c_type, c_order=case.c_order, ldc=case.ldc,
                                      bias=dbias, bias_type=case.bias_type, alpha=case.alpha,
                                      beta=case.beta, scale_a=case.scale_a, scale_b=case.scale_b,
                                      act=case.act, stream=stream.cuda_stream, variant=v)
                t = time_launches(run, stream, warmup if rnd == 0 else 2, steps)
                times.setdefault(v, []).append(t.mean())
        for v in (0, 3, 1):
            name = tla.gemm_variant_info(v, case.a_type)["name"]
            us = float(np.median(times[v])) * 1e6
            tf = case.flops() / (us * 1e-6) / 1e12
            print("%s %s %.1f us (rounds: %s) %.0f TFLOP/s %.3f of peak" % (
                case.name, name, us, " ".join("%.1f" % (x * 1e6) for x in times[v]), tf, tf / peak),
                flush=True)
        del dA, dB, dC, dbias, dD


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        sweep(max(args.steps, 1), args.warmup)
        return
    if args.variants:
        variants(max(args.steps, 1), args.warmup, args.pad)
        return

    import torch
    import tiled_layout_algebra_amd as tla
    import workloads as W
    from workloads.device import to_dev

    torch.cuda.set_device(0)
    g = W.GEMM_BF16_4096
    tc = W.TRANSPOSE_F32_16384
    tmc = W.THREAD_MAP_64x64
    inp = W.gemm_inputs(g)
    dA, dB, dC, dbias = (to_dev(inp[k]) for k in ("A", "B", "C", "bias"))
    dD = torch.empty(g.M * g.ldd, dtype=torch.int16, device="cuda")
    tsrc = to_dev(W.transpose_input(tc))
    tdst = torch.empty_like(tsrc)
    n_map = tmc.T * tmc.V * tmc.I
    midx = torch.empty(n_map, dtype=torch.int64, device="cuda")
    mval = torch.empty(n_map, dtype=torch.uint8, device="cuda")
    variant = tla.gemm_variant(g.M, g.N, g.K, dA, g.a_type, g.a_order, g.lda, dB, g.b_type,
                               g.b_order, g.ldb, dD, g.d_type, g.d_order, g.ldd, C=dC,
                               c_type=g.c_type, ldc=g.ldc, bias=dbias, bias_type=g.bias_type,
                               alpha=g.alpha, beta=g.beta, act=g.act)
    stream = torch.cuda.current_stream()

    def gemm():
        tla.gemm_epilogue(g.M, g.N, g.K, dA, g.a_type, g.a_order, g.lda, dB, g.b_type, g.b_order,
                          g.ldb, dD, g.d_type, g.d_order, g.ldd, C=dC, c_type=g.c_type,
                          c_order=g.c_order, ldc=g.ldc, bias=dbias, bias_type=g.bias_type,
                          alpha=g.alpha, beta=g.beta, act=g.act, stream=stream.cuda_stream)

    def transpose():
        tla.tiled_transpose(tsrc, tc.ld_src, tdst, tc.ld_dst, tc.M, tc.N, 4,
                            stream=stream.cuda_stream)

    def tmap():
        tla.thread_map_eval(tmc.R, tmc.C, tmc.T, tmc.V, tmc.I, tmc.contiguous_dim, tmc.R - 1,
                            tmc.C, midx, mval, stream=stream.cuda_stream)

    def step():
        gemm(); transpose(); tmap()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        ev[s][0].record(stream)
        gemm()
        ev[s][1].record(stream)
        transpose()
        ev[s][2].record(stream)
        tmap()
        ev[s][3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    t_gemm = np.array([ev[s][0].elapsed_time(ev[s][1]) for s in range(K)]) * 1e-3
    t_tr = np.array([ev[s][1].elapsed_time(ev[s][2]) for s in range(K)]) * 1e-3
    gemm_tflops = g.flops() / t_gemm.mean() / 1e12
    tr_gbs = tc.bytes_moved() / t_tr.mean() / 1e9

    out = {
        "metric": METRIC,
        "value": round(gemm_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s + %s + %s" % (g.name, tc.name, tmc.name),
                   "gemm": {"M": g.M, "N": g.N, "K": g.K, "a": "bf16 row-major",
                            "b": "bf16 column-major", "c": "bf16 row-major", "bias": "bf16[N]",
                            "alpha": g.alpha, "beta": g.beta, "act": "relu", "seed": g.seed,
                            "variant": variant},
                   "transpose": {"M": tc.M, "N": tc.N, "elem_bytes": 4, "seed": tc.seed}},
        "roofline": roofline(gemm_tflops, PEAK_BF16_TFLOPS, "mfma", "TFLOP/s", t_gemm,
                             kernel_counters("gemm_pingpong_kernel<bf16>", GEMM_SOURCES)),
        "transpose": {"value": round(tr_gbs, 1), "unit": "GB/s",
                      "roofline": roofline(tr_gbs, PEAK_HBM_GBS, "hbm", "GB/s", t_tr,
                                           kernel_counters("transpose_lds_kernel<256,64>",
                                                           TRANSPOSE_SOURCES))},
    }
    # The identity-layout copy of the same matrix (same bytes, unit-stride
    # runs on both sides), timed on its own: the memory-system ceiling the
    # transpose is measured against.
    cdst = torch.empty_like(tsrc)

    def copy():
        tla.tiled_copy(tsrc, tc.N, cdst, tc.N, tc.M, tc.N, 4, stream=stream.cuda_stream)
    t_cp = time_launches(copy, stream, max(args.warmup // 20, 3), K)
    cp_gbs = tc.bytes_moved() / t_cp.mean() / 1e9
    out["transpose"]["copy_ceiling"] = {
        "value": round(cp_gbs, 1), "unit": "GB/s", "frac_of_peak": round(cp_gbs / PEAK_HBM_GBS, 4),
        "kernel_us": round(t_cp.mean() * 1e6, 2),
        "transpose_frac_of_copy": round(tr_gbs / cp_gbs, 4)}
    del cdst

    # The other measured GEMMs, each timed on its own after the step loop
    # (not part of a step): the fp8 8192^3 + GELU against the fp8 peak, the
    # ragged fp16 3001 x 4097 x 777 with row-major B and odd pitches (the
    # general kernel), and the launch-bound fp16 256^3.
    if not args.no_extra:
        cpu_s = 0.0 if args.no_cpu_baseline else args.cpu_seconds / 3
        out["fp8"] = extra_gemm(tla, W, W.GEMM_E4M3_8192, PEAK_FP8_TFLOPS, stream, args.warmup,
                                K, cpu_s, "gemm_pingpong_kernel<e4m3>", GEMM_SOURCES)
        out["f16_ragged"] = extra_gemm(tla, W, W.GEMM_F16_RAGGED, PEAK_BF16_TFLOPS, stream,
                                       args.warmup, K, cpu_s / 2, "gemm_kernel<f16,nt>",
                                       GENERAL_SOURCES)
        out["f16_256"] = extra_gemm(tla, W, W.GEMM_F16_256, PEAK_BF16_TFLOPS, stream,
                                    args.warmup, K, 0.0)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(g, inp, args.cpu_seconds)
        out["transpose"]["cpu_baseline"] = cpu_baseline_transpose(
            tc, W.transpose_input(tc), args.cpu_seconds / 3)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
