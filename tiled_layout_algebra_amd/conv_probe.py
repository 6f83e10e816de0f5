"""Phase timing of the slab convolution kernel (conv_slab.hip).

    python -m tiled_layout_algebra_amd.conv_probe --build   # compile (no GPU needed)
    python -m tiled_layout_algebra_amd.conv_probe           # run (rebuilds if stale)

Builds a copy of conv_slab_kernel with an s_memtime stamp per wavefront at
each phase boundary, plus s_memrealtime at each wavefront's start and end,
runs it on the measured layer (fp16 32 x 56 x 56 x 64 -> 64, 3x3, pad 1,
bias, ReLU; the same seeded inputs as the tests and the sweep) with the
launch parameters the library picks, and prints:

  * the launch time (HIP events, 20 launches after 40 warm-up ones);
  * per wavefront slot (0-7, mean over the workgroups) the cycles spent
    issuing the filter and slab copies, waiting for them, at the first
    barrier, multiplying, at the barrier before the epilogue and in the
    epilogue;
  * workgroup durations and the spread of workgroup start times from
    s_memrealtime (100 MHz).

A development tool, not part of the library: the stamps add a few scalar
instructions and one store each.  The stores are unconditional (every lane
writes the same value), so the copy keeps the library kernel's branches.
"""
import os
import subprocess
import sys
import tempfile

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
EXE = os.path.join(HERE, "_build", "conv_probe")
_NST = 7  # memtime stamps per wave

_HOST = r'''
#include <cstdio>
#include <cstdlib>
#include <vector>
using namespace tla;
#define CK(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { \
  fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); exit(1); } } while (0)

static std::vector<uint8_t> slurp(const char* path) {
  std::vector<uint8_t> v;
  FILE* f = fopen(path, "rb");
  if (!f) { fprintf(stderr, "cannot open %s\n", path); exit(1); }
  fseek(f, 0, SEEK_END); v.resize(ftell(f)); fseek(f, 0, SEEK_SET);
  if (fread(v.data(), 1, v.size(), f) != v.size()) exit(1);
  fclose(f);
  return v;
}
static void* to_device(const std::vector<uint8_t>& h) {
  void* d; CK(hipMalloc(&d, h.size()));
  CK(hipMemcpy(d, h.data(), h.size(), hipMemcpyHostToDevice));
  return d;
}

// argv: N H W R S ph pw act x w bias out_stamps out_realtime  (fp16, 64 -> 64
// channels, stride 1, dilation 1)
int main(int argc, char** argv) {
  if (argc != 14) { fprintf(stderr, "usage\n"); return 2; }
  const int N = atoi(argv[1]), H = atoi(argv[2]), W = atoi(argv[3]), R = atoi(argv[4]),
            S = atoi(argv[5]), ph = atoi(argv[6]), pw = atoi(argv[7]), act = atoi(argv[8]);
  const int P = H + 2 * ph - R + 1, Q = W + 2 * pw - S + 1;
  void* dx = to_device(slurp(argv[9]));
  void* dw = to_device(slurp(argv[10]));
  void* db = to_device(slurp(argv[11]));
  void* dy; CK(hipMalloc(&dy, (size_t)N * P * Q * 64 * 2));
  // at most one workgroup per output row
  const size_t waves = (size_t)N * P * kWaves;
  CK(hipMalloc(&g_stamps, waves * NST * 8)); CK(hipMalloc(&g_rtime, waves * 2 * 8));
  CK(hipMemset(g_stamps, 0, waves * NST * 8)); CK(hipMemset(g_rtime, 0, waves * 2 * 8));
  // the implicit-GEMM view the convolution dispatch builds for this layer
  GemmParams p{};
  p.A = (const uint8_t*)dx; p.B = (const uint8_t*)dw; p.D = (uint8_t*)dy;
  p.bias = (const uint8_t*)db;
  p.M = N * P * Q; p.N = 64; p.K = R * S * 64;
  p.b_sr = p.K; p.b_sk = 1; p.c_sm = p.d_sm = 64; p.c_sn = p.d_sn = 1;
  p.c_type = p.d_type = p.bias_type = TLA_F16; p.act = act; p.alpha = 1.f; p.beta = 0.f;
  p.cH = H; p.cW = W; p.cC = 64; p.cR = R; p.cS = S; p.cP = P; p.cQ = Q; p.cu = 1; p.cv = 1;
  p.cph = ph; p.cpw = pw; p.cdh = 1; p.cdw = 1;
  p.flags = kCVec | kDVec | kC16 | kD16 | kBiasVec;
  for (int i = 0; i < 40; ++i) CK(launch_conv_slab(p, TLA_F16, 0) ? hipErrorUnknown : hipSuccess);
  CK(hipDeviceSynchronize());
  hipEvent_t a, b; CK(hipEventCreate(&a)); CK(hipEventCreate(&b));
  CK(hipEventRecord(a));
  for (int i = 0; i < 20; ++i) launch_conv_slab(p, TLA_F16, 0);
  CK(hipEventRecord(b)); CK(hipEventSynchronize(b));
  float ms; CK(hipEventElapsedTime(&ms, a, b));
  printf("%.2f %d\n", ms * 1000 / 20, g_grid);
  std::vector<uint64_t> hs(waves * NST), hr(waves * 2);
  CK(hipMemcpy(hs.data(), g_stamps, hs.size() * 8, hipMemcpyDeviceToHost));
  CK(hipMemcpy(hr.data(), g_rtime, hr.size() * 8, hipMemcpyDeviceToHost));
  FILE* f = fopen(argv[12], "wb"); fwrite(hs.data(), 8, hs.size(), f); fclose(f);
  f = fopen(argv[13], "wb"); fwrite(hr.data(), 8, hr.size(), f); fclose(f);
  return 0;
}
'''


def _edit(src, old, new):
    if old not in src:
        raise RuntimeError("conv_slab.hip changed: cannot place the stamps at %r" % old[:60])
    return src.replace(old, new, 1)


def probe_source():
    """The kernel file with stamps, and a host main, as one HIP source."""
    src = open(os.path.join(CSRC, "conv_slab.hip")).read()
    src = _edit(src, '#include "gemm_common.hpp"\n', '''#include "gemm_common.hpp"
#define NST %d
static uint64_t* g_stamps;
static uint64_t* g_rtime;
static int g_grid;
''' % _NST)
    src = _edit(src, """                                                                uint32_t sw_magic) {
""", """                                                                uint32_t sw_magic,
                                                                uint64_t* __restrict__ stamps,
                                                                uint64_t* __restrict__ rtime) {
  const size_t w_ = (size_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  auto stamp = [&](int k) {
    __builtin_amdgcn_sched_barrier(0);
    stamps[w_ * NST + k] = __builtin_amdgcn_s_memtime();
    __builtin_amdgcn_sched_barrier(0);
  };
  rtime[w_ * 2] = __builtin_amdgcn_s_memrealtime();
  stamp(0);
""")
    src = _edit(src, """  for (int i = 0; i < slab_rounds; ++i) copy_slab(i);
  wait_vmcnt<0>();
  stage_barrier();
""", """  for (int i = 0; i < slab_rounds; ++i) copy_slab(i);
  stamp(1);
  wait_vmcnt<0>();
  stamp(2);
  stage_barrier();
  stamp(3);
""")
    src = _edit(src, """  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  stage_barrier();
  if (!busy) return;
""", """  stamp(4);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  stage_barrier();
  stamp(5);
  if (!busy) {
    stamp(6);
    rtime[w_ * 2 + 1] = __builtin_amdgcn_s_memrealtime();
    return;
  }
""")
    src = _edit(src, """    epilogue_tiles<kGroups, 2>(e, m_base, 0, lane, acc, region);
}""", """    epilogue_tiles<kGroups, 2>(e, m_base, 0, lane, acc, region);
  stamp(6);
  rtime[w_ * 2 + 1] = __builtin_amdgcn_s_memrealtime();
}""")
    src = _edit(src, "  if (type == TLA_BF16)\n    hipLaunchKernelGGL(conv_slab_kernel<kBF16>",
                "  g_grid = (int)grid;\n  if (type == TLA_BF16)\n    hipLaunchKernelGGL(conv_slab_kernel<kBF16>")
    for _ in range(2):
        src = _edit(src, "slab_rounds, rows_per_image, sw_magic);",
                    "slab_rounds, rows_per_image, sw_magic,\n                       g_stamps, g_rtime);")
    return src + _HOST


def build(workdir=None):
    """Compile the stamped copy (into _build/ next to the library objects
    unless `workdir` is given) and return the executable's path."""
    from . import build as B
    workdir = workdir or os.path.dirname(EXE)
    os.makedirs(workdir, exist_ok=True)
    hip = os.path.join(workdir, "conv_probe.hip")
    exe = os.path.join(workdir, "conv_probe")
    with open(hip, "w") as f:
        f.write(probe_source())
    flags = [fl for fl in B.FLAGS if fl != "-fPIC"]
    r = subprocess.run([B.HIPCC, *flags, hip, "-o", exe], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stderr[-4000:])
    return exe


PHASES = ["copy issue", "copy wait", "barrier 1", "MFMAs", "barrier 2", "epilogue"]


def analyse(stamps, rtime, wgs):
    """Mean cycles per phase and wavefront slot, and workgroup timing."""
    t = stamps.reshape(-1, 8, _NST)[:wgs].astype(np.int64)
    d = np.diff(t, axis=2)                       # (wgs, 8, 6)
    rt = rtime.reshape(-1, 8, 2)[:wgs].astype(np.int64)
    start = rt[:, :, 0].min(1)
    dur = (rt[:, :, 1].max(1) - start) / 100.0   # us
    total = (t[:, :, -1] - t[:, :, 0]).max(1)    # cycles
    return dict(per_slot=d.mean(0), wg_us=float(np.median(dur)), wg_us_max=float(dur.max()),
                start_spread_us=float((start.max() - start.min()) / 100.0),
                clock_ghz=float(np.median(total / (dur * 1e3))),
                span_us=float((rt[:, :, 1].max() - start.min()) / 100.0))


def run():
    import workloads as W
    case = W.CONV_F16_56
    inp = W.conv_inputs(case)
    fresh = os.path.exists(EXE) and os.path.getmtime(EXE) >= max(
        os.path.getmtime(os.path.join(CSRC, f)) for f in ("conv_slab.hip", "gemm_common.hpp"))
    with tempfile.TemporaryDirectory() as wd:
        exe = EXE if fresh else build(wd)
        paths = {}
        for key in ("x", "w", "bias"):
            paths[key] = os.path.join(wd, key + ".bin")
            np.ascontiguousarray(inp[key]).tofile(paths[key])
        sp, rp = os.path.join(wd, "stamps.bin"), os.path.join(wd, "rtime.bin")
        cmd = [exe, str(case.N), str(case.H), str(case.W), str(case.R), str(case.S),
               str(case.pad[0]), str(case.pad[1]), str(case.act), paths["x"], paths["w"],
               paths["bias"], sp, rp]
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
        if r.returncode != 0:
            raise RuntimeError(r.stderr)
        us, grid = r.stdout.split()[-2:]
        a = analyse(np.fromfile(sp, np.uint64), np.fromfile(rp, np.uint64), int(grid))
    return case.name, float(us), int(grid), a


def report(name, us, grid, a):
    lines = ["%s: %.2f µs per launch, %d workgroups; workgroup %.2f µs (median; max %.2f), "
             "starts spread over %.2f µs, all done %.2f µs after the first start; clock %.2f GHz"
             % (name, us, grid, a["wg_us"], a["wg_us_max"], a["start_spread_us"], a["span_us"],
                a["clock_ghz"]), "",
             "| wavefront slot | " + " | ".join(PHASES) + " | total |",
             "|---|" + "---|" * (len(PHASES) + 1)]
    for w in range(8):
        row = a["per_slot"][w]
        lines.append("| %d | " % w + " | ".join("%.0f" % v for v in row) + " | %.0f |" % row.sum())
    return "\n".join(lines)


if __name__ == "__main__":
    if "--build" in sys.argv[1:]:
        print(build())
    else:
        print(report(*run()))
