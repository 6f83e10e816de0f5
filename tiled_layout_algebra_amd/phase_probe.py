"""Phase timing of the two-group GEMM kernel (gemm_pingpong.hip).

    python -m tiled_layout_algebra_amd.phase_probe --build      # compile (no GPU needed)
    python -m tiled_layout_algebra_amd.phase_probe [bf16] [e4m3]  # run (rebuilds if stale)

Builds a copy of the kernel with an s_memtime stamp on both sides of every
workgroup barrier and around the epilogue, plus s_memrealtime at each
workgroup's start and end, runs it on the measured workloads (bf16
4096^3 + C, bias, ReLU; e4m3 8192^3 + bias, GELU; the same seeded inputs
as the tests and the bench) and prints, per workload:

  * the launch time (HIP events, 20 launches after 40 warm-up ones);
  * cycles per k-tile (median period, two barriers), and for each kind of
    half period (group 0 multiplying while group 1 reads, and the other way
    round) how many cycles after the previous release each group reached
    the barrier (medians over the k-tiles of workgroups 0-7, one per XCD);
  * prologue (kernel start to the first release) and epilogue (last
    release to the end) cycles;
  * workgroup durations per XCD from s_memrealtime (100 MHz).

A development tool, not part of the library: the stamps add a few scalar
instructions and one store per barrier.  The stores are unconditional
(every lane writes the same value) so that the copy keeps the library
kernel's basic blocks -- a branch around a store lets the compiler move
MFMAs across a barrier, which changes the schedule being measured.
"""
import os
import subprocess
import sys
import tempfile

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")

_MAX_STAMPS = 272  # per wave: 1 + 2 per barrier (2*KT + 1 of them) + 2, KT <= 134

_HOST = r'''
}  // namespace
}  // namespace tla

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
  void* d; CK(hipMalloc(&d, h.size() ? h.size() : 16));
  if (h.size()) CK(hipMemcpy(d, h.data(), h.size(), hipMemcpyHostToDevice));
  return d;
}

// argv: code M N K alpha beta act A B C|- bias|- out_stamps out_realtime
int main(int argc, char** argv) {
  if (argc != 14) { fprintf(stderr, "usage\n"); return 2; }
  const int code = atoi(argv[1]), M = atoi(argv[2]), N = atoi(argv[3]), K = atoi(argv[4]);
  const float alpha = (float)atof(argv[5]), beta = (float)atof(argv[6]);
  const int act = atoi(argv[7]);
  const bool has_c = argv[10][0] != '-', has_bias = argv[11][0] != '-';
  if (M % 256 || N % 256 || K % (code == kE4M3 ? 128 : 64)) { fprintf(stderr, "shape\n"); return 2; }
  void* dA = to_device(slurp(argv[8]));
  void* dB = to_device(slurp(argv[9]));
  void* dC = has_c ? to_device(slurp(argv[10])) : nullptr;
  void* dbias = has_bias ? to_device(slurp(argv[11])) : nullptr;
  void* dD; CK(hipMalloc(&dD, (size_t)M * N * 2));
  const int wgs = (M / 256) * (N / 256);
  const size_t nst = (size_t)wgs * 8 * MAX_STAMPS, nrt = (size_t)wgs * 8 * 2;
  uint64_t *dst, *drt;
  CK(hipMalloc(&dst, nst * 8)); CK(hipMalloc(&drt, nrt * 8));
  CK(hipMemset(dst, 0, nst * 8)); CK(hipMemset(drt, 0, nrt * 8));
  GemmParams p{};
  p.A = (const uint8_t*)dA; p.B = (const uint8_t*)dB; p.C = (const uint8_t*)dC;
  p.D = (uint8_t*)dD; p.bias = (const uint8_t*)dbias;
  p.a_sr = K; p.a_sk = 1; p.b_sr = K; p.b_sk = 1;
  p.c_sm = N; p.c_sn = 1; p.d_sm = N; p.d_sn = 1;
  p.M = M; p.N = N; p.K = K;
  p.c_type = p.d_type = p.bias_type = kBF16; p.act = act;
  p.alpha = alpha; p.beta = has_c ? beta : 0.f;
  p.flags = kDVec | kD16 | (has_c ? kCVec | kC16 : 0) | (has_bias ? kBiasVec : 0);
  int64_t grid;
  set_grid(p, 256, 256, &grid);
  auto launch = [&]() {
    if (code == kE4M3)
      hipLaunchKernelGGL(gemm_pingpong_kernel<kE4M3>, dim3((unsigned)grid), dim3(512), 0, 0, p, dst, drt);
    else
      hipLaunchKernelGGL(gemm_pingpong_kernel<kBF16>, dim3((unsigned)grid), dim3(512), 0, 0, p, dst, drt);
  };
  for (int i = 0; i < 40; ++i) launch();
  CK(hipDeviceSynchronize());
  hipEvent_t a, b; CK(hipEventCreate(&a)); CK(hipEventCreate(&b));
  CK(hipEventRecord(a));
  for (int i = 0; i < 20; ++i) launch();
  CK(hipEventRecord(b)); CK(hipEventSynchronize(b));
  float ms; CK(hipEventElapsedTime(&ms, a, b));
  printf("%.2f\n", ms * 1000 / 20);
  std::vector<uint64_t> hs(nst), hr(nrt);
  CK(hipMemcpy(hs.data(), dst, nst * 8, hipMemcpyDeviceToHost));
  CK(hipMemcpy(hr.data(), drt, nrt * 8, hipMemcpyDeviceToHost));
  FILE* f = fopen(argv[12], "wb"); fwrite(hs.data(), 8, nst, f); fclose(f);
  f = fopen(argv[13], "wb"); fwrite(hr.data(), 8, nrt, f); fclose(f);
  return 0;
}
'''


def _edit(src, old, new):
    if old not in src:
        raise RuntimeError("gemm_pingpong.hip changed: cannot place the stamps at %r" % old[:60])
    return src.replace(old, new, 1)


def probe_source():
    """The kernel file with stamps, and a host main, as one HIP source."""
    src = open(os.path.join(CSRC, "gemm_pingpong.hip")).read()
    body = src[:src.index("}  // namespace\n\nint launch_pingpong")]
    body = _edit(body, "void gemm_pingpong_kernel(const GemmParams p) {",
                 "void gemm_pingpong_kernel(const GemmParams p, uint64_t* __restrict__ stamps,\n"
                 "                                              uint64_t* __restrict__ rtime) {")
    body = _edit(body, "  const int KT = (p.K + BK - 1) / BK;\n", """  const int KT = (p.K + BK - 1) / BK;
  uint64_t* const st_ = stamps + (size_t)(blockIdx.x * 8 + wave) * MAX_STAMPS;
  int ts_ = 0;
  auto stamp = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    st_[min(ts_, MAX_STAMPS - 1)] = __builtin_amdgcn_s_memtime();
    ++ts_;
    __builtin_amdgcn_sched_barrier(0);
  };
  rtime[(blockIdx.x * 8 + wave) * 2] = __builtin_amdgcn_s_memrealtime();
  stamp();
""")
    body = _edit(body, """  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    stage_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };""", """  auto barrier = [&]() {
    stamp();
    __builtin_amdgcn_sched_barrier(0);
    stage_barrier();
    __builtin_amdgcn_sched_barrier(0);
    stamp();
  };""")
    body = _edit(body, """  epilogue_tiles<FM, FN>(p, m0 + wm0, n0 + wn0, lane, acc, smem + wave * (32 * FM) * (64 * FN));
}""", """  stamp();
  epilogue_tiles<FM, FN>(p, m0 + wm0, n0 + wn0, lane, acc, smem + wave * (32 * FM) * (64 * FN));
  stamp();
  rtime[(blockIdx.x * 8 + wave) * 2 + 1] = __builtin_amdgcn_s_memrealtime();
}""")
    return "#define MAX_STAMPS %d\n" % _MAX_STAMPS + body + _HOST


EXE = os.path.join(HERE, "_build", "phase_probe")


def build(workdir=None):
    """Compile the stamped copy (into _build/ next to the library objects
    unless `workdir` is given) and return the executable's path."""
    from . import build as B
    workdir = workdir or os.path.dirname(EXE)
    os.makedirs(workdir, exist_ok=True)
    hip = os.path.join(workdir, "phase_probe.hip")
    exe = os.path.join(workdir, "phase_probe")
    with open(hip, "w") as f:
        f.write(probe_source())
    flags = [fl for fl in B.FLAGS if fl != "-fPIC"]
    r = subprocess.run([B.HIPCC, *flags, hip, "-o", exe], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + r.stderr[-4000:])
    return exe


def analyse(stamps, rtime, wgs):
    """Per-phase figures from the stamp arrays (see the module docstring).

    Barrier 0 ends the prologue.  From then on barriers alternate: group 0
    reaches an odd barrier after its memory phase and an even one after its
    compute phase, group 1 the other way round.
    """
    t = stamps.reshape(wgs, 8, _MAX_STAMPS).astype(np.int64)
    periods, g0m, g1m, pro, epi = [], [], [], [], []
    for wg in range(min(8, wgs)):  # one workgroup per XCD, first round
        T = t[wg]
        n = int((T[0] > 0).sum())
        nb = (n - 3) // 2                      # barriers
        arr = np.array([[T[w, 1 + 2 * b] for b in range(nb)] for w in range(8)])
        dep = np.array([[T[w, 2 + 2 * b] for b in range(nb)] for w in range(8)])
        rel = dep.max(0)                      # when each barrier released
        half = np.diff(rel)                   # half[b-1]: release b-1 -> release b
        core = half[2:-2]                     # halves ending at barriers 3 .. nb-3
        core = core[:len(core) // 2 * 2]
        periods.append(np.median(core[0::2] + core[1::2]))
        late = [arr[0:4, b].max() - rel[b - 1] for b in range(1, nb)]   # group 0
        late1 = [arr[4:8, b].max() - rel[b - 1] for b in range(1, nb)]  # group 1
        even = [i for i, b in enumerate(range(1, nb)) if b % 2 == 0 and 2 < b < nb - 2]
        odd = [i for i, b in enumerate(range(1, nb)) if b % 2 == 1 and 2 < b < nb - 2]
        # group 0 multiplies in the halves ending at even barriers
        g0m.append([np.median([late[i] for i in even]), np.median([late1[i] for i in even])])
        g1m.append([np.median([late[i] for i in odd]), np.median([late1[i] for i in odd])])
        pro.append(rel[0] - T[:, 0].min())
        epi.append(T[:, n - 1].max() - rel[-1])
    rt = rtime.reshape(wgs, 8, 2).astype(np.int64)
    dur = (rt[:, :, 1].max(1) - rt[:, :, 0].min(1)) / 100.0   # us
    xcd = np.arange(wgs) % 8
    return dict(period=float(np.median(periods)), g0m=np.median(g0m, 0), g1m=np.median(g1m, 0),
                prologue=float(np.median(pro)), epilogue=float(np.median(epi)),
                xcd_us=[float(np.median(dur[xcd == k])) for k in range(8)])


def run(which=("bf16", "e4m3")):
    import workloads as W
    cases = {"bf16": W.GEMM_BF16_4096, "e4m3": W.GEMM_E4M3_8192}
    codes = {"bf16": 1, "e4m3": 2}   # the kernel's operand codes
    out = []
    fresh = os.path.exists(EXE) and os.path.getmtime(EXE) >= max(
        os.path.getmtime(os.path.join(CSRC, f)) for f in ("gemm_pingpong.hip", "gemm_common.hpp"))
    with tempfile.TemporaryDirectory() as wd:
        exe = EXE if fresh else build(wd)
        for name in which:
            case = cases[name]
            inp = W.gemm_inputs(case)
            paths = {}
            for key in ("A", "B", "C", "bias"):
                if inp[key] is None:
                    paths[key] = "-"
                else:
                    paths[key] = os.path.join(wd, key + ".bin")
                    np.ascontiguousarray(inp[key]).tofile(paths[key])
            sp, rp = os.path.join(wd, "stamps.bin"), os.path.join(wd, "rtime.bin")
            alpha = case.alpha * case.scale_a * case.scale_b
            cmd = [exe, str(codes[name]), str(case.M), str(case.N), str(case.K), repr(alpha),
                   repr(case.beta), str(case.act), paths["A"], paths["B"], paths["C"],
                   paths["bias"], sp, rp]
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
            if r.returncode != 0:
                raise RuntimeError(r.stderr)
            us = float(r.stdout.split()[-1])
            wgs = (case.M // 256) * (case.N // 256)
            a = analyse(np.fromfile(sp, np.uint64), np.fromfile(rp, np.uint64), wgs)
            out.append((case.name, us, a))
    return out


def report(results):
    lines = ["| workload | µs per launch | cycles per k-tile | group 0 multiplies: "
             "group 0 / group 1 at the barrier | group 1 multiplies: group 0 / group 1 at the "
             "barrier | prologue cycles | epilogue cycles | workgroup µs on XCD 0–7 |",
             "|---|---|---|---|---|---|---|---|"]
    for name, us, a in results:
        lines.append("| %s | %.1f | %.0f | %.0f / %.0f | %.0f / %.0f | %.0f | %.0f | %s |" % (
            name, us, a["period"], a["g0m"][0], a["g0m"][1], a["g1m"][0], a["g1m"][1],
            a["prologue"], a["epilogue"], " ".join("%.1f" % x for x in a["xcd_us"])))
    return "\n".join(lines)


if __name__ == "__main__":
    sys.path.insert(0, ROOT)
    if "--build" in sys.argv:
        print(build())
    else:
        which = [w for w in sys.argv[1:] if w in ("bf16", "e4m3")] or ["bf16", "e4m3"]
        print(report(run(which)))
