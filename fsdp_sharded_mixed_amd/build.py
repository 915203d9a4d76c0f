"""Compile the HIP libraries in-tree for gfx950.

libzf.so         the step (planner + kernels + C ABI, include/zf.h) and the
                 host side of ZeRO-Offload (CPU-Adam, the offload step)
libzf_inputs.so  the seeded input generator (include/zf_inputs.h)
libzf_window_test.so
                 a test build of the step (planner + step kernels, the same
                 C ABI) whose memory-side cache window is 1 MiB for every
                 plan, so that the tests can run the split of pass 1's sum
                 stores (non-temporal below the window, cache-allocating in
                 it) and the update pass's backward walk on small plans

Flags that matter for the arithmetic contract:
  -ffp-contract=off                        no a*b+c -> fma fusion
  -fhip-fp32-correctly-rounded-divide-sqrt correctly rounded / and sqrtf
  -target-feature -packed-fp32-ops         no packed fp32 instructions
fp32 denormals are kept (the HIP default; nothing flushes them).
"""
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")

LIB_ZF = os.path.join(PKG, "libzf.so")
LIB_INPUTS = os.path.join(PKG, "libzf_inputs.so")
LIB_WINDOW_TEST = os.path.join(PKG, "libzf_window_test.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument", "-pthread",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc(out, sources, host_sources=(), defines=()):
    """Link `sources` (HIP) and `host_sources` (plain host C++) into `out`."""
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *defines, "-o", tmp]
    if host_sources:
        cmd += ["-x", "c++", *host_sources]
    cmd += ["-x", "hip", *sources]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build():
    """Build the libraries; returns their paths."""
    zf = _hipcc(LIB_ZF, [os.path.join(CSRC, f) for f in
                         ("zf_step.hip", "zf_backward.hip", "zf_gather.hip", "zf_offload.hip")],
                [os.path.join(CSRC, f) for f in ("zf_plan.cpp", "zf_cpu_adam.cpp")])
    inputs = _hipcc(LIB_INPUTS, [os.path.join(CSRC, "zf_inputs.hip")])
    window = _hipcc(LIB_WINDOW_TEST, [os.path.join(CSRC, "zf_step.hip")],
                    [os.path.join(CSRC, "zf_plan.cpp")], defines=["-DZF_TEST_CACHED_SUMS_MB=1"])
    return zf, inputs, window


if __name__ == "__main__":
    for p in build():
        print(p)
