"""Compile the HIP libraries in-tree for gfx950.

libzf.so         the step (planner + kernels + C ABI, include/zf.h) and the
                 host side of ZeRO-Offload (CPU-Adam, the offload step)
libzf_inputs.so  the seeded input generator (include/zf_inputs.h)

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

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument", "-pthread",
    "-I", INCLUDE, "-I", CSRC,
]


def _hipcc(out, sources, host_sources=()):
    """Link `sources` (HIP) and `host_sources` (plain host C++) into `out`."""
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, "-o", tmp]
    if host_sources:
        cmd += ["-x", "c++", *host_sources]
    cmd += ["-x", "hip", *sources]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build():
    """Build both libraries; returns their paths."""
    zf = _hipcc(LIB_ZF, [os.path.join(CSRC, f) for f in
                         ("zf_step.hip", "zf_backward.hip", "zf_gather.hip", "zf_offload.hip")],
                [os.path.join(CSRC, f) for f in ("zf_plan.cpp", "zf_cpu_adam.cpp")])
    inputs = _hipcc(LIB_INPUTS, [os.path.join(CSRC, "zf_inputs.hip")])
    return zf, inputs


if __name__ == "__main__":
    for p in build():
        print(p)
