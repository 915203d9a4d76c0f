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

Every translation unit compiles on its own (in parallel) into _build/ at the
repository root, and each library is linked from its objects.

Flags that matter for the arithmetic contract:
  -ffp-contract=off                        no a*b+c -> fma fusion
  -fhip-fp32-correctly-rounded-divide-sqrt correctly rounded / and sqrtf
  -target-feature -packed-fp32-ops         no packed fp32 instructions
fp32 denormals are kept (the HIP default; nothing flushes them).
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")

LIB_ZF = os.path.join(PKG, "libzf.so")
LIB_INPUTS = os.path.join(PKG, "libzf_inputs.so")
LIB_WINDOW_TEST = os.path.join(PKG, "libzf_window_test.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
BUILD_DIR = os.path.join(ROOT, "_build")  # objects; the libraries go in-tree
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument", "-pthread",
    "-I", INCLUDE, "-I", CSRC,
]
LINK = ["--offload-arch=gfx950", "-shared", "-fPIC", "-pthread"]


def _run(cmd):
    subprocess.run(cmd, check=True)


def _object(src, lang, defines=(), tag=""):
    """(output, command) compiling one source (lang "hip" or "c++")."""
    name = os.path.splitext(os.path.basename(src))[0]
    out = os.path.join(BUILD_DIR, f"{name}{tag}.o")
    return out, [HIPCC, *FLAGS, *defines, "-c", "-x", lang, src, "-o", out]


def _libraries():
    """Each library: (path, [(source, lang, defines, tag), ...])."""
    def c(f):
        return os.path.join(CSRC, f)
    step = [(c(f), "hip", (), "") for f in
            ("zf_step.hip", "zf_backward.hip", "zf_gather.hip", "zf_offload.hip")]
    host = [(c(f), "c++", (), "") for f in ("zf_plan.cpp", "zf_cpu_adam.cpp")]
    window = ("-DZF_TEST_CACHED_SUMS_MB=1",)
    return [
        (LIB_ZF, step + host),
        (LIB_INPUTS, [(c("zf_inputs.hip"), "hip", (), "")]),
        (LIB_WINDOW_TEST, [(c("zf_step.hip"), "hip", window, "_window"),
                           (c("zf_plan.cpp"), "c++", window, "_window")]),
    ]


def build(jobs=None):
    """Compile every translation unit (in parallel) and link the libraries;
    returns their paths."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    libs = _libraries()
    units = {}
    for _, srcs in libs:
        for src, lang, defines, tag in srcs:
            out, cmd = _object(src, lang, defines, tag)
            units[out] = cmd
    jobs = jobs or min(8, os.cpu_count() or 1, len(units))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(_run, units.values()))  # raises the first failure
    paths = []
    for path, srcs in libs:
        objs = [_object(src, lang, defines, tag)[0] for src, lang, defines, tag in srcs]
        tmp = path + ".tmp"
        _run([HIPCC, *LINK, *objs, "-o", tmp])
        os.replace(tmp, path)
        paths.append(path)
    return tuple(paths)


if __name__ == "__main__":
    for p in build():
        print(p)
