"""Sharded mixed-precision AdamW (ZeRO-1/2/3, FSDP FlatParameter) for MI355X.

Layers:
  include/zf.h, csrc/       the C ABI and its gfx950 HIP kernels (libzf.so)
  zf.py                     thin ctypes binding of the C ABI
  include/zf_inputs.h       seeded synthetic inputs (libzf_inputs.so), inputs.py
  workloads.py              the synthetic workloads (shapes, dtypes, hyperparameters)
  runner.py                 device buffers and the step sequence for a workload
  build.py                  in-tree hipcc build for gfx950

Importing the package does not load the HIP libraries; importing .zf does,
and fails loudly if libzf.so has not been built.
"""
__all__ = ["workloads"]
