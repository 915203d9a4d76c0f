"""Binding of include/zf_inputs.h: seeded synthetic inputs filled on the GPU.

Input generation only (no step arithmetic).  The values follow the
splitmix64 + Irwin-Hall(12) definition in zf_inputs.h and depend only on
(seed, stream, logical index).
"""
import ctypes as C
import os

from . import workloads as W

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libzf_inputs.so")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run fsdp_sharded_mixed_amd/build.py")
    lib = C.CDLL(LIB_PATH)
    lib.zfi_fill_normal16.restype = C.c_int
    lib.zfi_fill_normal16.argtypes = [C.c_void_p, C.c_int64, C.c_int32, C.c_uint64, C.c_uint64,
                                      C.c_int64, C.c_double, C.c_double, C.c_void_p]
    lib.zfi_fill_normal32.restype = C.c_int
    lib.zfi_fill_normal32.argtypes = [C.c_void_p, C.c_int64, C.c_uint64, C.c_uint64, C.c_int64,
                                      C.c_double, C.c_void_p]
    lib.zfi_stream_probe.restype = C.c_int
    lib.zfi_stream_probe.argtypes = [C.POINTER(C.c_void_p), C.c_int32, C.POINTER(C.c_void_p),
                                     C.c_int32, C.c_int64, C.c_void_p]
    lib.zfi_stream_probe_shaped.restype = C.c_int
    lib.zfi_stream_probe_shaped.argtypes = [C.POINTER(C.c_void_p), C.c_int32,
                                            C.POINTER(C.c_void_p), C.c_int32, C.c_int64,
                                            C.c_int32, C.c_int32, C.c_void_p]
    lib.zfi_stream_output.restype = C.c_uint64
    lib.zfi_stream_output.argtypes = [C.c_uint64, C.c_uint64, C.c_uint64]
    lib.zfi_update_mix_probe.restype = C.c_int
    lib.zfi_update_mix_probe.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                         C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64,
                                         C.c_int32, C.c_int32, C.c_void_p]
    lib.zfi_sqrt_probe.restype = C.c_int
    lib.zfi_sqrt_probe.argtypes = [C.c_void_p, C.c_int64, C.c_uint32, C.c_void_p]
    lib.zfi_div_probe.restype = C.c_int
    lib.zfi_div_probe.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p]
    return lib


lib = _load()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def fill_normal16(dst, n, dtype, seed, stream_id, logical_base, sigma, scale=1.0,
                  offset=0, stream=None):
    """Fill n 16-bit values of tensor `dst` starting at element `offset`."""
    addr = dst.data_ptr() + 2 * int(offset)
    rc = lib.zfi_fill_normal16(addr, int(n), int(dtype), int(seed), int(stream_id),
                               int(logical_base), float(sigma), float(scale), _stream(stream))
    if rc != 0:
        raise RuntimeError(f"zfi_fill_normal16 failed ({rc})")


def fill_normal32(dst, n, seed, stream_id, logical_base, sigma, offset=0, stream=None):
    addr = dst.data_ptr() + 4 * int(offset)
    rc = lib.zfi_fill_normal32(addr, int(n), int(seed), int(stream_id), int(logical_base),
                               float(sigma), _stream(stream))
    if rc != 0:
        raise RuntimeError(f"zfi_fill_normal32 failed ({rc})")


def stream_output(seed, stream_id, j):
    return lib.zfi_stream_output(int(seed), int(stream_id), int(j))


def inject_index(w, psi):
    """Logical index that receives a workload's injected +inf: output 0 of
    the inject stream, modulo Psi."""
    return stream_output(w.seed, W.STREAM_INJECT, 0) % psi


def stream_probe(srcs, dsts, n=None, stream=None):
    """zfi_stream_probe: dst[k] = sum of srcs, with the step's access pattern."""
    n = min(t.numel() for t in list(srcs) + list(dsts)) if n is None else n
    sp = (C.c_void_p * len(srcs))(*[t.data_ptr() for t in srcs])
    dp = (C.c_void_p * len(dsts))(*[t.data_ptr() for t in dsts])
    rc = lib.zfi_stream_probe(sp, len(srcs), dp, len(dsts), int(n), _stream(stream))
    if rc != 0:
        raise RuntimeError(f"zfi_stream_probe failed ({rc})")


def stream_probe_shaped(srcs, dsts, quads, blocks_per_cu, n=None, stream=None):
    """zfi_stream_probe_shaped: the same sums with `quads` quads per lane and
    at most `blocks_per_cu` resident blocks per CU (0: no limit)."""
    n = min(t.numel() for t in list(srcs) + list(dsts)) if n is None else n
    sp = (C.c_void_p * len(srcs))(*[t.data_ptr() for t in srcs])
    dp = (C.c_void_p * len(dsts))(*[t.data_ptr() for t in dsts])
    rc = lib.zfi_stream_probe_shaped(sp, len(srcs), dp, len(dsts), int(n), int(quads),
                                     int(blocks_per_cu), _stream(stream))
    if rc != 0:
        raise RuntimeError(f"zfi_stream_probe_shaped failed ({rc})")


def update_mix_probe(g, p, m, v, out16, n, block_threads, blocks_per_cu, stream=None):
    """zfi_update_mix_probe: the update pass's bytes with no arithmetic.  `g`
    is a pair of tensors (two 16-bit gradient replicas, read as n 16-bit
    elements each) or one fp32 tensor (sums); p, m, v fp32; out16 holds n
    16-bit elements."""
    if isinstance(g, (tuple, list)):
        g0, g1, sums = g[0].data_ptr(), g[1].data_ptr(), None
    else:
        g0, g1, sums = None, None, g.data_ptr()
    rc = lib.zfi_update_mix_probe(g0, g1, sums, p.data_ptr(), m.data_ptr(), v.data_ptr(),
                                  out16.data_ptr(), int(n), int(block_threads),
                                  int(blocks_per_cu), _stream(stream))
    if rc != 0:
        raise RuntimeError(f"zfi_update_mix_probe failed ({rc})")


def sqrt_probe(out, first_bits, n=None, stream=None):
    """zfi_sqrt_probe: out[i] = sqrtf of the binary32 with bits first_bits + i."""
    n = out.numel() if n is None else n
    rc = lib.zfi_sqrt_probe(out.data_ptr(), int(n), int(first_bits), _stream(stream))
    if rc != 0:
        raise RuntimeError(f"zfi_sqrt_probe failed ({rc})")


def div_probe(a, b, out, stream=None):
    """zfi_div_probe: out = a / b, elementwise, binary32."""
    n = min(a.numel(), b.numel(), out.numel())
    rc = lib.zfi_div_probe(a.data_ptr(), b.data_ptr(), out.data_ptr(), int(n), _stream(stream))
    if rc != 0:
        raise RuntimeError(f"zfi_div_probe failed ({rc})")
