"""Thin Python binding of include/zf.h (argument marshalling only).

Every step of the path runs in libzf.so; this module converts Python values
and torch tensors (device pointers via data_ptr(), the HIP stream via
torch.cuda.current_stream()) into the C ABI's arguments and raises ZfError
on a non-zero status.  If libzf.so is missing it raises at import: there is
no fallback.
"""
import ctypes as C
import os
from dataclasses import dataclass

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libzf.so")

F16, BF16, F32 = 1, 2, 3
GLOBAL_FLAT, PER_UNIT, PER_PARAM_DIM0 = 0, 1, 2
MAX_RANKS = 64
STATUS = {0: "ZF_OK", -1: "ZF_EINVAL", -2: "ZF_EALIGN", -3: "ZF_EDTYPE", -4: "ZF_ESIZE",
          -5: "ZF_EHIP", -6: "ZF_ENOMEM", -7: "ZF_EUNSUP"}


class ZfError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        detail = strerror(status)
        if status == -5:
            detail += ": " + lib.zf_hip_error_name().decode()
        super().__init__(f"{where}: {STATUS.get(status, status)} ({detail})")


class Segment(C.Structure):
    _fields_ = [("numel", C.c_int64), ("unit", C.c_int32), ("kind", C.c_int32),
                ("dim0", C.c_int64)]


class PlanSummary(C.Structure):
    _fields_ = [("psi", C.c_int64), ("psi_pad", C.c_int64), ("n_units", C.c_int64),
                ("max_unit_pad", C.c_int64), ("n_groups", C.c_int64),
                ("max_group_numel", C.c_int64), ("n_ranks", C.c_int32), ("layout", C.c_int32),
                ("stage", C.c_int32), ("policy", C.c_int32), ("workspace_bytes", C.c_int64),
                ("state_bytes", C.c_int64 * 5), ("stage3_peak_bytes", C.c_int64),
                ("comm_bytes", C.c_double * 5), ("cached_sums_bytes", C.c_int64)]


class UnitInfo(C.Structure):
    _fields_ = [("L", C.c_int64), ("P", C.c_int64), ("S", C.c_int64), ("O", C.c_int64),
                ("lam", C.c_int64)]


class GroupInfo(C.Structure):
    _fields_ = [("first_unit", C.c_int64), ("n_units", C.c_int64), ("numel", C.c_int64),
                ("padded", C.c_int64)]


class Hparams(C.Structure):
    _fields_ = [("lr", C.c_double), ("beta1", C.c_double), ("beta2", C.c_double),
                ("eps", C.c_double), ("weight_decay", C.c_double), ("max_norm", C.c_double)]


class StepArgs(C.Structure):
    _fields_ = [("grad_dtype", C.c_int32), ("param_dtype", C.c_int32),
                ("grads", C.POINTER(C.c_void_p)), ("master", C.c_void_p),
                ("exp_avg", C.c_void_p), ("exp_avg_sq", C.c_void_p), ("params", C.c_void_p),
                ("grad_shards", C.c_void_p), ("grads_reduced", C.c_int32),
                ("reserved", C.c_int32), ("numel", C.c_int64), ("workspace", C.c_void_p),
                ("workspace_size", C.c_int64),
                ("state", C.c_void_p), ("phase_events", C.POINTER(C.c_void_p))]


class StepResult(C.Structure):
    _fields_ = [("overflow", C.c_int32), ("skipped", C.c_int32), ("t", C.c_int64),
                ("sumsq", C.c_double), ("norm", C.c_double), ("coef", C.c_double),
                ("scale_used", C.c_double), ("scale_next", C.c_double), ("gs", C.c_float),
                ("growth_ctr", C.c_int32), ("bc1", C.c_float), ("bc2", C.c_float)]


class CpuAdamArgs(C.Structure):
    _fields_ = [("n", C.c_int64), ("grad", C.c_void_p), ("master", C.c_void_p),
                ("exp_avg", C.c_void_p), ("exp_avg_sq", C.c_void_p), ("params", C.c_void_p),
                ("param_dtype", C.c_int32), ("n_threads", C.c_int32), ("gs", C.c_float),
                ("bc1", C.c_float), ("bc2", C.c_float), ("grad_dtype", C.c_int32)]


class OffloadArgs(C.Structure):
    _fields_ = [("grad_dtype", C.c_int32), ("param_dtype", C.c_int32),
                ("grads", C.POINTER(C.c_void_p)), ("grad_shards", C.c_void_p),
                ("params", C.c_void_p), ("numel", C.c_int64), ("workspace", C.c_void_p),
                ("workspace_size", C.c_int64), ("state", C.c_void_p), ("h_state", C.c_void_p),
                ("h_grad", C.c_void_p), ("h_master", C.c_void_p), ("h_exp_avg", C.c_void_p),
                ("h_exp_avg_sq", C.c_void_p), ("h_params", C.c_void_p),
                ("grads_reduced", C.c_int32), ("n_threads", C.c_int32),
                ("n_chunks", C.c_int32), ("down16", C.c_int32),
                ("phase_events", C.POINTER(C.c_void_p))]


# Every function declared in include/zf.h, with its ctypes signature.
_SIGNATURES = {
    "zf_plan_flat": (C.c_int, [C.POINTER(Segment), C.c_int64, C.c_int32, C.c_int32, C.c_int32,
                               C.POINTER(C.c_void_p)]),
    "zf_plan_info": (C.c_int, [C.c_void_p, C.POINTER(PlanSummary)]),
    "zf_plan_unit": (C.c_int, [C.c_void_p, C.c_int64, C.POINTER(UnitInfo)]),
    "zf_plan_group": (C.c_int, [C.c_void_p, C.c_int64, C.POINTER(GroupInfo)]),
    "zf_gather_cast": (C.c_int, [C.c_void_p, C.c_int64, C.c_int32, C.c_void_p, C.c_int64,
                                 C.c_void_p, C.c_int64, C.c_void_p]),
    "zf_plan_free": (None, [C.c_void_p]),
    "zf_workspace_bytes": (C.c_int64, [C.c_void_p]),
    "zf_state_bytes": (C.c_int64, []),
    "zf_state_init": (C.c_int, [C.c_void_p, C.c_double, C.c_int32, C.c_int32, C.c_void_p]),
    "zf_shard_step": (C.c_int, [C.c_void_p, C.POINTER(Hparams), C.POINTER(StepArgs),
                                C.c_void_p]),
    "zf_shard_step_noalloc": (C.c_int, [C.c_void_p, C.POINTER(Hparams), C.POINTER(StepArgs),
                                        C.c_void_p]),
    "zf_reduce_scatter": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(C.c_void_p), C.c_void_p,
                                    C.c_int64, C.c_void_p]),
    "zf_gather": (C.c_int, [C.c_void_p, C.c_int64, C.c_int32, C.POINTER(C.c_void_p),
                            C.c_void_p, C.c_int64, C.c_void_p]),
    "zf_plan_buckets": (C.c_int, [C.POINTER(C.c_int64), C.c_int64, C.c_int32, C.c_int64,
                                  C.POINTER(C.c_int32), C.POINTER(C.c_int64)]),
    "zf_bucket_reduce_scatter": (C.c_int, [C.c_void_p, C.c_int64, C.c_int32,
                                           C.POINTER(C.c_void_p), C.c_void_p, C.c_int64,
                                           C.c_int32, C.c_void_p]),
    "zf_accumulate": (C.c_int, [C.c_int32, C.c_void_p, C.c_void_p, C.c_int64, C.c_int32,
                                C.c_void_p]),
    "zf_read_result": (C.c_int, [C.c_void_p, C.POINTER(StepResult), C.c_void_p]),
    "zf_cpu_adam": (C.c_int, [C.POINTER(Hparams), C.POINTER(CpuAdamArgs)]),
    "zf_offload_step": (C.c_int, [C.c_void_p, C.POINTER(Hparams), C.POINTER(OffloadArgs),
                                  C.c_void_p, C.POINTER(StepResult)]),
    "zf_reshard": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p,
                             C.c_int64, C.c_int32, C.c_void_p]),
    "zf_strerror": (C.c_char_p, [C.c_int]),
    "zf_hip_error_name": (C.c_char_p, []),
}


def _load(path=LIB_PATH, names=None):
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run fsdp_sharded_mixed_amd/build.py "
                          "(or __graft_entry__.build())")
    lib = C.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        if names is not None and name not in names:
            continue
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def load_library(path, names):
    """Another build of the library (a test build), with the signatures of
    the named calls set; its plans and state blocks are its own."""
    return _load(path, names)


def strerror(status):
    return lib.zf_strerror(int(status)).decode()


def _check(status, where):
    if status != 0:
        raise ZfError(status, where)


def _ptr(x):
    """Device pointer of a torch tensor, or an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    return x.ctypes.data  # a numpy host array


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _host_elems(x, elem_bytes):
    """Elements of elem_bytes bytes that a tensor or numpy array holds, or
    None for a raw address (its size is the caller's to pass as numel)."""
    if x is None or isinstance(x, int):
        return None
    nbytes = x.numel() * x.element_size() if hasattr(x, "element_size") else x.nbytes
    return nbytes // elem_bytes


def _default_numel(arrays, what):
    """The smallest element count of the tensors given (None entries
    skipped).  A raw address carries no size, so with one among them the
    caller must pass the count: refusing here keeps the library's size check
    meaningful."""
    arrays = [t for t in arrays if t is not None]
    if not arrays or any(isinstance(t, int) for t in arrays):
        raise ValueError(f"{what}: pass numel explicitly when an array is a raw address")
    return min(t.numel() for t in arrays)


def _ptr_array(items):
    return (C.c_void_p * len(items))(*[_ptr(t) for t in items])


@dataclass
class Plan:
    """An immutable layout plan (owns the C zf_plan)."""
    handle: int
    summary: PlanSummary
    units: list
    groups: list

    def __del__(self, _free=lib.zf_plan_free):
        h, self.handle = self.handle, None
        if h:
            _free(h)

    @property
    def n_ranks(self):
        return self.summary.n_ranks

    @property
    def psi_pad(self):
        return self.summary.psi_pad


def plan_flat(segments, n_ranks, layout, stage):
    """zf_plan_flat.  segments: sequence of (numel, unit[, kind]) or objects
    with .numel/.unit/.kind attributes."""
    arr = (Segment * len(segments))()
    for i, s in enumerate(segments):
        if isinstance(s, (tuple, list)):
            numel, unit, kind, dim0 = (list(s) + [0, 0])[:4]
        else:
            numel, unit = s.numel, s.unit
            kind, dim0 = getattr(s, "kind", 0), getattr(s, "rows", 0)
        arr[i] = Segment(int(numel), int(unit), int(kind), int(dim0))
    h = C.c_void_p()
    _check(lib.zf_plan_flat(arr, len(segments), int(n_ranks), int(layout), int(stage),
                            C.byref(h)), "zf_plan_flat")
    summary = plan_info(h.value)
    units = [plan_unit(h.value, u) for u in range(summary.n_units)]
    groups = [plan_group(h.value, g) for g in range(summary.n_groups)]
    return Plan(h.value, summary, units, groups)


def _handle(plan):
    return plan.handle if isinstance(plan, Plan) else plan


def plan_info(plan):
    out = PlanSummary()
    _check(lib.zf_plan_info(_handle(plan), C.byref(out)), "zf_plan_info")
    return out


def plan_unit(plan, u):
    out = UnitInfo()
    _check(lib.zf_plan_unit(_handle(plan), int(u), C.byref(out)), "zf_plan_unit")
    return out


def plan_group(plan, g):
    out = GroupInfo()
    _check(lib.zf_plan_group(_handle(plan), int(g), C.byref(out)), "zf_plan_group")
    return out


def workspace_bytes(plan):
    n = lib.zf_workspace_bytes(_handle(plan))
    if n < 0:
        raise ZfError(n, "zf_workspace_bytes")
    return n


def state_bytes():
    return lib.zf_state_bytes()


def state_init(state, loss_scale, dynamic, growth_interval=2000, stream=None):
    _check(lib.zf_state_init(_ptr(state), float(loss_scale), int(bool(dynamic)),
                             int(growth_interval), _stream(stream)), "zf_state_init")


def hparams(lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_norm=1.0):
    return Hparams(lr, beta1, beta2, eps, weight_decay, max_norm)


def _nbytes(t, nbytes):
    if nbytes is not None:
        return int(nbytes)
    if isinstance(t, int):
        raise ValueError("pass the size explicitly when a buffer is a raw address")
    return t.numel() * t.element_size() if t is not None else 0


def shard_step(plan, hp, grad_dtype, param_dtype, grads, master, exp_avg, exp_avg_sq, params,
               workspace, state, stream=None, phase_events=None, numel=None,
               workspace_size=None, grad_shards=None, grads_reduced=False):
    """zf_shard_step.  grads: N tensors (or addresses), or None with
    grads_reduced (grad_shards then hold the reduced gradients); params may
    be None (fp32 parameters); grad_shards: None or the fp32 gradient
    shards; phase_events: None or 4 raw hipEvent_t handles.  numel /
    workspace_size default to the sizes of the tensors passed (the smallest
    array)."""
    gp = _ptr_array(grads) if grads is not None else None
    ev = (C.c_void_p * 4)(*phase_events) if phase_events is not None else None
    if numel is None:
        numel = _default_numel(list(grads or []) + [master, exp_avg, exp_avg_sq, params,
                                                    grad_shards], "zf_shard_step")
    args = StepArgs(int(grad_dtype), int(param_dtype), gp, _ptr(master), _ptr(exp_avg),
                    _ptr(exp_avg_sq), _ptr(params), _ptr(grad_shards), int(bool(grads_reduced)),
                    0, int(numel), _ptr(workspace), _nbytes(workspace, workspace_size),
                    _ptr(state), ev)
    _check(lib.zf_shard_step(_handle(plan), C.byref(hp), C.byref(args), _stream(stream)),
           "zf_shard_step")


NOALLOC_SCRATCH_BYTES = 64 << 20


def shard_step_noalloc(plan, hp, grad_dtype, param_dtype, grads, master, exp_avg, exp_avg_sq,
                       params, state, stream=None, phase_events=None, numel=None,
                       grad_shards=None, grads_reduced=False):
    """zf_shard_step_noalloc: shard_step with the library's static scratch
    as the workspace (no workspace argument; nothing is allocated)."""
    gp = _ptr_array(grads) if grads is not None else None
    ev = (C.c_void_p * 4)(*phase_events) if phase_events is not None else None
    if numel is None:
        numel = _default_numel(list(grads or []) + [master, exp_avg, exp_avg_sq, params,
                                                    grad_shards], "zf_shard_step_noalloc")
    args = StepArgs(int(grad_dtype), int(param_dtype), gp, _ptr(master), _ptr(exp_avg),
                    _ptr(exp_avg_sq), _ptr(params), _ptr(grad_shards), int(bool(grads_reduced)),
                    0, int(numel), None, 0, _ptr(state), ev)
    _check(lib.zf_shard_step_noalloc(_handle(plan), C.byref(hp), C.byref(args),
                                     _stream(stream)), "zf_shard_step_noalloc")


def reduce_scatter(plan, grad_dtype, grads, rs_out, stream=None, numel=None):
    if numel is None:
        numel = _default_numel(list(grads) + [rs_out], "zf_reduce_scatter")
    _check(lib.zf_reduce_scatter(_handle(plan), int(grad_dtype), _ptr_array(grads),
                                 _ptr(rs_out), int(numel), _stream(stream)),
           "zf_reduce_scatter")


def plan_buckets(numel, n_ranks, bucket_numel=0):
    """zf_plan_buckets: the bucket id of every segment (buffer order) and the count."""
    n = len(numel)
    arr = (C.c_int64 * n)(*[int(x) for x in numel])
    out = (C.c_int32 * n)()
    nb = C.c_int64()
    _check(lib.zf_plan_buckets(arr, n, int(n_ranks), int(bucket_numel), out, C.byref(nb)),
           "zf_plan_buckets")
    return list(out), nb.value


def bucket_reduce_scatter(plan, group, grad_dtype, grads, grad_shards, accumulate,
                          stream=None, numel=None):
    """zf_bucket_reduce_scatter of group (bucket) `group` into grad_shards."""
    if numel is None:
        numel = _default_numel(list(grads) + [grad_shards], "zf_bucket_reduce_scatter")
    _check(lib.zf_bucket_reduce_scatter(_handle(plan), int(group), int(grad_dtype),
                                        _ptr_array(grads), _ptr(grad_shards), int(numel),
                                        int(bool(accumulate)), _stream(stream)),
           "zf_bucket_reduce_scatter")


def accumulate(grad_dtype, grad, acc, n=None, accumulate=True, stream=None):
    """zf_accumulate: acc (+)= f32(grad) over n elements (tensors or addresses)."""
    if n is None:
        n = _default_numel([grad, acc], "zf_accumulate")
    _check(lib.zf_accumulate(int(grad_dtype), _ptr(grad), _ptr(acc), int(n),
                             int(bool(accumulate)), _stream(stream)), "zf_accumulate")


def gather(plan, unit, dtype, shards, unit_buf, stream=None, unit_buf_numel=None):
    """zf_gather; unit_buf is a tensor, or an address with unit_buf_numel."""
    n = unit_buf_numel if unit_buf_numel is not None else _default_numel([unit_buf], "zf_gather")
    _check(lib.zf_gather(_handle(plan), int(unit), int(dtype), _ptr_array(shards),
                         _ptr(unit_buf), int(n), _stream(stream)), "zf_gather")


def gather_cast(plan, group, dtype, master, out, stream=None, master_numel=None,
                out_numel=None):
    """zf_gather_cast (FSDP2 unshard of one group into `out`)."""
    mn = master_numel if master_numel is not None else _default_numel([master], "zf_gather_cast")
    on = out_numel if out_numel is not None else _default_numel([out], "zf_gather_cast")
    _check(lib.zf_gather_cast(_handle(plan), int(group), int(dtype), _ptr(master), int(mn),
                              _ptr(out), int(on), _stream(stream)), "zf_gather_cast")


def read_result(state, stream=None):
    out = StepResult()
    _check(lib.zf_read_result(_ptr(state), C.byref(out), _stream(stream)), "zf_read_result")
    return out


def cpu_adam(hp, grad, master, exp_avg, exp_avg_sq, gs, bc1, bc2, params=None,
             param_dtype=BF16, n_threads=0, n=None, grad_dtype=F32):
    """zf_cpu_adam on host arrays (numpy arrays, CPU tensors or addresses);
    grad_dtype F32, or F16 / BF16 for 16-bit gradient sums."""
    def addr(x):
        if x is None or isinstance(x, int):
            return x
        if hasattr(x, "data_ptr"):
            return x.data_ptr()
        return x.ctypes.data
    if n is None:
        n = len(master)
    a = CpuAdamArgs(int(n), addr(grad), addr(master), addr(exp_avg), addr(exp_avg_sq),
                    addr(params), int(param_dtype), int(n_threads), float(gs), float(bc1),
                    float(bc2), int(grad_dtype))
    _check(lib.zf_cpu_adam(C.byref(hp), C.byref(a)), "zf_cpu_adam")


def offload_step(plan, hp, grad_dtype, param_dtype, grads, grad_shards, params, workspace,
                 state, h_state, h_grad, h_master, h_exp_avg, h_exp_avg_sq, h_params,
                 stream=None, grads_reduced=False, n_threads=0, n_chunks=8, numel=None,
                 phase_events=None, down16=False):
    """zf_offload_step; device tensors for grads/grad_shards/params/workspace/
    state, host (pinned) tensors for the h_ arrays; phase_events: None or 4
    raw hipEvent_t handles.  Returns the StepResult."""
    ev = (C.c_void_p * 4)(*phase_events) if phase_events is not None else None
    if numel is None:
        # every per-element array counts, host ones included: h_grad holds
        # the sums that come down (4 bytes each, 2 with down16), h_params the
        # 16-bit parameters going up, the h_ state arrays fp32
        dev = [t for t in list(grads or []) + [grad_shards, params] if t is not None]
        sized = [(t, t.element_size() if not isinstance(t, int) else 1) for t in dev]
        sized += [(h_grad, 2 if down16 else 4), (h_master, 4), (h_exp_avg, 4),
                  (h_exp_avg_sq, 4), (h_params, 2)]
        counts = [_host_elems(t, eb) for t, eb in sized]
        if any(c is None for c in counts):
            raise ValueError("zf_offload_step: pass numel explicitly when an array is a raw "
                             "address")
        numel = min(counts)
    gp = _ptr_array(grads) if grads is not None else None
    a = OffloadArgs(int(grad_dtype), int(param_dtype), gp, _ptr(grad_shards), _ptr(params),
                    int(numel), _ptr(workspace), _nbytes(workspace, None), _ptr(state),
                    _ptr(h_state), _ptr(h_grad), _ptr(h_master), _ptr(h_exp_avg),
                    _ptr(h_exp_avg_sq), _ptr(h_params), int(bool(grads_reduced)),
                    int(n_threads), int(n_chunks), int(bool(down16)), ev)
    out = StepResult()
    _check(lib.zf_offload_step(_handle(plan), C.byref(hp), C.byref(a), _stream(stream),
                               C.byref(out)), "zf_offload_step")
    return out


def reshard(plan_from, plan_to, src, dst, stream=None, elem_bytes=None, src_numel=None,
            dst_numel=None):
    """zf_reshard of one per-element array (tensors, or addresses with the
    counts and elem_bytes)."""
    if elem_bytes is None and isinstance(src, int):
        raise ValueError("zf_reshard: pass elem_bytes when src is a raw address")
    eb = elem_bytes if elem_bytes is not None else src.element_size()
    sn = src_numel if src_numel is not None else _default_numel([src], "zf_reshard")
    dn = dst_numel if dst_numel is not None else _default_numel([dst], "zf_reshard")
    _check(lib.zf_reshard(_handle(plan_from), _handle(plan_to), _ptr(src), int(sn), _ptr(dst),
                          int(dn), int(eb), _stream(stream)), "zf_reshard")
