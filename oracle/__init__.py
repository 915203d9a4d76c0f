"""CPU oracle for the sharded mixed-precision AdamW step -- TEST INFRASTRUCTURE.

Only the test suite, the package smoke check and the bench's CPU-baseline leg
may import this package.  It wraps oracle/liboracle.so (plain single-threaded
C, see zf_oracle.c) with numpy arrays and shares no code with the HIP library.

Array conventions (the oracle's own, independent of the GPU library):
  * a replica gradient is the full padded flat, Psi' 16-bit words (uint16);
  * rank r's master / exp_avg / exp_avg_sq / 16-bit shard is one buffer of
    sum_u S_u elements, unit u's shard at offset M_u (unit-major);
  * the full gathered 16-bit buffer is the padded flat (Psi' words).
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

F16, BF16 = 1, 2
GLOBAL_FLAT, PER_UNIT = 0, 1

UNIT_DTYPE = np.dtype([("L", "<i8"), ("P", "<i8"), ("S", "<i8"), ("O", "<i8"),
                       ("lam", "<i8"), ("M", "<i8")])


class Hparams(C.Structure):
    _fields_ = [("lr", C.c_double), ("beta1", C.c_double), ("beta2", C.c_double),
                ("eps", C.c_double), ("weight_decay", C.c_double), ("max_norm", C.c_double)]


class ScaleState(C.Structure):
    _fields_ = [("loss_scale", C.c_double), ("t", C.c_int64), ("growth_ctr", C.c_int32),
                ("growth_interval", C.c_int32), ("dynamic", C.c_int32), ("pad_", C.c_int32)]

    def copy(self):
        s = ScaleState()
        C.memmove(C.byref(s), C.byref(self), C.sizeof(ScaleState))
        return s


class Scalars(C.Structure):
    _fields_ = [(n, C.c_float) for n in
                ("gs", "dec", "b1", "c1", "b2", "c2", "bc1", "bc2", "lrf", "ef")]


class Result(C.Structure):
    _fields_ = [("overflow", C.c_int32), ("skipped", C.c_int32), ("sumsq", C.c_double),
                ("norm", C.c_double), ("coef", C.c_double), ("scale_used", C.c_double),
                ("scale_next", C.c_double), ("t", C.c_int64), ("gs", C.c_float),
                ("pad_", C.c_int32)]


class Inject(C.Structure):
    _fields_ = [("step", C.c_int64), ("replica", C.c_int64), ("index", C.c_int64),
                ("bits", C.c_uint16), ("pad_", C.c_uint16 * 3)]


_lib = None


def lib():
    """Load liboracle.so, building it first if it is missing."""
    global _lib
    if _lib is None:
        # ZF_ORACLE_LIB lets the mutation test load a deliberately broken copy
        path = os.environ.get("ZF_ORACLE_LIB", _build.LIB)
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        L = C.CDLL(path)
        vp, i32, i64, u64, dbl = C.c_void_p, C.c_int32, C.c_int64, C.c_uint64, C.c_double
        sig = {
            "or_f16_to_f32": (C.c_float, [C.c_uint16]),
            "or_bf16_to_f32": (C.c_float, [C.c_uint16]),
            "or_f32_to_f16": (C.c_uint16, [C.c_float]),
            "or_f32_to_bf16": (C.c_uint16, [C.c_float]),
            "or_cast_array": (None, [i32, i64, vp, vp]),
            "or_widen_array": (None, [i32, i64, vp, vp]),
            "or_splitmix64_next": (u64, [C.POINTER(u64)]),
            "or_stream_state": (u64, [u64, u64]),
            "or_normal_z": (C.c_float, [u64, i64]),
            "or_gen16": (None, [vp, i64, i32, u64, u64, i64, dbl, dbl]),
            "or_gen32": (None, [vp, i64, u64, u64, i64, dbl]),
            "or_layout": (C.c_int, [vp, vp, i64, i32, i32, vp, i64, C.POINTER(i64),
                                    C.POINTER(i64), C.POINTER(i64)]),
            "or_ledger": (C.c_int, [vp, i64, i32, i32, C.POINTER(i64), C.POINTER(i64)]),
            "or_layout_dim0": (C.c_int, [vp, vp, i64, i32, vp, i64, C.POINTER(i64),
                                         C.POINTER(i64), C.POINTER(i64)]),
            "or_fsdp2_step": (C.c_int, [i32, i32, vp, i64, vp, vp, vp, vp, vp,
                                        C.POINTER(Hparams), C.POINTER(ScaleState),
                                        C.POINTER(Result)]),
            "or_fsdp2_gather": (C.c_int, [vp, i64, i32, i64, i64, i32, vp, vp]),
            "or_comm_bytes": (dbl, [i64, i32, i32]),
            "or_reduce_scatter": (C.c_int, [i32, i32, vp, i64, vp, vp]),
            "or_finish": (C.c_int, [dbl, i32, i32, C.POINTER(Hparams), C.POINTER(ScaleState),
                                    C.POINTER(Scalars), C.POINTER(Result)]),
            "or_adamw_array": (None, [i64, vp, C.POINTER(Scalars), vp, vp, vp]),
            "or_zero_step": (C.c_int, [i32, i32, i32, vp, i64, i32, vp, vp, vp, vp, vp, vp,
                                       C.POINTER(Hparams), C.POINTER(ScaleState),
                                       C.POINTER(Result)]),
            "or_gather_unit": (C.c_int, [vp, i64, i32, i64, vp, vp]),
            "or_step_reduced": (C.c_int, [i32, i32, vp, i64, i32, vp, vp, vp, vp, vp, vp,
                                          C.POINTER(Hparams), C.POINTER(ScaleState),
                                          C.POINTER(Result)]),
            "or_rs_accumulate": (C.c_int, [i32, i32, vp, i64, i64, vp, vp, i32]),
            "or_local_accumulate": (C.c_int, [i32, i64, vp, vp, i32]),
            "or_reshard": (C.c_int, [vp, i64, i32, vp, vp, i64, i32, vp, i32]),
            "or_bucket_assign": (C.c_int, [vp, i64, i32, i64, vp, C.POINTER(i64)]),
            "or_regen_accum_sumsq": (C.c_int, [i32, i32, i32, i32, u64, i64, dbl, dbl, i64, i64,
                                               C.POINTER(Inject), C.POINTER(dbl),
                                               C.POINTER(i32)]),
            "or_regen_accum_acc": (C.c_int, [i32, i32, i32, i32, u64, i64, dbl, dbl, i64, vp,
                                             C.POINTER(Inject), vp]),
            "or_dp_step": (C.c_int, [i32, i32, i32, i64, vp, vp, vp, vp, vp,
                                     C.POINTER(Hparams), C.POINTER(ScaleState),
                                     C.POINTER(Result)]),
            "or_regen_sumsq": (C.c_int, [i32, i32, u64, i64, dbl, dbl, i64, i64,
                                         C.POINTER(Inject), C.POINTER(dbl), C.POINTER(i32)]),
            "or_regen_acc": (C.c_int, [i32, i32, u64, i64, dbl, dbl, i64, vp,
                                       C.POINTER(Inject), vp]),
            "or_sumsq_array": (C.c_int, [i64, vp, C.POINTER(dbl), C.POINTER(i32)]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(C.c_void_p)


def _ptrs(arrays):
    arr = (C.c_void_p * len(arrays))(*[a.ctypes.data for a in arrays])
    return arr


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with status {rc}")


def grad_stream(step, replica):
    """Stream id of replica `replica`'s gradient at step `step` (steps from 1)."""
    return (int(step) << 20) | int(replica)


# ---- casts ---------------------------------------------------------------
def narrow(dtype, x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().or_cast_array(dtype, x.size, _p(x), _p(out))
    return out


def widen(dtype, h):
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().or_widen_array(dtype, h.size, _p(h), _p(out))
    return out


# ---- generator -------------------------------------------------------------
def splitmix64_outputs(seed, n):
    s = C.c_uint64(seed)
    return [lib().or_splitmix64_next(C.byref(s)) for _ in range(n)]


def normal_z(seed, stream, idx):
    st = lib().or_stream_state(seed, stream)
    return np.array([lib().or_normal_z(st, int(i)) for i in idx], np.float32)


def gen16(n, dtype, seed, stream, logical_base, sigma, scale=1.0):
    out = np.empty(int(n), np.uint16)
    lib().or_gen16(_p(out), int(n), dtype, seed, stream, int(logical_base), sigma, scale)
    return out


def gen32(n, seed, stream, logical_base, sigma):
    out = np.empty(int(n), np.float32)
    lib().or_gen32(_p(out), int(n), seed, stream, int(logical_base), sigma)
    return out


# ---- layout ----------------------------------------------------------------
def layout(seg_numel, seg_unit, n_ranks, mode):
    """Returns (units, psi, psi_pad); units is a numpy record array (UNIT_DTYPE)."""
    seg_numel = np.ascontiguousarray(seg_numel, np.int64)
    seg_unit = np.ascontiguousarray(
        seg_unit if seg_unit is not None else np.zeros(len(seg_numel)), np.int32)
    units = np.zeros(max(1, len(seg_numel)), UNIT_DTYPE)
    nu, psi, psi_pad = C.c_int64(), C.c_int64(), C.c_int64()
    rc = lib().or_layout(_p(seg_numel), _p(seg_unit), len(seg_numel), n_ranks, mode, _p(units),
                         len(units), C.byref(nu), C.byref(psi), C.byref(psi_pad))
    _check(rc, "layout")
    return units[: nu.value].copy(), psi.value, psi_pad.value


def layout_dim0(seg_numel, seg_rows, n_ranks):
    """FSDP2 per-parameter dim-0 layout: (units, psi, psi_pad)."""
    seg_numel = np.ascontiguousarray(seg_numel, np.int64)
    seg_rows = np.ascontiguousarray(seg_rows, np.int64)
    units = np.zeros(max(1, len(seg_numel)), UNIT_DTYPE)
    nu, psi, psi_pad = C.c_int64(), C.c_int64(), C.c_int64()
    rc = lib().or_layout_dim0(_p(seg_numel), _p(seg_rows), len(seg_numel), n_ranks, _p(units),
                              len(units), C.byref(nu), C.byref(psi), C.byref(psi_pad))
    _check(rc, "layout_dim0")
    return units[: nu.value].copy(), psi.value, psi_pad.value


def fsdp2_step(grad_dtype, n_ranks, units, grads, master, exp_avg, exp_avg_sq, grad_shards, hp,
               st):
    units = np.ascontiguousarray(units, UNIT_DTYPE)
    grads = [np.ascontiguousarray(g, np.uint16) for g in grads]
    res = Result()
    _check(lib().or_fsdp2_step(grad_dtype, n_ranks, _p(units), len(units), _ptrs(grads),
                               _ptrs(master), _ptrs(exp_avg), _ptrs(exp_avg_sq),
                               _ptrs(grad_shards), C.byref(hp), C.byref(st), C.byref(res)),
           "fsdp2_step")
    return res


def fsdp2_gather(units, n_ranks, first, count, dtype, master):
    units = np.ascontiguousarray(units, UNIT_DTYPE)
    out = np.empty(int(units[first:first + count]["L"].sum()), np.uint16)
    _check(lib().or_fsdp2_gather(_p(units), len(units), n_ranks, first, count, dtype,
                                 _ptrs(master), _p(out)), "fsdp2_gather")
    return out


def ledger(units, n_ranks, stage):
    units = np.ascontiguousarray(units, UNIT_DTYPE)
    ab, pk = C.c_int64(), C.c_int64()
    _check(lib().or_ledger(_p(units), len(units), n_ranks, stage, C.byref(ab), C.byref(pk)),
           "ledger")
    return ab.value, pk.value


def comm_bytes(psi_pad, n_ranks, variant):
    return lib().or_comm_bytes(int(psi_pad), n_ranks, variant)


# ---- step ------------------------------------------------------------------
def reduce_scatter(dtype, n_ranks, units, grads):
    units = np.ascontiguousarray(units, UNIT_DTYPE)
    s_tot = int(units["S"].sum())
    outs = [np.empty(s_tot, np.float32) for _ in range(n_ranks)]
    grads = [np.ascontiguousarray(g, np.uint16) for g in grads]
    _check(lib().or_reduce_scatter(dtype, n_ranks, _p(units), len(units), _ptrs(grads),
                                   _ptrs(outs)), "reduce_scatter")
    return outs


def finish(sumsq, overflow, n_ranks, hp, st):
    sc, res = Scalars(), Result()
    _check(lib().or_finish(float(sumsq), int(overflow), n_ranks, C.byref(hp), C.byref(st),
                           C.byref(sc), C.byref(res)), "finish")
    return sc, res


def adamw_array(acc, sc, p, m, v):
    acc = np.ascontiguousarray(acc, np.float32)
    for a in (p, m, v):
        assert a.dtype == np.float32 and a.flags.c_contiguous and a.size == acc.size
    lib().or_adamw_array(acc.size, _p(acc), C.byref(sc), _p(p), _p(m), _p(v))


def zero_step(grad_dtype, param_dtype, n_ranks, units, stage, grads, master, exp_avg,
              exp_avg_sq, params_full, param_shards, hp, st):
    """One emulated step for all ranks; arrays are updated in place."""
    units = np.ascontiguousarray(units, UNIT_DTYPE)
    grads = [np.ascontiguousarray(g, np.uint16) for g in grads]
    res = Result()
    pf = _p(params_full) if params_full is not None else None
    ps = _ptrs(param_shards) if param_shards is not None else None
    _check(lib().or_zero_step(grad_dtype, param_dtype, n_ranks, _p(units), len(units), stage,
                              _ptrs(grads), _ptrs(master), _ptrs(exp_avg), _ptrs(exp_avg_sq),
                              pf, ps, C.byref(hp), C.byref(st), C.byref(res)), "zero_step")
    return res


def step_reduced(param_dtype, n_ranks, units, stage, acc, master, exp_avg, exp_avg_sq,
                 params_full, param_shards, hp, st):
    """The optimizer side of a step from already reduced fp32 gradient shards."""
    units = np.ascontiguousarray(units, UNIT_DTYPE)
    res = Result()
    pf = _p(params_full) if params_full is not None else None
    ps = _ptrs(param_shards) if param_shards is not None else None
    _check(lib().or_step_reduced(param_dtype, n_ranks, _p(units), len(units), stage, _ptrs(acc),
                                 _ptrs(master), _ptrs(exp_avg), _ptrs(exp_avg_sq), pf, ps,
                                 C.byref(hp), C.byref(st), C.byref(res)), "step_reduced")
    return res


F32 = 3


def rs_accumulate(grad_dtype, n_ranks, units, u, grads, shards, accumulate):
    """Bucket (unit) u's reduce-scatter of one micro-batch into fp32 shards;
    grads are 16-bit replicas, or fp32 ones when grad_dtype is F32."""
    units = np.ascontiguousarray(units, UNIT_DTYPE)
    gt = np.float32 if grad_dtype == F32 else np.uint16
    grads = [np.ascontiguousarray(g, gt) for g in grads]
    _check(lib().or_rs_accumulate(grad_dtype, n_ranks, _p(units), len(units), u, _ptrs(grads),
                                  _ptrs(shards), int(accumulate)), "rs_accumulate")


def local_accumulate(grad_dtype, grad, acc, accumulate):
    """acc (fp32, in place) += widened 16-bit grad, or = it when not accumulating."""
    grad = np.ascontiguousarray(grad, np.uint16)
    assert acc.dtype == np.float32 and acc.flags.c_contiguous and acc.size == grad.size
    _check(lib().or_local_accumulate(grad_dtype, grad.size, _p(grad), _p(acc), int(accumulate)),
           "local_accumulate")


def reshard(units_a, n_a, shards_a, units_b, n_b):
    """Rank shard buffers under layout A -> new ones under layout B (same
    dtype), by logical index; B's padding is zero."""
    ua = np.ascontiguousarray(units_a, UNIT_DTYPE)
    ub = np.ascontiguousarray(units_b, UNIT_DTYPE)
    shards_a = [np.ascontiguousarray(x) for x in shards_a]
    dt = shards_a[0].dtype
    s_tot = int(ub["S"].sum())
    out = [np.empty(s_tot, dt) for _ in range(n_b)]
    for x in out:  # every byte set, so that padding left unwritten shows
        x.view(np.uint8)[:] = 0xFF
    _check(lib().or_reshard(_p(ua), len(ua), n_a, _ptrs(shards_a), _p(ub), len(ub), n_b,
                            _ptrs(out), dt.itemsize), "reshard")
    return out


def bucket_assign(numel, n_ranks, bucket_numel=0):
    """Megatron bucket id of every segment, and the bucket count."""
    numel = np.ascontiguousarray(numel, np.int64)
    out = np.empty(numel.size, np.int32)
    nb = C.c_int64()
    _check(lib().or_bucket_assign(_p(numel), numel.size, n_ranks, int(bucket_numel), _p(out),
                                  C.byref(nb)), "bucket_assign")
    return out, nb.value


def gather_unit(units, n_ranks, u, param_shards):
    units = np.ascontiguousarray(units, UNIT_DTYPE)
    out = np.empty(int(units[u]["P"]), np.uint16)
    _check(lib().or_gather_unit(_p(units), len(units), n_ranks, u, _ptrs(param_shards),
                                _p(out)), "gather_unit")
    return out


def dp_step(grad_dtype, param_dtype, n_ranks, grads, master, exp_avg, exp_avg_sq, params, hp,
            st):
    grads = [np.ascontiguousarray(g, np.uint16) for g in grads]
    res = Result()
    _check(lib().or_dp_step(grad_dtype, param_dtype, n_ranks, master.size, _ptrs(grads),
                            _p(master), _p(exp_avg), _p(exp_avg_sq), _p(params), C.byref(hp),
                            C.byref(st), C.byref(res)), "dp_step")
    return res


def regen_sumsq(dtype, n_ranks, seed, step, sigma, scale, i0, i1, inject=None):
    ss, nf = C.c_double(), C.c_int32()
    inj = C.byref(inject) if inject is not None else None
    _check(lib().or_regen_sumsq(dtype, n_ranks, seed, step, sigma, scale, int(i0), int(i1), inj,
                                C.byref(ss), C.byref(nf)), "regen_sumsq")
    return ss.value, nf.value


def regen_acc(dtype, n_ranks, seed, step, sigma, scale, idx, inject=None):
    idx = np.ascontiguousarray(idx, np.int64)
    out = np.empty(idx.size, np.float32)
    inj = C.byref(inject) if inject is not None else None
    _check(lib().or_regen_acc(dtype, n_ranks, seed, step, sigma, scale, idx.size, _p(idx), inj,
                              _p(out)), "regen_acc")
    return out


def regen_accum_sumsq(dtype, n_ranks, n_micro, mode, seed, step, sigma, scale, i0, i1,
                      inject=None):
    ss, nf = C.c_double(), C.c_int32()
    inj = C.byref(inject) if inject is not None else None
    _check(lib().or_regen_accum_sumsq(dtype, n_ranks, n_micro, mode, seed, step, sigma, scale,
                                      int(i0), int(i1), inj, C.byref(ss), C.byref(nf)),
           "regen_accum_sumsq")
    return ss.value, nf.value


def regen_accum_acc(dtype, n_ranks, n_micro, mode, seed, step, sigma, scale, idx, inject=None):
    idx = np.ascontiguousarray(idx, np.int64)
    out = np.empty(idx.size, np.float32)
    inj = C.byref(inject) if inject is not None else None
    _check(lib().or_regen_accum_acc(dtype, n_ranks, n_micro, mode, seed, step, sigma, scale,
                                    idx.size, _p(idx), inj, _p(out)), "regen_accum_acc")
    return out


def sumsq_array(x):
    """Squared norm (double, in order) and overflow flag of given values."""
    x = np.ascontiguousarray(x, np.float32)
    ss, nf = C.c_double(), C.c_int32()
    _check(lib().or_sumsq_array(x.size, _p(x), C.byref(ss), C.byref(nf)), "sumsq_array")
    return ss.value, nf.value
