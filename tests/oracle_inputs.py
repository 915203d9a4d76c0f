"""Seeded inputs for the CPU oracle, built with the oracle's own generator.

Test infrastructure: arrays in the oracle's conventions (replicas as padded
flats, per-rank shard buffers).  Shapes and seeds come from the workload
table; no step arithmetic here.
"""
import ctypes as C

import numpy as np

import oracle as O
from fsdp_sharded_mixed_amd import workloads as W


def unit_ids(w):
    """Unit id of every segment: the workload's own, or the oracle's Megatron
    bucket assignment for a bucketed workload."""
    numel, unit = w.seg_arrays()
    if w.bucket_numel is not None:
        unit, _ = O.bucket_assign(numel, w.n_ranks, w.bucket_numel)
    return numel, list(unit)


def plan(w):
    numel, unit = unit_ids(w)
    if w.layout == W.PER_PARAM_DIM0:
        return O.layout_dim0(numel, [s.rows for s in w.segments], w.n_ranks)
    return O.layout(numel, unit, w.n_ranks, w.layout)


def groups(w):
    """FSDP units as (first parameter, count) for a per-parameter layout."""
    out = []
    _, unit = unit_ids(w)
    for i in range(len(w.segments)):
        if not out or unit[i] != unit[out[-1][0]]:
            out.append([i, 0])
        out[-1][1] += 1
    return [tuple(g) for g in out]


def hparams(w):
    return O.Hparams(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps,
                     weight_decay=w.weight_decay, max_norm=w.max_norm)


def scale_state(w):
    return O.ScaleState(loss_scale=w.loss_scale, t=0, growth_ctr=0,
                        growth_interval=w.growth_interval, dynamic=int(w.dynamic))


def replicas(w, units, psi_pad, step, scale, sigma=None, seed=None, micro=0):
    """N padded replica gradients for `step` (micro-batch `micro`), keyed by
    logical index (pads zero)."""
    sigma = w.sigma if sigma is None else sigma
    seed = w.seed if seed is None else seed
    out = []
    for q in range(w.n_ranks):
        g = np.zeros(psi_pad, np.uint16)
        for u in units:
            g[u["O"]:u["O"] + u["L"]] = O.gen16(u["L"], w.grad_dtype, seed,
                                                W.grad_stream(step, q, micro), u["lam"], sigma,
                                                scale)
        out.append(g)
    return out


def master_logical(w, psi):
    """fp32 master initialisation in logical order."""
    m = O.gen32(psi, w.seed, W.STREAM_MASTER, 0, w.master_sigma)
    if w.norm_weights_one:
        for a, b in w.norm_ranges():
            m[a:b] = 1.0
    return m


def to_rank_shards(units, n_ranks, logical, dtype=np.float32):
    """Split a logical-order array into per-rank shard buffers (pads zero)."""
    s_tot = int(units["S"].sum())
    shards = [np.zeros(s_tot, dtype) for _ in range(n_ranks)]
    for u in units:
        for r in range(n_ranks):
            a = r * u["S"]
            b = min(u["L"], a + u["S"])
            if b > a:
                shards[r][u["M"]:u["M"] + (b - a)] = logical[u["lam"] + a:u["lam"] + b]
    return shards


def rank_shards_to_logical(units, shards):
    """Inverse of to_rank_shards (drops the padding)."""
    psi = int(units["L"].sum())
    out = np.zeros(psi, shards[0].dtype)
    for u in units:
        for r in range(len(shards)):
            a = r * u["S"]
            b = min(u["L"], a + u["S"])
            if b > a:
                out[u["lam"] + a:u["lam"] + b] = shards[r][u["M"]:u["M"] + (b - a)]
    return out


def rank_shards_to_padded(units, shards):
    """Per-rank shard buffers to one padded-flat array (rank r of unit u at O_u + r*S_u)."""
    psi_pad = int(units["P"].sum())
    out = np.zeros(psi_pad, shards[0].dtype)
    for u in units:
        for r in range(len(shards)):
            out[u["O"] + r * u["S"]:u["O"] + (r + 1) * u["S"]] = shards[r][u["M"]:u["M"] + u["S"]]
    return out


def padded_to_logical(units, padded):
    return np.concatenate([padded[u["O"]:u["O"] + u["L"]] for u in units])


class OracleRun:
    """An oracle model state for a workload, stepped with O.zero_step."""

    def __init__(self, w, units=None, psi=None, psi_pad=None):
        self.w = w
        if units is None:
            units, psi, psi_pad = plan(w)
        self.units, self.psi, self.psi_pad = units, psi, psi_pad
        n = w.n_ranks
        self.master = to_rank_shards(units, n, master_logical(w, psi))
        s_tot = int(units["S"].sum())
        self.m = [np.zeros(s_tot, np.float32) for _ in range(n)]
        self.v = [np.zeros(s_tot, np.float32) for _ in range(n)]
        init16 = O.narrow(w.param_dtype, np.concatenate(self.master))
        self.grad_shards = None
        if w.backward_rs:
            self.grad_shards = [np.zeros(s_tot, np.float32) for _ in range(n)]
        if w.fp32_params:
            # FSDP2: fp32 parameters (no 16-bit copy) and fp32 grad shards
            self.full = self.shards = None
            self.grad_shards = [np.zeros(s_tot, np.float32) for _ in range(n)]
        elif w.stage < 3:
            self.full = rank_shards_to_padded(
                units, [init16[r * s_tot:(r + 1) * s_tot] for r in range(n)])
            self.shards = None
        else:
            self.full = None
            self.shards = [init16[r * s_tot:(r + 1) * s_tot].copy() for r in range(n)]
        self.hp = hparams(w)
        self.st = scale_state(w)
        self.step_no = 0

    def backward(self, micro_grads):
        """The backward-side reduction of one step's micro-batches into the
        fp32 gradient shards, bucket by bucket (O.rs_accumulate), either for
        every micro-batch or, no_sync, once over fp32 local accumulations."""
        w, units = self.w, self.units
        if w.accum_mode == W.ACCUM_REDUCE_EACH:
            for a, grads in enumerate(micro_grads):
                for u in range(len(units)):
                    O.rs_accumulate(w.grad_dtype, w.n_ranks, units, u, grads, self.grad_shards,
                                    a > 0)
        else:
            loc = [np.zeros(self.psi_pad, np.float32) for _ in range(w.n_ranks)]
            for a, grads in enumerate(micro_grads):
                for q in range(w.n_ranks):
                    O.local_accumulate(w.grad_dtype, grads[q], loc[q], a > 0)
            for u in range(len(units)):
                O.rs_accumulate(O.F32, w.n_ranks, units, u, loc, self.grad_shards, False)

    def step(self, grads=None):
        self.step_no += 1
        if self.w.backward_rs:
            micro_grads = grads
            if micro_grads is None:
                micro_grads = [replicas(self.w, self.units, self.psi_pad, self.step_no,
                                        self.st.loss_scale, micro=a)
                               for a in range(self.w.n_micro)]
                if self.w.inject_step == self.step_no:
                    inject_inf(self.w, self.units, micro_grads[0])
            self.backward(micro_grads)
            return O.step_reduced(self.w.param_dtype, self.w.n_ranks, self.units, self.w.stage,
                                  self.grad_shards, self.master, self.m, self.v, self.full,
                                  self.shards, self.hp, self.st)
        if grads is None:
            grads = replicas(self.w, self.units, self.psi_pad, self.step_no, self.st.loss_scale)
            if self.w.inject_step == self.step_no:
                inject_inf(self.w, self.units, grads)
        if self.w.offload and self.w.offload_down16:
            # the sums rounded to the gradient dtype, then the step from them
            w = self.w
            acc = O.reduce_scatter(w.grad_dtype, w.n_ranks, self.units, grads)
            acc = [O.widen(w.grad_dtype, O.narrow(w.grad_dtype, a)) for a in acc]
            return O.step_reduced(w.param_dtype, w.n_ranks, self.units, w.stage, acc,
                                  self.master, self.m, self.v, self.full, self.shards, self.hp,
                                  self.st)
        if self.w.fp32_params:
            return O.fsdp2_step(self.w.grad_dtype, self.w.n_ranks, self.units, grads,
                                self.master, self.m, self.v, self.grad_shards, self.hp, self.st)
        return O.zero_step(self.w.grad_dtype, self.w.param_dtype, self.w.n_ranks, self.units,
                           self.w.stage, grads, self.master, self.m, self.v, self.full,
                           self.shards, self.hp, self.st)


def inject_index(w, psi):
    """Logical index that receives the injected +inf: first output of the inject stream."""
    # output 0 of a splitmix64 generator whose state starts at the stream's state
    state = C.c_uint64(O.lib().or_stream_state(w.seed, W.STREAM_INJECT))
    return int(O.lib().or_splitmix64_next(C.byref(state)) % psi)


def inf_bits(dtype):
    return 0x7C00 if dtype == W.F16 else 0x7F80


def inject_inf(w, units, grads):
    psi = int(units["L"].sum())
    i = inject_index(w, psi)
    for u in units:
        if u["lam"] <= i < u["lam"] + u["L"]:
            grads[w.inject_replica][u["O"] + (i - u["lam"])] = inf_bits(w.grad_dtype)
            return i
    raise AssertionError("inject index outside every unit")
