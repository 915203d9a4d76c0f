"""Host-side checks of the C-ABI libraries (no GPU needed).

The libraries load, export every function their headers declare, and their
host logic (layout plan, ledger, would-be traffic, argument validation)
agrees with the CPU oracle.  No call here reaches a kernel launch: every
invalid-argument call returns before the HIP runtime is touched.
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle as O
from fsdp_sharded_mixed_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")


def _declared(header):
    text = open(os.path.join(INCLUDE, header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:zf|zfi)_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def zf():
    from fsdp_sharded_mixed_amd import zf as Z
    return Z


def test_headers_declare_the_calls():
    names = _declared("zf.h")
    for required in ("zf_plan_flat", "zf_shard_step", "zf_gather"):
        assert required in names
    assert _declared("zf_inputs.h") == sorted(["zfi_fill_normal16", "zfi_fill_normal32",
                                               "zfi_stream_output", "zfi_stream_probe",
                                               "zfi_stream_probe_shaped", "zfi_sqrt_probe",
                                               "zfi_div_probe", "zfi_update_mix_probe"])


@pytest.mark.parametrize("header,lib", [("zf.h", "libzf.so"), ("zf_inputs.h", "libzf_inputs.so")])
def test_library_exports_every_declared_symbol(header, lib):
    path = os.path.join(ROOT, "fsdp_sharded_mixed_amd", lib)
    L = C.CDLL(path)
    for name in _declared(header):
        assert hasattr(L, name), f"{lib} does not export {name}"


def test_binding_covers_every_declared_call(zf):
    assert set(_declared("zf.h")) == set(zf._SIGNATURES)


def _oracle_units(w):
    from tests import oracle_inputs as OI
    return OI.plan(w)


@pytest.mark.parametrize("name", list(W.ALL))
def test_plan_matches_oracle_layout(zf, name):
    from fsdp_sharded_mixed_amd import runner
    w = W.get(name)
    plan = runner.plan_workload(w)
    units, psi, psi_pad = _oracle_units(w)
    s = plan.summary
    assert (s.psi, s.psi_pad, s.n_units) == (psi, psi_pad, len(units))
    for mine, ref in zip(plan.units, units):
        assert (mine.L, mine.P, mine.S, mine.O, mine.lam) == (ref["L"], ref["P"], ref["S"],
                                                                ref["O"], ref["lam"])
    assert s.max_unit_pad == units["P"].max()
    for stage in range(5):
        ab, peak = O.ledger(units, w.n_ranks, stage)
        assert s.state_bytes[stage] == ab
        if stage == 3:
            assert s.stage3_peak_bytes == peak
    for v in range(5):
        assert s.comm_bytes[v] == pytest.approx(O.comm_bytes(psi_pad, w.n_ranks, v), rel=1e-15)


def test_plan_bruteforce_small(zf):
    rng = np.random.default_rng(3)
    for _ in range(300):
        n = int(rng.integers(1, 17))
        k = int(rng.integers(1, 6))
        lens = [int(x) for x in rng.integers(1, 40, k)]
        layout = int(rng.integers(0, 2))
        uid = sorted(int(x) for x in rng.integers(0, k, k)) if layout else [0] * k
        # make unit ids run 0,0,..,1,..
        remap, nxt = {}, 0
        for u in uid:
            if u not in remap:
                remap[u] = nxt
                nxt += 1
        uid = [remap[u] for u in uid]
        plan = zf.plan_flat(list(zip(lens, uid)), n, layout, 2)
        units, psi, psi_pad = O.layout(lens, uid, n, layout)
        assert plan.summary.psi_pad == psi_pad
        assert [(u.P, u.S, u.O) for u in plan.units] == [(u["P"], u["S"], u["O"]) for u in units]


def test_fsdp2_plan_matches_oracle(zf):
    """ZF_PER_PARAM_DIM0 units and groups against the oracle's dim-0 layout."""
    rng = np.random.default_rng(6)
    for _ in range(100):
        n = int(rng.integers(1, 9))
        k = int(rng.integers(1, 8))
        rows = [int(x) for x in rng.integers(1, 30, k)]
        cols = [int(x) for x in rng.integers(1, 6, k)]
        ngroups = int(rng.integers(1, k + 1))
        cuts = sorted(rng.choice(range(1, k), ngroups - 1, replace=False)) if k > 1 else []
        gid, g = [], 0
        for i in range(k):
            if g < len(cuts) and i == cuts[g]:
                g += 1
            gid.append(g)
        segs = [(r * c, gi, 0, r) for r, c, gi in zip(rows, cols, gid)]
        plan = zf.plan_flat(segs, n, zf.PER_PARAM_DIM0, 3)
        units, psi, psi_pad = O.layout_dim0([r * c for r, c in zip(rows, cols)], rows, n)
        assert plan.summary.psi_pad == psi_pad and plan.summary.policy == 2
        assert [(u.L, u.P, u.S, u.O, u.lam) for u in plan.units] == \
            [(u["L"], u["P"], u["S"], u["O"], u["lam"]) for u in units]
        assert plan.summary.n_groups == len(set(gid))
        for gi, grp in enumerate(plan.groups):
            members = [i for i in range(k) if gid[i] == gi]
            assert (grp.first_unit, grp.n_units) == (members[0], len(members))
            assert grp.numel == sum(rows[i] * cols[i] for i in members)
        ab, _ = O.ledger(units, n, 4)
        assert plan.summary.state_bytes[4] == ab
    with pytest.raises(zf.ZfError):
        zf.plan_flat([(10, 0, 0, 3)], 2, zf.PER_PARAM_DIM0, 3)  # 3 rows do not divide 10


def test_policy_and_workspace(zf):
    for n, pol in ((1, 0), (2, 0), (4, 0), (5, 1), (8, 1)):
        plan = zf.plan_flat([(1000, 0)], n, W.GLOBAL_FLAT, 2)
        assert plan.summary.policy == pol
        ws = zf.workspace_bytes(plan)
        if pol:
            assert ws >= plan.summary.psi_pad * 4
        assert ws % 256 == 0


def test_cached_sums_window(zf):
    """The plan reports how many bytes of materialised sums pass 1 keeps in
    the memory-side cache: the last 256 MiB of them when all the sums take
    at most 448 MiB, none when they are recomputed or larger."""
    MiB = 1 << 20
    for numel, n, layout, want in (
            (1000, 8, W.GLOBAL_FLAT, 4000),                       # small: all of them
            (1000, 4, W.GLOBAL_FLAT, 0),                          # recomputed
            (1000, 2, W.PER_PARAM_DIM0, 4000),                    # FSDP2's fp32 shard
            (73_417_728, 8, W.GLOBAL_FLAT, 256 * MiB),            # 280 MiB of sums
            (448 * MiB // 4, 8, W.GLOBAL_FLAT, 256 * MiB),        # exactly at the limit
            (448 * MiB // 4 + 8, 8, W.GLOBAL_FLAT, 0),            # just past it
            (120_000_011, 5, W.GLOBAL_FLAT, 0)):
        plan = zf.plan_flat([(numel, 0)], n, layout, 2)
        assert plan.summary.cached_sums_bytes == want, (numel, n, layout)


def test_plan_errors(zf):
    Z = zf
    with pytest.raises(Z.ZfError) as e:
        Z.plan_flat([(10, 0)], 0, W.GLOBAL_FLAT, 2)
    assert e.value.status == -4
    with pytest.raises(Z.ZfError) as e:
        Z.plan_flat([(10, 0)], Z.MAX_RANKS + 1, W.GLOBAL_FLAT, 2)
    assert e.value.status == -4
    for bad in ([(0, 0)], [(5, 0), (5, 2)], [(5, 1)]):
        with pytest.raises(Z.ZfError) as e:
            Z.plan_flat(bad, 2, W.PER_UNIT, 2)
        assert e.value.status == -1
    with pytest.raises(Z.ZfError):
        Z.plan_flat([(10, 0)], 2, 7, 2)
    with pytest.raises(Z.ZfError):
        Z.plan_flat([(10, 0)], 2, W.GLOBAL_FLAT, 4)
    # launch grids hold at most 2^31 - 1 blocks: the update pass's smallest
    # tiles are 128 threads x 1 quad = 512 elements
    edge = (2 ** 31 - 1) * 512
    Z.plan_flat([(edge, 0)], 2, W.GLOBAL_FLAT, 2)
    with pytest.raises(Z.ZfError) as e:
        Z.plan_flat([(edge + 512, 0)], 2, W.GLOBAL_FLAT, 2)
    assert e.value.status == -4
    assert Z.lib.zf_plan_info(None, C.byref(Z.PlanSummary())) == -1
    assert Z.lib.zf_plan_unit(None, 0, C.byref(Z.UnitInfo())) == -1
    plan = Z.plan_flat([(10, 0)], 2, W.GLOBAL_FLAT, 2)
    assert Z.lib.zf_plan_unit(plan.handle, 1, C.byref(Z.UnitInfo())) == -1
    Z.lib.zf_plan_free(None)  # NULL is allowed
    assert Z.strerror(-2) and Z.strerror(12345) == "unknown status"


def test_every_status_has_its_own_text(zf):
    """Every value of enum zf_status in include/zf.h maps to a text of its
    own (never the fallback for an unknown code), and the binding names
    every one of them."""
    text = open(os.path.join(INCLUDE, "zf.h")).read()
    body = re.search(r"enum zf_status\s*\{(.*?)\};", text, flags=re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    codes = {name: int(val) for name, val in re.findall(r"(ZF_[A-Z]+)\s*=\s*(-?\d+)", body)}
    assert len(codes) >= 8 and codes["ZF_OK"] == 0 and codes["ZF_EUNSUP"] == -7
    texts = {c: zf.strerror(c) for c in codes.values()}
    assert all(t and t != "unknown status" for t in texts.values()), texts
    assert len(set(texts.values())) == len(texts), "two codes share one text"
    assert {zf.STATUS[c] for c in codes.values()} == set(codes)
    assert "AVX2" in zf.strerror(codes["ZF_EUNSUP"])


def test_step_argument_errors_enqueue_nothing(zf):
    """Invalid arguments are rejected before any HIP call (so this runs on a
    machine without a GPU): NULLs, bad dtypes, misaligned pointers."""
    Z = zf
    plan = Z.plan_flat([(100, 0)], 2, W.GLOBAL_FLAT, 2)
    hp = Z.hparams(1e-3)
    ok = 0x10000
    grads = (C.c_void_p * 2)(ok, ok)

    need = Z.workspace_bytes(plan)

    def args(**kw):
        d = dict(grad_dtype=1, param_dtype=1, grads=grads, master=ok, exp_avg=ok, exp_avg_sq=ok,
                 params=ok, grad_shards=None, grads_reduced=0, reserved=0, numel=100,
                 workspace=ok, workspace_size=need, state=ok, phase_events=None)
        d.update(kw)
        return Z.StepArgs(d["grad_dtype"], d["param_dtype"], d["grads"], d["master"],
                          d["exp_avg"], d["exp_avg_sq"], d["params"], d["grad_shards"],
                          d["grads_reduced"], d["reserved"], d["numel"], d["workspace"],
                          d["workspace_size"], d["state"], d["phase_events"])

    step = lambda a, p=plan.handle, h=hp: Z.lib.zf_shard_step(p, C.byref(h), C.byref(a), None)
    assert step(args(), p=None) == -1
    assert step(args(grad_dtype=3)) == -3
    assert step(args(param_dtype=0)) == -3
    assert step(args(master=None)) == -1
    assert step(args(master=ok + 4)) == -2
    assert step(args(params=ok + 8)) == -2
    assert step(args(grads=(C.c_void_p * 2)(ok, None))) == -1
    assert step(args(grads=(C.c_void_p * 2)(ok, ok + 2))) == -2
    assert step(args(state=None)) == -1
    assert step(args(workspace=None)) == -1
    # sizes: a short workspace or short arrays are rejected before any launch
    assert step(args(workspace_size=need - 1)) == -4
    assert step(args(numel=99)) == -4
    assert step(args(), h=Z.hparams(1e-3, beta1=1.0)) == -1
    assert step(args(grad_shards=ok + 4)) == -2
    # an FSDP2 plan needs the fp32 gradient shards
    p2 = Z.plan_flat([(100, 0, 0, 10)], 2, Z.PER_PARAM_DIM0, 3)
    assert p2.summary.policy == 2
    assert Z.lib.zf_shard_step(p2.handle, C.byref(hp),
                               C.byref(args(workspace_size=Z.workspace_bytes(p2))), None) == -1
    assert Z.lib.zf_gather_cast(p2.handle, 1, 1, ok, 100, ok, 100, None) == -1
    assert Z.lib.zf_gather_cast(p2.handle, 0, 3, ok, 100, ok, 100, None) == -3
    assert Z.lib.zf_gather_cast(p2.handle, 0, 1, ok + 4, 100, ok, 100, None) == -2
    assert Z.lib.zf_gather_cast(p2.handle, 0, 1, ok, 99, ok, 100, None) == -4
    assert Z.lib.zf_gather_cast(p2.handle, 0, 1, ok, 100, ok, 99, None) == -4
    assert Z.lib.zf_shard_step(plan.handle, None, C.byref(args()), None) == -1
    assert Z.lib.zf_reduce_scatter(plan.handle, 9, grads, ok, 100, None) == -3
    assert Z.lib.zf_reduce_scatter(plan.handle, 1, grads, ok + 4, 100, None) == -2
    assert Z.lib.zf_reduce_scatter(plan.handle, 1, None, ok, 100, None) == -1
    assert Z.lib.zf_reduce_scatter(plan.handle, 1, grads, ok, 99, None) == -4
    shards = (C.c_void_p * 2)(ok, ok)
    assert Z.lib.zf_gather(plan.handle, 1, 1, shards, ok, 100, None) == -1
    assert Z.lib.zf_gather(plan.handle, 0, 5, shards, ok, 100, None) == -3
    assert Z.lib.zf_gather(plan.handle, 0, 1, (C.c_void_p * 2)(ok, ok + 1), ok, 100, None) == -2
    assert Z.lib.zf_gather(plan.handle, 0, 1, shards, None, 100, None) == -1
    assert Z.lib.zf_gather(plan.handle, 0, 1, shards, ok, 99, None) == -4
    # reduced gradients: the fp32 shards are required, the flag is 0 or 1
    assert step(args(grads_reduced=1, grads=None)) == -1
    assert step(args(grads_reduced=2, grad_shards=ok)) == -1
    assert step(args(reserved=1)) == -1
    assert step(args(grads_reduced=1, grads=None, grad_shards=ok, param_dtype=7)) == -3
    assert step(args(grads_reduced=1, grads=None, grad_shards=ok + 8)) == -2
    # bucket reduce-scatter
    brs = Z.lib.zf_bucket_reduce_scatter
    assert brs(None, 0, 1, grads, ok, 100, 0, None) == -1
    assert brs(plan.handle, 1, 1, grads, ok, 100, 0, None) == -1
    assert brs(plan.handle, -1, 1, grads, ok, 100, 0, None) == -1
    assert brs(plan.handle, 0, 4, grads, ok, 100, 0, None) == -3
    assert brs(plan.handle, 0, 0, grads, ok, 100, 0, None) == -3
    assert brs(plan.handle, 0, 1, None, ok, 100, 0, None) == -1
    assert brs(plan.handle, 0, 1, grads, None, 100, 0, None) == -1
    assert brs(plan.handle, 0, 1, grads, ok + 4, 100, 0, None) == -2
    assert brs(plan.handle, 0, 3, (C.c_void_p * 2)(ok, ok + 8), ok, 100, 0, None) == -2
    assert brs(plan.handle, 0, 1, (C.c_void_p * 2)(None, ok), ok, 100, 0, None) == -1
    assert brs(plan.handle, 0, 1, grads, ok, 99, 0, None) == -4
    assert brs(plan.handle, 0, 1, grads, ok, 100, 2, None) == -1
    # local accumulation (16-bit gradients only; element alignment)
    acc = Z.lib.zf_accumulate
    assert acc(1, None, ok, 10, 0, None) == -1
    assert acc(1, ok, None, 10, 0, None) == -1
    assert acc(3, ok, ok, 10, 0, None) == -3
    assert acc(1, ok + 1, ok, 10, 0, None) == -2
    assert acc(1, ok, ok + 2, 10, 0, None) == -2
    assert acc(1, ok, ok, -1, 0, None) == -1
    assert acc(1, ok, ok, 10, 5, None) == -1
    assert acc(2, ok + 2, ok + 4, 0, 1, None) == 0  # nothing to do: no launch
    # the offload step
    def off(**kw):
        d = dict(grad_dtype=1, param_dtype=1, grads=grads, grad_shards=ok, params=ok, numel=100,
                 workspace=ok, workspace_size=need, state=ok, h_state=ok, h_grad=ok,
                 h_master=ok, h_exp_avg=ok, h_exp_avg_sq=ok, h_params=ok, grads_reduced=0,
                 n_threads=1, n_chunks=2, down16=0, phase_events=None)
        d.update(kw)
        a = Z.OffloadArgs(*[d[f] for f, _ in Z.OffloadArgs._fields_])
        return Z.lib.zf_offload_step(plan.handle, C.byref(hp), C.byref(a), None, None)
    assert off(n_chunks=0) == -1
    assert off(n_chunks=5000) == -1
    assert off(down16=2) == -1
    assert off(down16=1, grads_reduced=1, grads=None) == -1
    assert off(param_dtype=3) == -3
    assert off(h_grad=None) == -1
    assert off(params=None) == -1
    assert off(h_master=ok + 4) == -2
    assert off(params=ok + 2) == -2
    assert off(numel=99) == -4
    assert off(workspace_size=need - 1) == -4
    assert off(grad_dtype=0) == -3
    assert Z.lib.zf_offload_step(None, C.byref(hp), None, None, None) == -1
    # resharding: plans of the same model only, sizes, alignment, no overlap
    rs = Z.lib.zf_reshard
    p3 = Z.plan_flat([(100, 0)], 3, W.GLOBAL_FLAT, 2)
    p_other = Z.plan_flat([(99, 0)], 3, W.GLOBAL_FLAT, 2)
    far = ok + (1 << 20)
    assert rs(plan.handle, p3.handle, ok, 100, far, 102, 3, None) == -1
    assert rs(plan.handle, p_other.handle, ok, 100, far, 102, 4, None) == -1
    assert rs(plan.handle, None, ok, 100, far, 102, 4, None) == -1
    assert rs(plan.handle, p3.handle, None, 100, far, 102, 4, None) == -1
    assert rs(plan.handle, p3.handle, ok + 2, 100, far, 102, 4, None) == -2
    assert rs(plan.handle, p3.handle, ok, 100, far + 1, 102, 2, None) == -2
    assert rs(plan.handle, p3.handle, ok, 99, far, 102, 4, None) == -4
    assert rs(plan.handle, p3.handle, ok, 100, far, 101, 4, None) == -4
    assert rs(plan.handle, p3.handle, ok, 100, ok + 200, 102, 4, None) == -1  # overlap
    assert Z.lib.zf_state_init(None, 1.0, 0, 10, None) == -1
    assert Z.lib.zf_state_init(ok, 0.0, 0, 10, None) == -1
    assert Z.lib.zf_state_init(ok + 4, 1.0, 0, 10, None) == -2
    assert Z.lib.zf_read_result(None, C.byref(Z.StepResult()), None) == -1
    assert Z.state_bytes() == 256


def test_input_library_stream_output_matches_oracle():
    """The host half of the GPU input generator (stream starting state and
    splitmix64 outputs) agrees with the oracle's own implementation."""
    from fsdp_sharded_mixed_amd import inputs as I
    for seed in (0, 1, 5, 2**63 + 7):
        for stream in (0, 1, W.STREAM_MASTER, W.STREAM_INJECT, W.grad_stream(3, 1)):
            st = O.lib().or_stream_state(seed, stream)
            state = C.c_uint64(st)
            for j in range(3):
                assert I.stream_output(seed, stream, j) == O.lib().or_splitmix64_next(
                    C.byref(state))


def test_bucket_plan_matches_oracle(zf):
    """zf_plan_buckets and the oracle's Megatron bucket rule agree on random
    segment lists, explicit and default bucket sizes, and the 654M decoder
    in Megatron's order; bad arguments are rejected."""
    rng = np.random.default_rng(5)
    for trial in range(300):
        k = int(rng.integers(1, 40))
        numel = [int(x) for x in rng.integers(1, 50, k)]
        n = int(rng.integers(1, 65))
        b = int(rng.integers(-1, 120))
        ids, nb = zf.plan_buckets(numel, n, b)
        ref, nref = O.bucket_assign(numel, n, b)
        assert ids == list(ref) and nb == nref
    w = W.get("llama-654m-n2-buckets-a4")
    numel = [s.numel for s in w.segments]
    ids, nb = zf.plan_buckets(numel, 2, 0)
    ref, nref = O.bucket_assign(numel, 2, 0)
    assert ids == list(ref) and nb == nref == 12
    for bad in (([], 2, 0), ([5, 0], 2, 0)):
        with pytest.raises(zf.ZfError):
            zf.plan_buckets(*bad)
    with pytest.raises(zf.ZfError):
        zf.plan_buckets([5], 65, 0)
    # a bucketed plan's groups are the buckets, padded to a multiple of N
    p = zf.plan_flat([(nm, i) for nm, i in zip(numel, ids)], 2, W.PER_UNIT, 2)
    assert p.summary.n_groups == p.summary.n_units == 12
    for g, u in zip(p.groups, p.units):
        assert g.padded == u.P and u.P % 2 == 0 and u.P - u.L < 2


def test_offload_default_size_counts_host_arrays(zf):
    """offload_step's default element count is the smallest over every
    per-element array, the host ones included (h_grad counted in the bytes
    of what comes down: 4 per element, 2 with down16), so a short host array
    is refused with ZF_ESIZE before anything is enqueued instead of being
    overrun by the copies or by CPU-Adam.  Device pointers here are
    addresses the library never dereferences: every call fails validation."""
    Z = zf
    import torch
    plan = Z.plan_flat([(100, 0)], 2, W.GLOBAL_FLAT, 2)
    hp = Z.hparams(1e-3)
    ok = 0x10000
    ws = torch.zeros(Z.workspace_bytes(plan), dtype=torch.uint8)

    # stand-ins for the device arrays: sized, never dereferenced
    grads = [torch.zeros(100, dtype=torch.bfloat16) for _ in range(2)]
    shards, params = torch.zeros(100), torch.zeros(100, dtype=torch.bfloat16)

    def call(down16=False, h_grad=100, h_master=100, h_avg=100, h_avg_sq=100, h_params=100):
        h = dict(h_state=np.zeros(256, np.uint8), h_grad=np.zeros(h_grad, np.float32),
                 h_master=np.zeros(h_master, np.float32), h_exp_avg=np.zeros(h_avg, np.float32),
                 h_exp_avg_sq=np.zeros(h_avg_sq, np.float32),
                 h_params=np.zeros(h_params, np.uint16))
        with pytest.raises(Z.ZfError) as e:
            Z.offload_step(plan, hp, W.BF16, W.BF16, grads, shards, params, ws, ok, stream=0,
                           down16=down16, **h)
        return e.value.status

    assert call(h_master=99) == -4
    assert call(h_avg=99) == -4
    assert call(h_avg_sq=1) == -4
    assert call(h_params=99) == -4
    assert call(h_grad=99) == -4
    # 16-bit sums come down into h_grad's first 2 bytes per element
    assert call(down16=True, h_grad=49) == -4
    # a raw address carries no size: without numel the binding refuses
    with pytest.raises(ValueError):
        Z.offload_step(plan, hp, W.BF16, W.BF16, [ok, ok], ok, ok, ws, ok, ok, ok, ok, ok, ok,
                       ok, stream=0)
    # an explicit numel is the caller's statement of every array's size
    with pytest.raises(Z.ZfError) as e:
        Z.offload_step(plan, hp, W.BF16, W.BF16, [ok, ok], ok, ok, ws, ok, ok, ok, ok, ok, ok,
                       ok, stream=0, numel=99)
    assert e.value.status == -4


def test_noalloc_step_refuses_before_enqueueing(zf):
    """zf_shard_step_noalloc checks its arguments and the scratch it needs
    before it touches the HIP runtime (so this runs without a GPU): a
    caller workspace is refused, and a plan whose workspace does not fit the
    static scratch gets ZF_ESIZE, unless the sums go to the caller's fp32
    gradient shards.  Only failing calls are made here."""
    Z = zf
    hp = Z.hparams(1e-3)
    ok = 0x10000
    cap = Z.NOALLOC_SCRATCH_BYTES
    text = open(os.path.join(INCLUDE, "zf.h")).read()
    assert re.search(r"#define ZF_NOALLOC_SCRATCH_BYTES \(64ll << 20\)", text)

    def call(plan, n, **kw):
        grads = (C.c_void_p * plan.n_ranks)(*([ok] * plan.n_ranks))
        d = dict(grad_dtype=2, param_dtype=2, grads=grads, master=ok, exp_avg=ok,
                 exp_avg_sq=ok, params=ok, grad_shards=None, grads_reduced=0, reserved=0,
                 numel=n, workspace=None, workspace_size=0, state=ok, phase_events=None)
        d.update(kw)
        a = Z.StepArgs(*[d[f] for f, _ in Z.StepArgs._fields_])
        return Z.lib.zf_shard_step_noalloc(plan.handle, C.byref(hp), C.byref(a), None)

    # N = 8 materialises the sums: 20M elements need 80 MB of them
    n = 20_000_000
    big = Z.plan_flat([(n, 0)], 8, W.GLOBAL_FLAT, 2)
    assert big.summary.policy == 1 and big.summary.workspace_bytes > cap
    assert call(big, n) == -4
    assert call(big, n, workspace=ok, workspace_size=big.summary.workspace_bytes) == -1
    assert call(big, n, workspace_size=16) == -1
    assert call(big, n - 1, grad_shards=ok) == -4   # the usual checks still come first
    assert call(big, n, master=ok + 4, grad_shards=ok) == -2
    # the partials alone: past about 8.5e9 elements they do not fit either
    huge_n = 9_000_000_000
    huge = Z.plan_flat([(huge_n, 0)], 2, W.GLOBAL_FLAT, 2)
    assert huge.summary.policy == 0 and huge.summary.workspace_bytes > cap
    assert call(huge, huge_n) == -4
    assert Z.lib.zf_shard_step_noalloc(None, C.byref(hp), None, None) == -1


def test_input_library_probes_refuse_before_launching():
    """The bandwidth probes validate every argument before any HIP call: a
    missing, misaligned or mixed gradient operand, a size that is not a
    whole number of quads, or an unsupported shape returns -1 (the
    addresses below are never dereferenced)."""
    from fsdp_sharded_mixed_amd import inputs as I
    f = I.lib.zfi_update_mix_probe
    a, b, c, p, m, v, o = (0x10000 * k for k in range(1, 8))

    def call(g0=a, g1=b, s=None, p=p, m=m, v=v, o=o, n=1024, t=128, cap=0):
        return f(g0, g1, s, p, m, v, o, n, t, cap, None)

    assert call(g1=None) == -1                       # one replica only
    assert call(g0=None) == -1
    assert call(s=c) == -1                           # replicas and sums both
    assert call(g0=None, g1=None) == -1              # neither
    assert call(g0=None, g1=None, s=c + 4) == -1     # misaligned sums
    assert call(p=p + 8) == -1 and call(o=o + 2) == -1 and call(g1=b + 4) == -1
    assert call(m=None) == -1 and call(o=None) == -1
    assert call(n=0) == -1 and call(n=1026) == -1 and call(n=-4) == -1
    assert call(t=64) == -1 and call(t=512) == -1
    assert call(cap=-1) == -1 and call(cap=9) == -1
    srcs = (C.c_void_p * 8)(*([a] * 8))
    dsts = (C.c_void_p * 8)(*([b] * 8))
    g = I.lib.zfi_stream_probe_shaped
    assert g(srcs, 3, dsts, 1, 1024, 1, 0, None) == -1   # 3 sources
    assert g(srcs, 1, dsts, 1, 1024, 3, 0, None) == -1   # 3 quads per lane
    assert g(srcs, 1, dsts, 1, 1022, 1, 0, None) == -1
    assert g(srcs, 1, dsts, 1, 1024, 1, 9, None) == -1
    srcs[0] = a + 4
    assert g(srcs, 1, dsts, 1, 1024, 1, 0, None) == -1


def test_binding_refuses_unsized_raw_addresses(zf):
    """A raw address carries no size, so the binding's default element
    counts refuse it (ValueError before any library call) instead of
    ignoring it and letting a short buffer pass the library's size check."""
    Z = zf
    import torch
    plan = Z.plan_flat([(100, 0)], 2, W.GLOBAL_FLAT, 2)
    hp = Z.hparams(1e-3)
    t = torch.zeros(100)
    ok = 0x10000
    with pytest.raises(ValueError):
        Z.shard_step(plan, hp, W.BF16, W.BF16, [t, ok], t, t, t, t, t, ok)
    with pytest.raises(ValueError):
        Z.shard_step_noalloc(plan, hp, W.BF16, W.BF16, [t, t], ok, t, t, t, ok)
    with pytest.raises(ValueError):
        Z.reduce_scatter(plan, W.BF16, [t, t], ok)
    with pytest.raises(ValueError):
        Z.bucket_reduce_scatter(plan, 0, W.BF16, [ok, t], t, False)
    with pytest.raises(ValueError):
        Z.accumulate(W.BF16, ok, t)
    with pytest.raises(ValueError):
        Z.gather(plan, 0, W.BF16, [ok, ok], ok)
    with pytest.raises(ValueError):
        Z.reshard(plan, plan, ok, t)
    with pytest.raises(ValueError):
        Z.shard_step(plan, hp, W.BF16, W.BF16, [t, t], t, t, t, t, ok, ok, numel=100)
