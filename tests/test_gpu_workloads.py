"""GPU parity at full size for the workloads whose every element the full
oracle harness (test_gpu_full_parity.py) does not carry: a plan with
padding whose materialised sums lie past the memory-side cache window, the
bucketed backward-side reduction over micro-batches (both accumulation
schemes) and ZeRO-Offload, in the launch configuration the bench times;
and the full-size determinism of every workload.

These are checked by regeneration: the exact global squared norm and
overflow flag of every step come from re-deriving every reduced gradient on
the host (a thread pool over index ranges, partials added in order), and a
sample of elements -- random indices, every rank's shard edges, norm
weights, the injected index and its neighbours -- is carried through the
oracle's element update and compared with the device every step.
"""
import numpy as np
import pytest
import torch

import oracle as O
from fsdp_sharded_mixed_amd import workloads as W
from tests import gpu_common as G
from tests import oracle_inputs as OI

pytestmark = pytest.mark.gpu


def sample_indices(w, plan, k=4096, extra=()):
    rng = np.random.default_rng(w.seed)
    idx = set(int(i) for i in rng.integers(0, w.psi, k))
    for u in plan.units:
        for r in range(w.n_ranks):
            for j in (u.lam + r * u.S, u.lam + r * u.S + u.S - 1):
                if u.lam <= j < u.lam + u.L:
                    idx.add(int(j))
    for a, b in w.norm_ranges()[:4]:
        idx.update({a, a + 1, b - 1})
    idx.update({0, w.psi - 1})
    idx.update(int(e) for e in extra if 0 <= e < w.psi)
    return np.array(sorted(idx), np.int64)


def padded_of(plan, idx):
    lam = np.array([u.lam for u in plan.units], np.int64)
    off = np.array([u.O for u in plan.units], np.int64)
    k = np.searchsorted(lam, idx, side="right") - 1
    return off[k] + (idx - lam[k])


def take(t, pidx):
    return t[torch.from_numpy(pidx).to(t.device)].cpu()


def check_samples(dev, so, pidx, what):
    m = take(dev.master, pidx).numpy()
    ea = take(dev.exp_avg, pidx).numpy()
    eas = take(dev.exp_avg_sq, pidx).numpy()
    G.assert_state_close(f"{what} master", m, so.p)
    G.assert_state_close(f"{what} exp_avg", ea, so.m)
    G.assert_state_close(f"{what} exp_avg_sq", eas, so.v)
    if dev.params is not None:
        prm = take(dev.params.view(torch.int16), pidx).numpy().view(np.uint16)
        ref = O.narrow(dev.w.param_dtype, so.p)
        assert G.ulp16_distance(prm, ref).max() <= 1, f"{what} params"
    return float((m.view(np.uint32) == so.p.view(np.uint32)).mean())


def run_workload(R, name, rs_check_step=1):
    w = W.get(name) if isinstance(name, str) else name
    G.say(f"workload {w.name}: Psi={w.psi:,} N={w.n_ranks} stage={w.stage} steps={w.steps}")
    dev = R.DeviceRun(w)
    dev.init_state()
    from fsdp_sharded_mixed_amd import inputs as I
    inj = I.inject_index(w, w.psi) if w.inject_step else None
    extra = [] if inj is None else [inj - 1, inj, inj + 1]
    idx = sample_indices(w, dev.plan, extra=extra)
    pidx = padded_of(dev.plan, idx)
    so = G.SampledOracle(w, w.psi, idx)
    assert np.array_equal(take(dev.master, pidx).numpy().view(np.uint32), so.p.view(np.uint32))
    trace = []
    for k in range(1, w.steps + 1):
        scale = dev.loss_scale
        if w.backward_rs:
            # every micro-batch filled and reduced bucket by bucket, then the step
            for a in range(w.n_micro):
                dev.fill_grads(k, scale, micro=a)
                if w.inject_step == k and a == 0:
                    dev.inject_inf()
                dev.backward(a)
        else:
            dev.fill_grads(k, scale)
            if w.inject_step == k:
                dev.inject_inf()
        if k == rs_check_step and not w.backward_rs:
            from fsdp_sharded_mixed_amd import zf
            rs = torch.empty(dev.psi_pad, dtype=torch.float32, device=dev.device)
            zf.reduce_scatter(dev.plan, w.grad_dtype, dev.grads, rs)
            ref = O.regen_acc(w.grad_dtype, w.n_ranks, w.seed, k, w.sigma, scale, idx)
            got = take(rs, pidx).numpy()
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), "RS sums"
            del rs
        dev.step()
        res_d = dev.result()
        dev.loss_scale = res_d.scale_next
        res_o = so.step(inject_index=inj if w.inject_step == k else None)
        G.assert_result_matches(res_d, res_o, f"{w.name} step {k}")
        share = check_samples(dev, so, pidx, f"{w.name} step {k}")
        trace.append((k, res_d.skipped, res_d.t, res_d.scale_used, res_d.scale_next,
                      round(res_d.norm, 6), round(res_d.coef, 6), share))
        G.say(f"  step {k}: skipped={res_d.skipped} t={res_d.t} S={res_d.scale_used}->"
              f"{res_d.scale_next} norm={res_d.norm:.6f} (oracle {res_o.norm:.6f}) "
              f"coef={res_d.coef:.6f} exact-share={share:.4f}")
        if (w.fp32_params or w.backward_rs) and not res_d.skipped:
            acc = O.regen_accum_acc(w.grad_dtype, w.n_ranks, w.n_micro, w.accum_mode, w.seed, k,
                                    w.sigma, scale, idx)
            got = take(dev.grad_shards, pidx).numpy()
            assert np.array_equal(got.view(np.uint32), acc.view(np.uint32)), "grad shards"
        if w.fp32_params:
            check_group_gathers(dev, so, idx, w)
        elif w.stage == 3:
            check_unit_gathers(dev, so, idx, w)
    return dev, trace


def check_group_gathers(dev, so, idx, w):
    """FSDP2: cast-gather every group in forward order and check the sampled
    elements (a group buffer holds its parameters unpadded, in order)."""
    ref16 = O.narrow(w.param_dtype, so.p)
    for g, info in enumerate(dev.plan.groups):
        buf = dev.gather_cast(g)
        lam0 = dev.plan.units[info.first_unit].lam
        sel = (idx >= lam0) & (idx < lam0 + info.numel)
        if sel.any():
            k = torch.from_numpy(idx[sel] - lam0).to(buf.device)
            got = buf.view(torch.int16)[k].cpu().numpy().view(np.uint16)
            assert G.ulp16_distance(got, ref16[sel]).max() <= 1, f"group {g}"


def check_unit_gathers(dev, so, idx, w):
    """ZeRO-3: gather every unit into the reused buffer (forward order) and
    check the sampled elements and the unit's padding."""
    ref16 = O.narrow(w.param_dtype, so.p)
    for u, info in enumerate(dev.plan.units):
        buf = dev.gather(u)
        sel = (idx >= info.lam) & (idx < info.lam + info.L)
        if sel.any():
            k = torch.from_numpy(idx[sel] - info.lam).to(buf.device)
            got = buf.view(torch.int16)[k].cpu().numpy().view(np.uint16)
            assert G.ulp16_distance(got, ref16[sel]).max() <= 1, f"unit {u}"
        if info.P > info.L:
            assert torch.all(buf[info.L:info.P].view(torch.int16) == 0)


@pytest.fixture(scope="module")
def R():
    from fsdp_sharded_mixed_amd import runner
    assert torch.cuda.is_available()
    return runner


def test_materialised_sums_beyond_cache_window(R):
    """N = 5 over 120M parameters in three ragged FlatParameter units.  The
    fp32 sums (480 MB) are larger than the size up to which pass 1 keeps a
    share of them in the Infinity Cache, so every sum goes out non-temporal
    and the update pass walks its tiles forward: the materialising path that
    the smaller plans, which all take the cache window, no longer reach.
    Three steps against the oracle, the reduce-scatter sums checked too."""
    w = W.Workload(name="flat-120m-n5", description="three ragged units past the cache window",
                   segments=[W.Segment("a", 50_000_001, 0), W.Segment("b", 40_000_003, 1),
                             W.Segment("c", 30_000_007, 2)],
                   n_ranks=5, layout=W.PER_UNIT, stage=2, grad_dtype=W.BF16,
                   param_dtype=W.BF16, sigma=1e-3, loss_scale=1.0, dynamic=False, lr=1e-4,
                   steps=3, seed=7)
    from fsdp_sharded_mixed_amd import zf
    plan = zf.plan_flat(w.segments, w.n_ranks, w.layout, w.stage)
    assert plan.summary.psi_pad * 4 > 448 << 20, "the plan must be past the cache window"
    dev, trace = run_workload(R, w)
    assert all(t[1] == 0 for t in trace)


@pytest.mark.parametrize("name", ["llama-654m-n2-buckets-a4", "llama-654m-n2-nosync-a4"])
def test_llama654m_bucketed_accumulation(R, name):
    """654M decoder in Megatron's gradient buffer (12 buckets of >= 40M
    elements, last layer first), N = 2, four micro-batches per step: every
    bucket reduce-scattered into the fp32 gradient shards each micro-batch,
    or (no_sync) fp32 local accumulation and one reduction; global norm
    about 3, so clipping is active."""
    dev, trace = run_workload(R, name, rs_check_step=0)
    assert len(dev.plan.groups) == 12
    assert all(t[1] == 0 and abs(t[5] - 3.0) < 0.1 and t[6] < 1.0 for t in trace)


def test_llama654m_offload(R):
    """654M decoder under ZeRO-Offload: the GPU reduces, the fp32 state and
    CPU-Adam live on the host, bf16 parameters come back in chunks."""
    dev, trace = run_workload(R, "llama-654m-n2-offload")
    assert dev.master.device.type == "cpu"
    assert all(t[1] == 0 and abs(t[5] - 3.0) < 0.1 and t[6] < 1.0 for t in trace)


def _device_buffers(dev):
    out = {n: getattr(dev, n) for n in ("master", "exp_avg", "exp_avg_sq", "params", "state",
                                        "grad_shards", "unit_buf", "group_buf")}
    if dev.main_grads is not None:
        out.update({f"main_grad{q}": t for q, t in enumerate(dev.main_grads)})
    return {k: v for k, v in out.items() if v is not None}


@pytest.mark.parametrize("name", ["llama-73m-n8", "llama-654m-n2", "llama-2.1b-n2-zero3",
                                  "llama-2.1b-n2-fsdp2", "llama-4.06b-n2",
                                  "llama-654m-n2-buckets-a4", "llama-654m-n2-nosync-a4",
                                  "llama-654m-n2-offload"])
def test_full_size_determinism(R, name):
    """Two independent runs of the workload's first two steps (fresh state,
    the same seeded inputs, gathers included) leave every buffer bitwise
    identical, and report the same squared norm: the grids and the
    reduction trees are fixed by the plan, never by timing."""
    G.say(f"determinism {name}")
    torch.cuda.empty_cache()
    w = W.get(name)
    runs, norms = [], []
    for _ in range(2):
        dev = R.DeviceRun(w)
        dev.init_state()
        norms.append([dev.run_workload_step().sumsq for _ in range(2)])
        dev.gather_all()
        runs.append(dev)
    torch.cuda.synchronize()
    assert norms[0] == norms[1]
    a, b = _device_buffers(runs[0]), _device_buffers(runs[1])
    assert a.keys() == b.keys()
    for k in a:
        ta, tb = a[k], b[k]
        if ta.dtype.is_floating_point:
            ta, tb = ta.view(torch.int32 if ta.element_size() == 4 else torch.int16), \
                tb.view(torch.int32 if tb.element_size() == 4 else torch.int16)
        assert torch.equal(ta, tb), f"{name}: {k} differs between two runs"
    del runs, a, b
    torch.cuda.empty_cache()
