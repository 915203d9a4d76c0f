"""The split of materialised sums around the memory-side cache window, on
small plans, against the oracle.

The step keeps the last 256 MiB of materialised fp32 sums in the chip's
memory-side cache when all of them take 256-448 MiB: pass 1 stores the sums
of its full tiles below the window non-temporal and those inside it with
plain, cache-allocating stores (its ragged last tile one quad at a time),
and the update pass walks its tiles from the last to the first.  Only plans
of 64-117M elements reach that split, so these tests run a test build of the
step (libzf_window_test.so: the same sources and C ABI, with a 1 MiB window
for every plan) on plans of 1-2.5M elements.  Every element is compared
with the oracle after every step: the sums bit for bit (read from fp32
gradient shards given to a twin run, where the same kernels write them),
master / exp_avg / exp_avg_sq within 4 ulp, 16-bit parameters within 1 ulp.
The regular library, which keeps all of these small plans' sums in the
window (every store cache-allocating), must produce the same bits.
"""
import ctypes as C

import numpy as np
import pytest
import torch

import oracle as O
from fsdp_sharded_mixed_amd import build as B
from fsdp_sharded_mixed_amd import workloads as W
from fsdp_sharded_mixed_amd import zf
from tests import gpu_common as G
from tests import oracle_inputs as OI

pytestmark = pytest.mark.gpu

CALLS = ("zf_plan_flat", "zf_plan_info", "zf_plan_free", "zf_state_init", "zf_shard_step",
         "zf_read_result")


@pytest.fixture(scope="module")
def V():
    assert torch.cuda.is_available()
    return zf.load_library(B.LIB_WINDOW_TEST, CALLS)


@pytest.fixture(scope="module")
def R():
    from fsdp_sharded_mixed_amd import runner
    return runner


def workload(n, lengths, layout, gdt=W.BF16, seed=51, steps=3, inject_step=None):
    segs = [W.Segment(f"u{i}", L, i) for i, L in enumerate(lengths)]
    dyn = gdt == W.F16
    return W.Workload(name=f"window-n{n}-{len(lengths)}u", description="", segments=segs,
                      n_ranks=n, layout=layout, stage=2, grad_dtype=gdt, param_dtype=gdt,
                      sigma=1e-3, loss_scale=8192.0 if dyn else 1.0, dynamic=dyn, lr=1e-3,
                      steps=steps, seed=seed, max_norm=0.5, inject_step=inject_step)


def v_plan(V, w):
    arr = (zf.Segment * len(w.segments))(*[zf.Segment(s.numel, s.unit, s.kind, 0)
                                           for s in w.segments])
    h = C.c_void_p()
    assert V.zf_plan_flat(arr, len(w.segments), w.n_ranks, w.layout, w.stage, C.byref(h)) == 0
    s = zf.PlanSummary()
    assert V.zf_plan_info(h.value, C.byref(s)) == 0
    return h.value, s


def v_step(V, plan, dev, grad_shards=None):
    w = dev.w
    gp = (C.c_void_p * w.n_ranks)(*[g.data_ptr() for g in dev.grads])
    a = zf.StepArgs(w.grad_dtype, w.param_dtype, gp, dev.master.data_ptr(),
                    dev.exp_avg.data_ptr(), dev.exp_avg_sq.data_ptr(), dev.params.data_ptr(),
                    None if grad_shards is None else grad_shards.data_ptr(), 0, 0, dev.psi_pad,
                    dev.workspace.data_ptr(), dev.workspace.numel(), dev.state.data_ptr(), None)
    rc = V.zf_shard_step(plan, C.byref(dev.hp), C.byref(a),
                         torch.cuda.current_stream().cuda_stream)
    assert rc == 0, zf.strerror(rc)


def v_result(V, dev):
    out = zf.StepResult()
    assert V.zf_read_result(dev.state.data_ptr(), C.byref(out),
                            torch.cuda.current_stream().cuda_stream) == 0
    return out


def run_case(V, R, w):
    G.say(f"window case {w.name}: Psi={w.psi:,} N={w.n_ranks} layout={w.layout} "
          f"gdt={w.grad_dtype} inject={w.inject_step}")
    vplan, vs = v_plan(V, w)
    try:
        # `a` steps as the bench would (sums in the workspace), `b` with fp32
        # gradient shards (the sums readable), both through the test build;
        # `c` through the regular library, where all of the sums are in the
        # window (every store cache-allocating)
        a, b, c = R.DeviceRun(w), R.DeviceRun(w, grads=False), R.DeviceRun(w, grads=False)
        s = a.plan.summary
        assert (vs.psi_pad, vs.policy, vs.workspace_bytes) == (s.psi_pad, 1, s.workspace_bytes)
        assert s.cached_sums_bytes == s.psi_pad * 4 and vs.cached_sums_bytes == 1 << 20
        assert vs.psi_pad * 4 > 2 * vs.cached_sums_bytes, "the sums must straddle the window"
        b.grads = c.grads = a.grads
        shards = torch.zeros(a.psi_pad, dtype=torch.float32, device=a.device)
        for d in (a, b, c):
            d.init_state()
        for d in (a, b):
            assert V.zf_state_init(d.state.data_ptr(), w.loss_scale, int(w.dynamic),
                                   w.growth_interval, None) == 0
        orc = OI.OracleRun(w)
        units = orc.units
        for k in range(1, w.steps + 1):
            scale = orc.st.loss_scale
            grads = OI.replicas(w, units, orc.psi_pad, k, scale)
            a.fill_grads(k, scale)
            if w.inject_step == k:
                OI.inject_inf(w, units, grads)
                a.inject_inf()
            # the oracle's reduce-scatter (per-rank shard buffers) in the padded flat
            want_sums = OI.rank_shards_to_padded(
                units, O.reduce_scatter(w.grad_dtype, w.n_ranks, units, grads))
            res_o = orc.step(grads)
            v_step(V, vplan, a)
            v_step(V, vplan, b, grad_shards=shards)
            c.step()
            res_d = v_result(V, a)
            G.assert_result_matches(res_d, res_o, f"{w.name} step {k}")
            assert (v_result(V, b).t, c.result().t) == (res_d.t, res_d.t)
            got = G.bits32(shards)
            assert np.array_equal(got, want_sums.view(np.uint32)), f"step {k}: sums"
            mo, mmo, vo = G.oracle_padded_state(orc)
            share = G.assert_state_close("master", G.f32(a.master), mo)
            G.assert_state_close("exp_avg", G.f32(a.exp_avg), mmo)
            G.assert_state_close("exp_avg_sq", G.f32(a.exp_avg_sq), vo)
            pref = G.oracle_padded_params(orc)
            assert G.ulp16_distance(G.bits16(a.params), pref).max() <= 1
            for name in ("master", "exp_avg", "exp_avg_sq", "params"):
                for other in (b, c):
                    assert torch.equal(G.bits_view(getattr(a, name)),
                                       G.bits_view(getattr(other, name))), f"step {k} {name}"
            G.say(f"  step {k}: skipped={res_d.skipped} norm={res_d.norm:.6f} sums bit-exact, "
                  f"master exact share {share:.4f}")
    finally:
        V.zf_plan_free(vplan)


def test_window_split_global_flat_n8(V, R):
    """N = 8, one flat of 2,500,001 elements (ragged last tile)."""
    run_case(V, R, workload(8, [2_500_001], W.GLOBAL_FLAT))


def test_window_split_per_unit_n6_ragged_tail(V, R):
    """N = 6, three ragged FlatParameter units whose padded total leaves a
    tail of two elements after the last quad."""
    w = workload(6, [500_001, 300_007, 200_005], W.PER_UNIT, seed=52)
    assert zf.plan_flat(w.segments, 6, w.layout, 2).summary.psi_pad % 4 == 2
    run_case(V, R, w)


def test_window_split_fp16_skip(V, R):
    """N = 5 (the smallest rank count that materialises the sums), fp16
    under a dynamic loss scale, +inf injected at step 2: the step is
    skipped, the loss scale halves, and the sums still match."""
    run_case(V, R, workload(5, [1_048_579], W.GLOBAL_FLAT, gdt=W.F16, seed=53, steps=4,
                            inject_step=2))
