"""The step captured in a HIP graph and replayed.

The library's step, gathers and bucket launches enqueue kernels only (no
memset, copy, allocation or synchronisation; every pointer travels by value
in the kernel arguments), so a caller can capture them once and replay the
graph every step: the device state block carries t, the loss scale and the
skip decision from one replay to the next.  Each case runs a graph-replayed
run beside an eager twin on the same inputs, with eager work (the next
step's gradients, a read of the result) and a synchronisation between the
replays.  Every replay must equal the eager step bit for bit: fp32 state,
16-bit parameters, gradient shards, the gather buffers and the state block.
The eager twin is held to the oracle's bars on the way (the same bars as
the parity tests), so the replays are too.
"""
import numpy as np
import pytest
import torch

import oracle as O  # noqa: F401  (the oracle's library is loaded by OracleRun)
from fsdp_sharded_mixed_amd import workloads as W
from tests import gpu_common as G
from tests import oracle_inputs as OI

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def R():
    from fsdp_sharded_mixed_amd import runner
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return runner


def small(n, layout, lens, gdt=W.BF16, stage=2, seed=31, steps=5, **kw):
    dyn = gdt == W.F16
    segs = [W.Segment(f"s{i}", int(l), i if layout == W.PER_UNIT else 0)
            for i, l in enumerate(lens)]
    return W.Workload(name=f"graph-n{n}-l{layout}-g{gdt}-s{stage}", description="",
                      segments=segs, n_ranks=n, layout=layout, stage=stage, grad_dtype=gdt,
                      param_dtype=gdt, sigma=1e-3, loss_scale=1024.0 if dyn else 1.0,
                      dynamic=dyn, lr=1e-3, steps=steps, seed=seed, max_norm=1.0, **kw)


def set_bits(t, p, bits):
    t.view(torch.int16)[p] = int(np.array(bits, np.uint16).view(np.int16))


def buffers(dev):
    """Everything a step or its gathers write, as host byte arrays."""
    out = {n: getattr(dev, n) for n in ("master", "exp_avg", "exp_avg_sq", "params", "state",
                                        "grad_shards", "unit_buf", "group_buf")}
    if dev.main_grads is not None:
        out.update({f"main_grad{q}": t for q, t in enumerate(dev.main_grads)})
    return {n: t.detach().view(torch.uint8).cpu().numpy() for n, t in out.items()
            if t is not None}


def assert_same(a, b, what):
    ba, bb = buffers(a), buffers(b)
    assert ba.keys() == bb.keys()
    for n in ba:
        assert np.array_equal(ba[n], bb[n]), f"{what}: {n} differs from the eager step"


def one_step(dev):
    if dev.w.backward_rs:
        dev.backward_all()
    dev.step()
    dev.gather_all()


def fill(dev, k, scale, injections):
    if dev.w.backward_rs:
        dev.fill_micro(k, scale)
        bufs = dev.micro_grads[0]
    else:
        dev.fill_grads(k, scale)
        bufs = dev.grads
    for q, p, bits in injections.get(k, []):
        set_bits(bufs[q], p, bits)


def capture(fn, reps=1):
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    torch.cuda.synchronize()
    return g


def check_oracle(dev, orc, res_d, res_o, what):
    G.assert_result_matches(res_d, res_o, what)
    mo, mmo, vo = G.oracle_padded_state(orc)
    G.assert_state_close("master", G.f32(dev.master), mo)
    G.assert_state_close("exp_avg", G.f32(dev.exp_avg), mmo)
    G.assert_state_close("exp_avg_sq", G.f32(dev.exp_avg_sq), vo)
    if dev.params is not None:
        po = G.oracle_padded_params(orc)
        assert G.ulp16_distance(G.bits16(dev.params), po).max() <= 1, f"{what}: params"


def graph_pair(R, w, steps, injections=None, oracle=True):
    """Eager twin and graph replays side by side, one step per replay."""
    injections = injections or {}
    G.say(f"case {w.name} psi={w.psi} N={w.n_ranks} steps={steps} (graph replay)")
    eag = R.DeviceRun(w, resident_micro=True)
    gr = R.DeviceRun(w, resident_micro=True)
    eag.init_state()
    gr.init_state()
    orc = OI.OracleRun(w) if oracle else None
    graph = None
    skipped = 0
    for k in range(1, steps + 1):
        scale = eag.loss_scale
        assert gr.loss_scale == scale
        fill(eag, k, scale, injections)
        fill(gr, k, scale, injections)
        one_step(eag)
        if graph is None:  # captured after the eager twin has loaded every kernel
            graph = capture(lambda: one_step(gr))
        graph.replay()
        torch.cuda.synchronize()
        res_e, res_g = eag.result(), gr.result()
        eag.loss_scale = gr.loss_scale = res_e.scale_next
        skipped += res_e.skipped
        assert (res_g.t, res_g.skipped, res_g.scale_next) == (res_e.t, res_e.skipped,
                                                              res_e.scale_next)
        assert_same(gr, eag, f"{w.name} step {k}")
        if orc is not None:
            grads = OI.replicas(w, orc.units, orc.psi_pad, k, scale)
            for q, p, bits in injections.get(k, []):
                grads[q][p] = bits
            res_o = orc.step(grads)
            check_oracle(eag, orc, res_e, res_o, f"{w.name} step {k}")
    return skipped


def test_tiny_stage3_with_unit_gathers(R):
    """The 5-layer MLP (N = 4) at stage 3: each replay holds the step and the
    five unit gathers."""
    w = W.tiny(3)
    graph_pair(R, w, w.steps)


@pytest.mark.parametrize("n", [3, 8])
def test_fp16_overflow_skip_inside_replay(R, n):
    """fp16 under dynamic loss scaling with an inf at step 2: the replay
    skips on the device (t unchanged, scale halved) and the next replays
    go on from there."""
    w = small(n, W.PER_UNIT, [5003, 77, 20000, 1, 3333], gdt=W.F16, stage=2)
    assert graph_pair(R, w, 5, injections={2: [(n - 1, 9, 0x7C00)]}) == 1


def test_global_flat_materialized(R):
    """N = 8 on one global flat: the sums are materialised in the workspace
    by pass 1 and read back by the update pass within the replay."""
    w = small(8, W.GLOBAL_FLAT, [40001, 17, 9000])
    graph_pair(R, w, 4)


def test_fsdp2_gather_cast(R):
    """FSDP2 (fp32 parameters, per-parameter dim-0 shards): the replay holds
    the step and every group's cast-gather."""
    shapes = [(33, 100), (7, 1), (64, 64), (5, 300), (1, 17)]
    segs = [W.Segment(f"s{i}", r * c, g, rows=r if c > 1 else 0)
            for i, ((r, c), g) in enumerate(zip(shapes, [0, 0, 1, 1, 2]))]
    w = W.Workload(name="graph-fsdp2", description="", segments=segs, n_ranks=2,
                   layout=W.PER_PARAM_DIM0, stage=3, grad_dtype=W.BF16, param_dtype=W.BF16,
                   sigma=1e-3, loss_scale=1.0, dynamic=False, lr=1e-3, steps=4, seed=37,
                   max_norm=1.0, fp32_params=True)
    graph_pair(R, w, 4)


@pytest.mark.parametrize("mode", [W.ACCUM_REDUCE_EACH, W.ACCUM_NO_SYNC])
def test_bucketed_accumulation(R, mode):
    """Three micro-batches reduced bucket by bucket (or accumulated locally,
    no_sync) and the step on the reduced shards, all in one replay; the eager
    twin is checked against the oracle by the accumulation tests, here the
    replays are compared with it bit for bit."""
    segs = [W.Segment(f"s{i}", l, 0) for i, l in enumerate([7001, 333, 12000, 5, 4096])]
    w = W.Workload(name=f"graph-acc-m{mode}", description="", segments=segs, n_ranks=4,
                   layout=W.PER_UNIT, stage=2, grad_dtype=W.F16, param_dtype=W.F16,
                   sigma=1e-2, loss_scale=1024.0, dynamic=True, lr=1e-3, steps=4, seed=43,
                   max_norm=0.5, n_micro=3, accum_mode=mode, bucket_numel=6000)
    graph_pair(R, w, 4, injections={3: [(1, 5, 0x7C00)]}, oracle=False)


def test_several_steps_in_one_graph(R):
    """Three steps in one graph on the same gradients: t advances three times
    per replay, and two replays equal six eager steps."""
    w = small(2, W.GLOBAL_FLAT, [50001, 999])
    eag = R.DeviceRun(w)
    gr = R.DeviceRun(w)
    eag.init_state()
    gr.init_state()
    for d in (eag, gr):
        d.fill_grads(1, 1.0)
    one_step(eag)  # loads the kernels before the capture
    graph = capture(lambda: one_step(gr), reps=3)
    gr.step_no = 0
    graph.replay()
    for _ in range(2):
        one_step(eag)
    torch.cuda.synchronize()
    assert gr.result().t == 3
    assert_same(gr, eag, "after one replay")
    graph.replay()
    for _ in range(3):
        one_step(eag)
    torch.cuda.synchronize()
    assert gr.result().t == 6
    assert_same(gr, eag, "after two replays")
