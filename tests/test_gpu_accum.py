"""GPU parity of the backward-side path: bucket-by-bucket reduce-scatter
with gradient accumulation (every micro-batch reduced into the fp32
gradient shards, or no_sync local fp32 accumulation reduced once), and the
step that consumes the reduced shards -- through the C ABI, against the CPU
oracle.

Bars: the fp32 gradient shards (reduced and accumulated sums), overflow,
skip, gathered layout and padding bit-exact; fp32 state within 4 ulp;
16-bit params within 1 ulp; norm within 1e-5.
"""
import numpy as np
import pytest
import torch

import oracle as O
from fsdp_sharded_mixed_amd import workloads as W
from tests import gpu_common as G
from tests import oracle_inputs as OI

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def R():
    from fsdp_sharded_mixed_amd import runner
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return runner


def bucketed(n, lens, bucket, gdt=W.BF16, stage=2, mode=W.ACCUM_REDUCE_EACH, n_micro=3,
             seed=41, max_norm=0.5, layout=W.PER_UNIT, rows=None, fp32_params=False,
             units=None):
    """Segments in buffer order, cut into buckets of `bucket` elements by each
    side's own bucket planner (units=None), or given FSDP units."""
    dyn = gdt == W.F16
    segs = [W.Segment(f"s{i}", int(l), 0 if units is None else units[i],
                      rows=0 if rows is None else rows[i]) for i, l in enumerate(lens)]
    return W.Workload(name=f"acc-n{n}-m{mode}-a{n_micro}-g{gdt}-s{stage}", description="",
                      segments=segs, n_ranks=n, layout=layout, stage=stage, grad_dtype=gdt,
                      param_dtype=gdt, sigma=1e-2, loss_scale=1024.0 if dyn else 1.0,
                      dynamic=dyn, lr=1e-3, steps=4, seed=seed, max_norm=max_norm,
                      n_micro=n_micro, accum_mode=mode,
                      bucket_numel=bucket if units is None else None,
                      fp32_params=fp32_params)


def set_bits(t, p, bits):
    t.view(torch.int16)[p] = int(np.array(bits, np.uint16).view(np.int16))


def assert_f32_bits(got, ref, what):
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), what
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32)), what


def run_accum_pair(R, w, steps, inject=None, reverse_buckets=False):
    """Device and oracle step by step: every micro-batch filled on both sides
    from the same generator, reduced bucket by bucket, then the step.
    inject: {step: (replica, padded index, bits)} into micro-batch 0."""
    G.say(f"case {w.name} psi={w.psi} N={w.n_ranks} A={w.n_micro} mode={w.accum_mode}")
    dev = R.DeviceRun(w)
    dev.init_state()
    orc = OI.OracleRun(w)
    assert (dev.plan.summary.n_units, dev.psi_pad) == (len(orc.units), orc.psi_pad)
    m0, _, _ = G.oracle_padded_state(orc)
    assert np.array_equal(G.bits32(dev.master), m0.view(np.uint32)), "master init"
    for k in range(1, steps + 1):
        scale = orc.st.loss_scale
        micro = []
        for a in range(w.n_micro):
            reps = OI.replicas(w, orc.units, orc.psi_pad, k, scale, micro=a)
            dev.fill_grads(k, scale, micro=a)
            if inject and k in inject and a == 0:
                q, p, bits = inject[k]
                reps[q][p] = bits
                set_bits(dev.grads[q], p, bits)
            for q in range(w.n_ranks):
                assert np.array_equal(G.bits16(dev.grads[q]), reps[q]), "grad input"
            micro.append(reps)
            if reverse_buckets and w.accum_mode == W.ACCUM_REDUCE_EACH:
                from fsdp_sharded_mixed_amd import zf
                for g in reversed(range(len(dev.plan.groups))):
                    zf.bucket_reduce_scatter(dev.plan, g, w.grad_dtype, dev.grads,
                                             dev.grad_shards, a > 0)
            else:
                dev.backward(a)
        res_o = orc.step(micro)
        # the reduced, accumulated gradients are bit-exact before the step
        assert_f32_bits(G.f32(dev.grad_shards),
                        OI.rank_shards_to_padded(orc.units, orc.grad_shards),
                        f"grad shards step {k}")
        dev.step()
        res_d = dev.result()
        dev.loss_scale = res_d.scale_next
        G.assert_result_matches(res_d, res_o, f"{w.name} step {k}")
        mo, mmo, vo = G.oracle_padded_state(orc)
        G.assert_state_close("master", G.f32(dev.master), mo)
        G.assert_state_close("exp_avg", G.f32(dev.exp_avg), mmo)
        G.assert_state_close("exp_avg_sq", G.f32(dev.exp_avg_sq), vo)
        if dev.params is not None:
            po = G.oracle_padded_params(orc)
            assert G.ulp16_distance(G.bits16(dev.params), po).max() <= 1, "params"
        pad = np.ones(orc.psi_pad, bool)
        for u in orc.units:
            pad[u["O"]:u["O"] + u["L"]] = False
        if pad.any():
            for t in (dev.master, dev.exp_avg, dev.exp_avg_sq):
                assert np.all(G.bits32(t)[pad] == 0)
        if w.fp32_params:
            for g, (first, count) in enumerate(OI.groups(w)):
                got16 = G.bits16(dev.gather_cast(g))
                ref16 = O.fsdp2_gather(orc.units, w.n_ranks, first, count, w.param_dtype,
                                       orc.master)
                assert G.ulp16_distance(got16, ref16).max() <= 1, f"group {g}"
        elif w.stage == 3:
            for u in range(len(orc.units)):
                assert np.array_equal(G.bits16(dev.gather(u)),
                                      O.gather_unit(orc.units, w.n_ranks, u, orc.shards))
    return dev, orc


# buckets of odd sizes: offsets that are not multiples of 4, buckets shorter
# than a quad, and one spanning several 2048-element tiles with a ragged end
LENS = [3, 1, 2, 9001, 5, 7, 1200, 2, 4100, 13]


@pytest.mark.parametrize("n", [1, 2, 3, 5, 8, 9])
@pytest.mark.parametrize("mode", [W.ACCUM_REDUCE_EACH, W.ACCUM_NO_SYNC])
def test_bucketed_accumulation(R, n, mode):
    """Every compiled rank count and the run-time-N path (9), both schemes,
    three micro-batches, bf16, overflow injected in micro-batch 0 of step 2."""
    w = bucketed(n, LENS, bucket=6, mode=mode)
    run_accum_pair(R, w, 3, inject={2: (n - 1, 4, 0x7F80)})


@pytest.mark.parametrize("stage", [2, 3])
@pytest.mark.parametrize("mode", [W.ACCUM_REDUCE_EACH, W.ACCUM_NO_SYNC])
def test_fp16_dynamic_accumulation(R, stage, mode):
    """fp16 under dynamic loss scaling (the scale halves after the injected
    overflow and every later micro-batch uses the new scale), stages 2 and 3
    (per-bucket gathers), four micro-batches."""
    w = bucketed(4, LENS, bucket=1000, gdt=W.F16, stage=stage, mode=mode, n_micro=4)
    dev, orc = run_accum_pair(R, w, 4, inject={2: (1, 9000, 0x7C00)})
    assert orc.st.loss_scale == 512.0


def test_one_micro_batch_is_the_plain_step(R):
    """One micro-batch, one bucket over everything: the backward-side path
    then gives the plain step's state bit for bit on the device."""
    w_acc = bucketed(4, [40001, 17, 9000], bucket=10 ** 9, n_micro=1)
    w_acc.layout = W.GLOBAL_FLAT
    w_plain = bucketed(4, [40001, 17, 9000], bucket=None, n_micro=1, units=[0, 0, 0])
    w_plain.layout = W.GLOBAL_FLAT
    assert w_acc.backward_rs and not w_plain.backward_rs
    d1, d2 = R.DeviceRun(w_acc), R.DeviceRun(w_plain)
    for d in (d1, d2):
        d.init_state()
    for k in (1, 2, 3):
        for d in (d1, d2):
            d.run_workload_step()
        for a, b in ((d1.master, d2.master), (d1.exp_avg, d2.exp_avg),
                     (d1.exp_avg_sq, d2.exp_avg_sq), (d1.params, d2.params)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_bucket_order_and_second_stream(R):
    """Buckets touch disjoint ranges: reduced in reverse order, or on a side
    stream that waits on an event, they give the same shards."""
    w = bucketed(3, LENS, bucket=6, n_micro=2)
    run_accum_pair(R, w, 2, reverse_buckets=True)
    dev = R.DeviceRun(w)
    dev.init_state()
    dev.fill_grads(1, 1.0)
    side = torch.cuda.Stream()
    ev = torch.cuda.Event()
    ev.record()
    side.wait_event(ev)
    with torch.cuda.stream(side):
        dev.backward(0, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    ref = dev.grad_shards.clone()
    dev.backward(0)
    assert torch.equal(ref.view(torch.int32), dev.grad_shards.view(torch.int32))


def test_buckets_on_two_concurrent_streams(R):
    """Even buckets on one stream, odd buckets on another, both in flight at
    once, over two accumulating micro-batches: the same shards bit for bit
    as one stream in order."""
    from fsdp_sharded_mixed_amd import zf
    w = bucketed(4, [5003, 77, 20000, 1, 3333, 9000, 12, 4096], bucket=3000, n_micro=2)
    dev = R.DeviceRun(w)
    dev.init_state()
    ng = len(dev.plan.groups)
    assert ng >= 4
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    out = []
    for split in (False, True):
        dev.grad_shards.fill_(float("nan"))  # every bucket must overwrite it
        for micro in range(2):
            dev.fill_grads(1, 1.0, micro=micro)
            ready = torch.cuda.Event()
            ready.record()
            for s in streams:
                s.wait_event(ready)
            for g in range(ng):
                s = streams[g % 2] if split else streams[0]
                zf.bucket_reduce_scatter(dev.plan, g, w.grad_dtype, dev.grads,
                                         dev.grad_shards, micro > 0, stream=s)
            for s in streams:
                torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        out.append(dev.grad_shards.clone())
    assert not torch.isnan(out[0]).any()
    assert torch.equal(out[0].view(torch.int32), out[1].view(torch.int32))


def test_fsdp2_accumulation(R):
    """FSDP2 with torchtitan's default accumulation: every FSDP unit
    reduce-scattered each micro-batch into the fp32 gradient shards
    (one bucket per unit), fp32 parameters, cast at the unit gather."""
    shapes = [(7, 6), (3, 1), (16, 4), (1, 9), (5, 1), (33, 8), (2, 64)]
    units = [0, 0, 1, 2, 2, 2, 3]
    w = bucketed(3, [r * c for r, c in shapes], bucket=None, layout=W.PER_PARAM_DIM0,
                 stage=3, rows=[r if c > 1 else 0 for r, c in shapes], fp32_params=True,
                 units=units, n_micro=3)
    assert w.backward_rs
    run_accum_pair(R, w, 3, inject={2: (2, 11, 0x7F80)})


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
def test_accumulate_offsets_and_lengths(R, dtype):
    """zf_accumulate over sub-ranges at every pair of element offsets modulo
    the vector width (vector and scalar paths, heads and tails), lengths from
    0 to a few tiles, first and later micro-batches."""
    from fsdp_sharded_mixed_amd import zf
    rng = np.random.default_rng(9)
    n_all = 20000
    vals = (rng.standard_normal(n_all) * 3).astype(np.float32)
    g16 = O.narrow(dtype, vals)
    tdt = torch.float16 if dtype == W.F16 else torch.bfloat16
    g_dev = torch.from_numpy(g16.view(np.int16)).to("cuda").view(tdt)
    for go in range(4):
        for ao in range(4):
            for n in (0, 1, 3, 5, 8, 37, 4096, 9001):
                base = (rng.standard_normal(n + 8) * 1e-3).astype(np.float32)
                acc_dev = torch.from_numpy(base.copy()).to("cuda")
                ref = base.copy()
                for first in (True, False):
                    sub = g16[go:go + n]
                    zf.accumulate(dtype, g_dev[go:], acc_dev[ao:], n=n, accumulate=not first)
                    view = ref[ao:ao + n]
                    O.local_accumulate(dtype, sub, view, not first)
                    ref[ao:ao + n] = view
                    got = acc_dev.cpu().numpy()
                    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), \
                        (go, ao, n, first)


def test_fp32_bucket_rs_wide_range(R):
    """The fp32-replica reduce-scatter on values spanning twelve decades
    (rounding in every addition), buckets at odd offsets."""
    from fsdp_sharded_mixed_amd import zf
    n = 5
    w = bucketed(n, LENS, bucket=6, mode=W.ACCUM_NO_SYNC)
    dev = R.DeviceRun(w)
    units = OI.plan(w)[0]
    rng = np.random.default_rng(4)
    reps = [(rng.standard_normal(dev.psi_pad) * 10.0 ** rng.integers(-6, 6, dev.psi_pad))
            .astype(np.float32) for _ in range(n)]
    dreps = [torch.from_numpy(r).to("cuda") for r in reps]
    s_tot = int(units["S"].sum())
    sh = [np.zeros(s_tot, np.float32) for _ in range(n)]
    for acc in (False, True):
        for g in range(len(dev.plan.groups)):
            zf.bucket_reduce_scatter(dev.plan, g, zf.F32, dreps, dev.grad_shards, acc)
            O.rs_accumulate(O.F32, n, units, g, reps, sh, acc)
        assert_f32_bits(G.f32(dev.grad_shards), OI.rank_shards_to_padded(units, sh),
                        f"accumulate={acc}")
