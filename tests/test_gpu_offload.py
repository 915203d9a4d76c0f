"""GPU parity of the ZeRO-Offload step (zf_offload_step): the GPU reduces,
the host runs CPU-Adam on its fp32 state, the 16-bit parameters come back
in chunks.  Given the device's own step scalars the host update is the
device update's arithmetic, so the offload step must equal zf_shard_step
bit for bit; against the oracle the usual bars hold.
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


def wl(n, layout, lens, gdt=W.BF16, stage=2, offload=True, seed=51, max_norm=0.5, **kw):
    dyn = gdt == W.F16
    segs = [W.Segment(f"s{i}", int(l), i if layout == W.PER_UNIT else 0)
            for i, l in enumerate(lens)]
    w = W.Workload(name=f"off-n{n}-g{gdt}-s{stage}", description="", segments=segs, n_ranks=n,
                   layout=layout, stage=stage, grad_dtype=gdt, param_dtype=gdt, sigma=1e-2,
                   loss_scale=1024.0 if dyn else 1.0, dynamic=dyn, lr=1e-3, steps=5, seed=seed,
                   max_norm=max_norm, offload=offload)
    for k, v in kw.items():
        setattr(w, k, v)
    return w


def same_bits(a, b, what):
    a, b = a.detach().cpu(), b.detach().cpu()
    if a.dtype == torch.float32:
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), what
    else:
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), what


def run_both(R, w_off, w_dev, steps, inject_step=None, chunks=8, threads=0):
    """Offload and device-only runs side by side on the same inputs."""
    G.say(f"case {w_off.name} psi={w_off.psi} chunks={chunks} threads={threads}")
    d_off, d_dev = R.DeviceRun(w_off), R.DeviceRun(w_dev)
    d_off.n_chunks, d_off.n_threads = chunks, threads
    for d in (d_off, d_dev):
        d.init_state()
    same_bits(d_off.master, d_dev.master, "init")
    for k in range(1, steps + 1):
        for d in (d_off, d_dev):
            if d.w.inject_step is None and inject_step == k:
                d.w.inject_step = k
            d.run_workload_step()
        r_off, r_dev = d_off.last_result, d_dev.result()
        assert (r_off.skipped, r_off.t, r_off.scale_next, r_off.sumsq, r_off.gs) == \
            (r_dev.skipped, r_dev.t, r_dev.scale_next, r_dev.sumsq, r_dev.gs)
        for name in ("master", "exp_avg", "exp_avg_sq", "params"):
            same_bits(getattr(d_off, name), getattr(d_dev, name), f"{name} step {k}")
    return d_off, d_dev


@pytest.mark.parametrize("n", [1, 2, 3, 8])
def test_offload_equals_device_step(R, n):
    """Global flat, bf16, ragged length: five steps, offload == device."""
    lens = [40001, 17, 9000]
    run_both(R, wl(n, W.GLOBAL_FLAT, lens), wl(n, W.GLOBAL_FLAT, lens, offload=False), 5)


@pytest.mark.parametrize("stage", [2, 3])
def test_offload_fp16_dynamic_skip(R, stage):
    """Per-unit layout with padding, fp16 under dynamic loss scaling, an
    overflow at step 3 (nothing moves, the scale halves), stages 2 and 3."""
    lens = [37, 5, 101, 6400, 3]
    w1 = wl(3, W.PER_UNIT, lens, gdt=W.F16, stage=stage, inject_replica=2)
    w2 = wl(3, W.PER_UNIT, lens, gdt=W.F16, stage=stage, offload=False, inject_replica=2)
    d_off, _ = run_both(R, w1, w2, 5, inject_step=3)
    assert d_off.last_result.scale_next == 512.0


@pytest.mark.parametrize("chunks,threads", [(1, 1), (3, 5), (64, 2), (4096, 0)])
def test_offload_chunks_and_threads(R, chunks, threads):
    """Pipeline depth and thread count change nothing but the timing."""
    lens = [100003, 77]
    run_both(R, wl(2, W.GLOBAL_FLAT, lens), wl(2, W.GLOBAL_FLAT, lens, offload=False), 3,
             chunks=chunks, threads=threads)


def test_offload_with_bucketed_accumulation(R):
    """The backward-side bucketed reduction with accumulation feeding the
    offload step (the reduced shards go down): equals the device path."""
    lens = [3, 1, 2, 9001, 5, 7, 1200, 2, 4100, 13]
    kw = dict(n_micro=3, bucket_numel=6)
    run_both(R, wl(4, W.PER_UNIT, lens, **kw), wl(4, W.PER_UNIT, lens, offload=False, **kw), 3)


def test_offload_against_oracle(R):
    """The offload step against the CPU oracle, to the usual bars."""
    w = wl(4, W.PER_UNIT, [37, 5, 101, 6400, 3], gdt=W.F16)
    dev = R.DeviceRun(w)
    dev.init_state()
    orc = OI.OracleRun(w)
    for k in range(1, 5):
        scale = orc.st.loss_scale
        grads = OI.replicas(w, orc.units, orc.psi_pad, k, scale)
        dev.fill_grads(k, scale)
        res_o = orc.step(grads)
        dev.step()
        res_d = dev.last_result
        dev.loss_scale = res_d.scale_next
        G.assert_result_matches(res_d, res_o, f"step {k}")
        mo, mmo, vo = G.oracle_padded_state(orc)
        G.assert_state_close("master", dev.master.numpy(), mo)
        G.assert_state_close("exp_avg", dev.exp_avg.numpy(), mmo)
        G.assert_state_close("exp_avg_sq", dev.exp_avg_sq.numpy(), vo)
        po = G.oracle_padded_params(orc)
        assert G.ulp16_distance(G.bits16(dev.params), po).max() <= 1


@pytest.mark.parametrize("gdt,n", [(W.BF16, 2), (W.F16, 3), (W.BF16, 8)])
def test_offload16_against_oracle(R, gdt, n):
    """The 16-bit download (the pages' fp16 gradient edge): the sums are
    rounded to the gradient dtype on the GPU, the norm and overflow check use
    the rounded values, CPU-Adam widens them.  Against the oracle doing the
    same: the downloaded sums bit-exact, state within 4 ulp, params within
    1 ulp, norm within 1e-5, over five steps (a fp16 loss scale that halves)."""
    w = wl(n, W.PER_UNIT, [37, 5, 101, 64001, 3, 9000], gdt=gdt, offload_down16=True)
    dev = R.DeviceRun(w)
    dev.init_state()
    orc = OI.OracleRun(w)
    for k in range(1, 6):
        scale = orc.st.loss_scale
        grads = OI.replicas(w, orc.units, orc.psi_pad, k, scale)
        if k == 3:
            grads[0][orc.units[3]["O"] + 7] = OI.inf_bits(gdt)
        dev.fill_grads(k, scale)
        if k == 3:
            dev.grads[0].view(torch.int16)[orc.units[3]["O"] + 7] = \
                int(np.array(OI.inf_bits(gdt), np.uint16).view(np.int16))
        res_o = orc.step(grads)
        dev.step()
        res_d = dev.last_result
        dev.loss_scale = res_d.scale_next
        G.assert_result_matches(res_d, res_o, f"step {k}")
        assert res_d.skipped == (k == 3)
        if not res_d.skipped:
            sums = O.reduce_scatter(gdt, n, orc.units, grads)
            ref16 = OI.rank_shards_to_padded(orc.units, [O.narrow(gdt, a) for a in sums])
            got16 = dev.h_grad.view(torch.int16)[:orc.psi_pad].numpy().view(np.uint16)
            assert np.array_equal(got16, ref16)
        mo, mmo, vo = G.oracle_padded_state(orc)
        G.assert_state_close("master", dev.master.numpy(), mo)
        G.assert_state_close("exp_avg", dev.exp_avg.numpy(), mmo)
        G.assert_state_close("exp_avg_sq", dev.exp_avg_sq.numpy(), vo)
        assert G.ulp16_distance(G.bits16(dev.params), G.oracle_padded_params(orc)).max() <= 1


def test_offload16_overflow_only_in_16_bits(R):
    """fp16 replicas whose fp32 sum is finite but beyond fp16's range: the
    plain step applies, the 16-bit download sees +inf and skips (and the
    dynamic loss scale halves), exactly as the oracle doing the same."""
    lens = [4096]
    results = {}
    for down16 in (False, True):
        w = wl(2, W.GLOBAL_FLAT, lens, gdt=W.F16, offload_down16=down16)
        dev = R.DeviceRun(w)
        dev.init_state()
        dev.fill_grads(1, w.loss_scale)
        big = int(np.array(0x7BFF, np.uint16).view(np.int16))  # 65504, the largest fp16
        for q in range(2):
            dev.grads[q].view(torch.int16)[10] = big
        dev.step()
        results[down16] = dev.last_result
    assert results[False].skipped == 0
    assert results[True].skipped == 1 and results[True].scale_next == 512.0
