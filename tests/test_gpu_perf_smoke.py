"""Performance smoke: the kernels keep their measured bandwidth, relative to
the same GPU's own stream ceiling (so machine-to-machine variance does not
matter).

The ceiling of an access mix is the best of the fixed-shape zfi_stream_probe
and zfi_stream_probe_shaped in six shapes, measured in the same process.
The update pass (4 reads + 4 writes per element, fp32 or a mix of 16-bit
replicas and fp32 state) must reach 85% of the best 4-read/4-write figure,
on the 73M workload (materialised sums) and the 654M one (recomputed sums);
73M's pass 1 (8 replicas in, the fp32 sums out) 85% of the best
8-read/1-write figure.  They run at 97% or more today.  The update pass
must also reach an absolute 70% of the MI355X's 8 TB/s on the bytes it
moves, so that a device-wide slowdown that lowers the probes too (placement,
clocks) still fails; it runs at 78-86% today.  And it must reach 90% of
zfi_update_mix_probe, a kernel that moves the update pass's own 30 bytes
per element (the fp32 sums, or two 16-bit replicas, in; the state in and
out; the 16-bit parameter out) with no arithmetic, best of ten shapes; it
runs at 99-112% of it today.
"""
import pytest
import torch

from fsdp_sharded_mixed_amd import workloads as W

pytestmark = pytest.mark.gpu


SHAPES = ((1, 0), (2, 0), (1, 3), (1, 4), (2, 3), (2, 4))
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, vendor figure


def _probe(I, r, w, n=1 << 28, reps=10):
    """Best GB/s of the fixed probe and the shaped probe in SHAPES, on 1 GiB
    arrays allocated one by one (smaller arrays carved from one allocation
    can share DRAM address bits and read lower)."""
    bufs = [torch.ones(n, device="cuda") for _ in range(r + w)]
    runs = [lambda: I.stream_probe(bufs[:r], bufs[r:])]
    runs += [lambda q=q, c=c: I.stream_probe_shaped(bufs[:r], bufs[r:], q, c) for q, c in SHAPES]
    best = 0.0
    for run in runs:
        for _ in range(3):
            run()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        best = max(best, (r + w) * 4 * n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del bufs
    torch.cuda.empty_cache()
    return best


def _mix_probe(I, replicas, n=1 << 28, reps=10):
    """Best GB/s of zfi_update_mix_probe over its block sizes and occupancy
    caps, on 1 GiB arrays allocated one by one."""
    bufs = [torch.ones(n, device="cuda") for _ in range(6)]
    g = (bufs[0], bufs[1]) if replicas else bufs[0]
    best = 0.0
    for t in (128, 256):
        for c in (0, 2, 3, 4, 6):
            def run():
                I.update_mix_probe(g, bufs[2], bufs[3], bufs[4], bufs[5], n, t, c)
            for _ in range(3):
                run()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                run()
            e1.record()
            torch.cuda.synchronize()
            best = max(best, 30 * n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del bufs, g
    torch.cuda.empty_cache()
    return best


@pytest.mark.parametrize("name", ["llama-73m-n8", "llama-654m-n2"])
def test_update_pass_near_box_ceiling(name):
    from fsdp_sharded_mixed_amd import inputs as I, runner
    w = W.get(name)
    dev = runner.DeviceRun(w)
    dev.init_state()
    dev.fill_grads(1, w.loss_scale)
    for _ in range(3):
        dev.step()
    steps = 10
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for row in evs:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    for row in evs:
        dev.step(phase_events=[e.cuda_event for e in row])
    torch.cuda.synchronize()
    n = dev.psi_pad
    p1 = sorted(r[0].elapsed_time(r[1]) for r in evs)[steps // 2]
    p2 = sorted(r[2].elapsed_time(r[3]) for r in evs)[steps // 2]
    # pass 1 reads the N replicas, and writes the fp32 sums only when it
    # materialises them (N > 4)
    pass1_gbs = (2 * w.n_ranks + (4 if w.n_ranks > 4 else 0)) * n / (p1 * 1e-3) / 1e9
    pass2_gbs = 30 * n / (p2 * 1e-3) / 1e9
    del dev
    torch.cuda.empty_cache()
    c44, c81 = _probe(I, 4, 4), _probe(I, 8, 1)
    mix = _mix_probe(I, replicas=w.n_ranks <= 4)
    print(f"{name}: pass1 {pass1_gbs:.0f} GB/s, pass2 {pass2_gbs:.0f} GB/s, best probes 4+4 "
          f"{c44:.0f}, 8+1 {c81:.0f}, update mix {mix:.0f}", flush=True)
    assert pass2_gbs >= 0.85 * c44, (pass2_gbs, c44)
    assert pass2_gbs >= 0.90 * mix, (pass2_gbs, mix)
    assert pass2_gbs >= 0.70 * PEAK_HBM_GBS, (pass2_gbs, PEAK_HBM_GBS)
    if w.n_ranks == 8:
        assert pass1_gbs >= 0.85 * c81, (pass1_gbs, c81)
