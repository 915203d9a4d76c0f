"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small seeded cases are compared element by element; they span several
pass-1 grid sweeps and ragged tails.  Bars:
  * reduce-scatter sums, overflow flag, skip decision, gathered layout and
    padding: bit-exact;
  * fp32 master, exp_avg, exp_avg_sq: within 4 ulp (relative ~1e-6);
  * 16-bit params: within 1 ulp;
  * global norm: relative 1e-5.
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


def small(n, layout, lens, gdt=W.BF16, pdt=None, stage=2, dynamic=None, scale=None,
          sigma=1e-3, max_norm=1.0, lr=1e-3, seed=21, steps=5):
    dynamic = (gdt == W.F16) if dynamic is None else dynamic
    scale = (1024.0 if gdt == W.F16 else 1.0) if scale is None else scale
    segs = [W.Segment(f"s{i}", int(l), i if layout == W.PER_UNIT else 0)
            for i, l in enumerate(lens)]
    return W.Workload(name=f"n{n}-l{layout}-g{gdt}-s{stage}", description="", segments=segs,
                      n_ranks=n, layout=layout, stage=stage, grad_dtype=gdt,
                      param_dtype=pdt or gdt, sigma=sigma, loss_scale=scale, dynamic=dynamic,
                      lr=lr, steps=steps, seed=seed, max_norm=max_norm)


def set_bits(t, p, bits):
    t.view(torch.int16)[p] = int(np.array(bits, np.uint16).view(np.int16))


def run_pair(R, w, steps, injections=None, check_rs=True):
    """Step device and oracle side by side; compare everything every step.
    injections: {step: [(replica, padded_index, bits16), ...]}"""
    injections = injections or {}
    G.say(f"case {w.name} psi={w.psi} N={w.n_ranks} steps={steps}")
    dev = R.DeviceRun(w)
    dev.init_state()
    orc = OI.OracleRun(w)
    m0, _, _ = G.oracle_padded_state(orc)
    assert np.array_equal(G.bits32(dev.master), m0.view(np.uint32)), "master init"
    assert np.array_equal(G.bits16(dev.params), G.oracle_padded_params(orc)), "param init"
    exact = []
    for k in range(1, steps + 1):
        scale = orc.st.loss_scale
        assert dev.loss_scale == scale
        grads = OI.replicas(w, orc.units, orc.psi_pad, k, scale)
        dev.fill_grads(k, scale)
        for q, p, bits in injections.get(k, []):
            grads[q][p] = bits
            set_bits(dev.grads[q], p, bits)
        for q in range(w.n_ranks):
            assert np.array_equal(G.bits16(dev.grads[q]), grads[q]), f"grad input {q}"
        if check_rs:
            rs = torch.empty(orc.psi_pad, dtype=torch.float32, device=dev.device)
            from fsdp_sharded_mixed_amd import zf
            zf.reduce_scatter(dev.plan, w.grad_dtype, dev.grads, rs)
            ref = OI.rank_shards_to_padded(orc.units,
                                           O.reduce_scatter(w.grad_dtype, w.n_ranks, orc.units,
                                                            grads))
            got = G.f32(rs)
            nan = np.isnan(ref)
            assert np.array_equal(np.isnan(got), nan)
            assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32)), "RS"
        res_o = orc.step(grads)
        dev.step()
        res_d = dev.result()
        dev.loss_scale = res_d.scale_next
        G.assert_result_matches(res_d, res_o, f"{w.name} step {k}")
        mo, mmo, vo = G.oracle_padded_state(orc)
        fr = [G.assert_state_close("master", G.f32(dev.master), mo),
              G.assert_state_close("exp_avg", G.f32(dev.exp_avg), mmo),
              G.assert_state_close("exp_avg_sq", G.f32(dev.exp_avg_sq), vo)]
        po = G.oracle_padded_params(orc)
        assert G.ulp16_distance(G.bits16(dev.params), po).max() <= 1, "params"
        exact.append(min(fr))
        # padding is zero everywhere, bit for bit
        pad = np.ones(orc.psi_pad, bool)
        for u in orc.units:
            pad[u["O"]:u["O"] + u["L"]] = False
        if pad.any():
            for t in (dev.master, dev.exp_avg, dev.exp_avg_sq):
                assert np.all(G.bits32(t)[pad] == 0)
            assert np.all(G.bits16(dev.params)[pad] == 0)
        if w.stage == 3:
            for u in range(len(orc.units)):
                got = G.bits16(dev.gather(u))
                ref = O.gather_unit(orc.units, w.n_ranks, u, orc.shards)
                assert np.array_equal(got, ref), f"gather unit {u}"
    G.say(f"  exact-bit share of fp32 state per step: {exact}")
    return dev, orc


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6, 7, 8, 12])
def test_global_flat_all_rank_counts(R, n):
    """One global flat (ZeRO-1/2), ragged length, every compiled rank count
    and the run-time-N path (12)."""
    w = small(n, W.GLOBAL_FLAT, [40001, 17, 9000], gdt=W.BF16)
    run_pair(R, w, 5, injections={3: [(n - 1, 123, 0x7F80)]})


@pytest.mark.parametrize("n", [2, 3, 8])
@pytest.mark.parametrize("stage", [2, 3])
def test_per_unit_fp16_dynamic(R, n, stage):
    """Per-unit FlatParameters with padding, fp16 under dynamic loss scaling,
    an overflow at step 2 (scale halves, step skipped), stages 2 and 3."""
    w = small(n, W.PER_UNIT, [5003, 77, 20000, 1, 3333], gdt=W.F16, stage=stage)
    run_pair(R, w, 5, injections={2: [(0, 7, 0x7C00)]})


def test_tiny_workload_all_stages(R):
    """The 5-layer MLP workload (Psi = 32,656, N = 4), ten steps, stages 1-3."""
    for stage in (1, 2, 3):
        w = W.tiny(stage)
        run_pair(R, w, w.steps)


def test_multi_sweep_sizes(R):
    """Psi' above one pass-1 grid sweep (2048 blocks x 256 x 8), both
    policies (N = 2 recomputes the sums, N = 8 materialises them)."""
    for n in (2, 8):
        w = small(n, W.GLOBAL_FLAT, [4_500_003, 5], gdt=W.BF16, max_norm=0.5)
        run_pair(R, w, 3, check_rs=(n == 8))


def test_mixed_dtypes(R):
    """bf16 gradients with fp16 parameters and the reverse."""
    run_pair(R, small(3, W.PER_UNIT, [1000, 2001], gdt=W.BF16, pdt=W.F16), 3)
    run_pair(R, small(3, W.PER_UNIT, [1000, 2001], gdt=W.F16, pdt=W.BF16), 3)


def test_overflow_cases(R):
    """inf / NaN in any replica, at shard edges and in the padding; finite
    bf16 values whose fp32 sum overflows; consecutive overflows keep
    halving the scale; a static scale stays put but still skips."""
    w = small(3, W.PER_UNIT, [100, 31], gdt=W.F16, stage=2)
    # unit 0: L=100, P=102, S=34 (pads at 100, 101); unit 1 at O=102: L=31,
    # P=33, S=11 (rank shards start at 102, 113, 124; pads at 133, 134)
    inj = {1: [(2, 0, 0x7C00)], 2: [(1, 101, 0x7E00)], 3: [(0, 33, 0xFC00), (2, 113, 0x7C00)],
           5: [(1, 134, 0x7C00)]}
    run_pair(R, w, 6, injections=inj)
    wb = small(2, W.GLOBAL_FLAT, [64], gdt=W.BF16, dynamic=False, scale=1.0)
    big = 0x7F7F  # ~3.39e38: two of them overflow binary32
    run_pair(R, wb, 3, injections={2: [(0, 5, big), (1, 5, big)]})


def test_degenerate_cases(R):
    """N = 1 (the sum is the replica), a single-element model over 8 ranks
    (7 pads), clipping disabled, lr = 0, and N = 64."""
    run_pair(R, small(1, W.GLOBAL_FLAT, [1001]), 3)
    run_pair(R, small(8, W.PER_UNIT, [1]), 3)
    run_pair(R, small(4, W.GLOBAL_FLAT, [999], max_norm=0.0), 3)
    run_pair(R, small(4, W.GLOBAL_FLAT, [999], lr=0.0), 3)
    run_pair(R, small(64, W.PER_UNIT, [640, 65, 1]), 2, check_rs=True)


def test_many_units(R):
    """ZeRO-3 with 300 small units of assorted lengths, per-unit gathers."""
    rng = np.random.default_rng(4)
    lens = [int(x) for x in rng.integers(1, 300, 300)]
    run_pair(R, small(3, W.PER_UNIT, lens, stage=3), 2)


def test_wide_range_arithmetic(R):
    """Master over the whole binary32 range and m, v over 2^-149 .. 2^60
    (subnormals included), with fp16 gradients of every finite magnitude:
    the divisions, square root and casts agree with the oracle bit for bit.
    (m and v are bounded so that the update itself cannot overflow into a
    NaN, whose 16-bit encoding the method never produces.)"""
    from fsdp_sharded_mixed_amd import zf
    n = 3
    w = small(n, W.GLOBAL_FLAT, [65536 + 5], gdt=W.F16, dynamic=False, scale=1.0,
              max_norm=0.0)
    dev = R.DeviceRun(w)
    orc = OI.OracleRun(w)
    rng = np.random.default_rng(9)
    psi = orc.psi_pad

    def wide(lo, hi, sign=True):
        e = rng.uniform(lo, hi, psi)
        x = (rng.uniform(1, 2, psi) * np.exp2(e)).astype(np.float32)
        if sign:
            x *= np.where(rng.integers(0, 2, psi) == 1, -1, 1).astype(np.float32)
        return x

    p, m, v = wide(-149, 127), wide(-149, 60), wide(-149, 60, sign=False)
    for a in (p, m, v):
        a[orc.psi:] = 0
    grads = [rng.integers(0, 65536, psi).astype(np.uint16) for _ in range(n)]
    for g in grads:
        g[(g & 0x7C00) == 0x7C00] &= 0xBFFF  # no inf/NaN
        g[orc.psi:] = 0
    orc.master = OI.to_rank_shards(orc.units, n, p[:orc.psi])
    orc.m = OI.to_rank_shards(orc.units, n, m[:orc.psi])
    orc.v = OI.to_rank_shards(orc.units, n, v[:orc.psi])
    dev.master.copy_(torch.from_numpy(p))
    dev.exp_avg.copy_(torch.from_numpy(m))
    dev.exp_avg_sq.copy_(torch.from_numpy(v))
    zf.state_init(dev.state, 1.0, False)
    for q in range(n):
        dev.grads[q].copy_(torch.from_numpy(grads[q].view(np.int16)).view(torch.float16))
    for _ in range(2):
        res_o = orc.step(grads)
        dev.step()
        G.assert_result_matches(dev.result(), res_o, "wide")
        mo, mmo, vo = G.oracle_padded_state(orc)
        for name, t, ref in (("p", dev.master, mo), ("m", dev.exp_avg, mmo),
                             ("v", dev.exp_avg_sq, vo)):
            got = G.bits32(t)
            refb = ref.view(np.uint32)
            nan = np.isnan(ref)
            assert np.array_equal(np.isnan(G.f32(t)), nan)
            same = got[~nan] == refb[~nan]
            assert same.all(), f"{name}: {(~same).sum()} mismatches"
        got16 = G.bits16(dev.params)
        ref16 = G.oracle_padded_params(orc)
        nan16 = np.isnan(mo)
        assert np.array_equal(got16[~nan16], ref16[~nan16])


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
def test_cast_patterns(R, dtype):
    """With lr = 0, no decay and zero gradients the update is the identity,
    so the written params are RNE16(master) for any finite master: every
    2^16 upper half with 64 lower halves, plus dense windows at fp16's
    subnormal boundary and overflow threshold, against the oracle's cast."""
    rng = np.random.default_rng(5)
    low = np.array([0x0000, 0x0001, 0x0FFF, 0x1000, 0x1001, 0x1FFF, 0x2000, 0x7FFF, 0x8000,
                    0x8001, 0xEFFF, 0xF000, 0xF001, 0xFFFE, 0xFFFF]
                   + list(rng.integers(0, 65536, 49)), np.uint32)
    high = np.arange(65536, dtype=np.uint32) << 16
    pats = np.concatenate([(high[:, None] | low[None, :]).ravel(),
                           np.arange(0x37FF0000, 0x38810000, dtype=np.uint32),
                           np.arange(0x477F0000, 0x47810000, dtype=np.uint32)])
    x = pats.view(np.float32)
    x = x[~np.isnan(x)]
    w = small(1, W.GLOBAL_FLAT, [x.size], gdt=dtype, dynamic=False, scale=1.0, lr=0.0,
              max_norm=0.0)
    w.weight_decay = 0.0
    dev = R.DeviceRun(w)
    from fsdp_sharded_mixed_amd import zf
    zf.state_init(dev.state, 1.0, False)
    n = dev.psi_pad
    host = np.zeros(n, np.float32)
    host[:x.size] = x
    dev.master.copy_(torch.from_numpy(host))
    dev.step()
    assert dev.result().skipped == 0
    assert np.array_equal(G.bits32(dev.master), host.view(np.uint32)), "identity update"
    assert np.array_equal(G.bits16(dev.params), O.narrow(dtype, host))


def test_generator_matches_oracle(R):
    """The GPU input library reproduces the oracle's generator bit for bit
    (fp16, bf16, fp32; arbitrary logical offsets and streams)."""
    from fsdp_sharded_mixed_amd import inputs as I
    n = 300_001
    for dt, tdt in ((W.F16, torch.float16), (W.BF16, torch.bfloat16)):
        t = torch.zeros(n + 3, dtype=tdt, device="cuda")
        I.fill_normal16(t, n, dt, 77, W.grad_stream(5, 3), 123456789, 1e-3, 32768.0, offset=3)
        ref = O.gen16(n, dt, 77, W.grad_stream(5, 3), 123456789, 1e-3, 32768.0)
        assert np.array_equal(G.bits16(t)[3:], ref)
        assert np.all(G.bits16(t)[:3] == 0)
    t = torch.zeros(n, dtype=torch.float32, device="cuda")
    I.fill_normal32(t, n, 9, W.STREAM_MASTER, 4_000_000_000, 0.02)
    assert np.array_equal(G.bits32(t), O.gen32(n, 9, W.STREAM_MASTER, 4_000_000_000,
                                                0.02).view(np.uint32))


def test_determinism(R):
    """Two runs of the same steps give identical bits, norm included."""
    w = small(8, W.GLOBAL_FLAT, [300_007], gdt=W.BF16)
    outs = []
    for _ in range(2):
        dev = R.DeviceRun(w)
        dev.init_state()
        norms = [dev.run_workload_step().sumsq for _ in range(3)]
        outs.append((norms, G.bits32(dev.master), G.bits16(dev.params)))
    assert outs[0][0] == outs[1][0]
    assert np.array_equal(outs[0][1], outs[1][1]) and np.array_equal(outs[0][2], outs[1][2])


def test_gather_misaligned_shards(R):
    """zf_gather with shard pointers at every 2-byte misalignment, including
    source and destination misaligned differently."""
    from fsdp_sharded_mixed_amd import zf
    n = 3
    plan = zf.plan_flat([(1000, 0), (5003, 1)], n, W.PER_UNIT, 3)
    info = plan.units[1]
    S = info.S
    src = torch.arange(n * S + 64, dtype=torch.int32, device="cuda").to(torch.int16)
    host = src.cpu().numpy().view(np.uint16)
    for offs in ([0, 1, 2], [3, 7, 5], [8, 9, 15]):
        buf = torch.zeros(info.P + 16, dtype=torch.int16, device="cuda")
        base = src.data_ptr()
        ptrs = [base + 2 * (offs[r] + r * S) for r in range(n)]
        for dst_off in (0, 1):
            zf.gather(plan, 1, W.BF16, ptrs, buf.data_ptr() + 2 * dst_off,
                      unit_buf_numel=buf.numel() - dst_off)
            got = buf.cpu().numpy().view(np.uint16)[dst_off:dst_off + info.P]
            want = np.concatenate([host[offs[r] + r * S:offs[r] + (r + 1) * S]
                                   for r in range(n)])
            assert np.array_equal(got, want)


def test_phase_events_and_no_sync(R):
    """Phase events are recorded in order on the stream and the step does
    not synchronise the host (the next call queues behind it)."""
    w = small(2, W.GLOBAL_FLAT, [1 << 20], gdt=W.BF16)
    dev = R.DeviceRun(w)
    dev.init_state()
    dev.fill_grads(1, 1.0)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    dev.step(phase_events=[e.cuda_event for e in evs])
    torch.cuda.synchronize()
    t = [evs[0].elapsed_time(evs[i]) for i in (1, 2, 3)]
    assert 0 <= t[0] <= t[1] <= t[2]
    assert dev.result().t == 1


@pytest.mark.parametrize("dtype", [W.F16, W.BF16])
def test_rs_pair_sweep(R, dtype):
    """The N = 2 reduce-scatter over every 16-bit value of replica 0 against
    512 values of replica 1 that cover every exponent with edge mantissas
    (33.5M pairs: rounding ties, cancellation, overflow to inf, NaN
    propagation), and N = 1 over all 65,536 values: bit-exact against the
    oracle (NaN positions equal)."""
    from fsdp_sharded_mixed_amd import zf
    allv = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    man_bits = 10 if dtype == W.F16 else 7
    exps = np.arange(1 << (15 - man_bits), dtype=np.uint32) << man_bits
    top = (1 << man_bits) - 1
    half = 1 << (man_bits - 1)
    mans = np.array([0, 1, 2, top, top - 1, half, half - 1, half + 1], np.uint32)
    other = (exps[:, None] | mans[None, :]).ravel()
    other = np.concatenate([other, other | 0x8000]).astype(np.uint16)
    assert other.size >= 512
    other = other[np.linspace(0, other.size - 1, 512).astype(np.int64)]
    r0 = np.repeat(allv, other.size)
    r1 = np.tile(other, allv.size)
    n = r0.size
    for reps in ([r0, r1], [allv]):
        nr = len(reps)
        w = small(nr, W.GLOBAL_FLAT, [reps[0].size], gdt=dtype)
        plan = R.plan_workload(w)
        tdt = torch.float16 if dtype == W.F16 else torch.bfloat16
        dev_g = [torch.from_numpy(x.view(np.int16)).cuda().view(tdt) for x in reps]
        out = torch.empty(plan.psi_pad, dtype=torch.float32, device="cuda")
        zf.reduce_scatter(plan, dtype, dev_g, out)
        units, _, _ = OI.plan(w)
        ref = OI.rank_shards_to_padded(units, O.reduce_scatter(dtype, nr, units, reps))
        got = G.f32(out)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert n == (1 << 16) * 512


@pytest.mark.parametrize("dtype", [W.BF16, W.F16])
def test_rank_order_on_device(R, dtype):
    """Floating-point addition is not associative ([L13] 3.4, condition 2):
    three replicas holding a large value, a small one and the large value's
    negation, in every order, at every element position of several tiles.
    The device sums in rank order exactly as the oracle does, so the small
    value survives only when the large ones cancel first."""
    from fsdp_sharded_mixed_amd import zf
    if dtype == W.BF16:
        big, small_v, nbig, small_f = 0x4B80, 0x3F80, 0xCB80, 1.0        # 2^24, 1, -2^24
    else:
        big, small_v, nbig, small_f = 0x7BFF, 0x0001, 0xFBFF, 2.0 ** -24  # 65504, 2^-24
    import itertools
    orders = list(itertools.permutations([big, small_v, nbig]))
    n = 6 * 5003  # every order at every residue mod 4 and across tiles, ragged end
    reps = [np.empty(n, np.uint16) for _ in range(3)]
    for i in range(n):
        o = orders[i % 6]
        for q in range(3):
            reps[q][i] = o[q]
    w = small(3, W.GLOBAL_FLAT, [n], gdt=dtype)
    plan = R.plan_workload(w)
    tdt = torch.float16 if dtype == W.F16 else torch.bfloat16
    dev_g = [torch.from_numpy(np.concatenate([x, np.zeros(plan.summary.psi_pad - n, np.uint16)])
                              .view(np.int16)).cuda().view(tdt) for x in reps]
    out = torch.empty(plan.summary.psi_pad, dtype=torch.float32, device="cuda")
    zf.reduce_scatter(plan, dtype, dev_g, out)
    got = G.f32(out)[:n]
    # each order's sum by its definition: binary32 additions left to right
    widen = (lambda h: np.float32(np.array([h], np.uint16).view(np.float16)[0])) \
        if dtype == W.F16 else (lambda h: np.array([h << 16], np.uint32).view(np.float32)[0])
    want = np.array([(widen(o[0]) + widen(o[1])) + widen(o[2]) for o in orders], np.float32)
    assert set(want.tolist()) == {0.0, small_f}  # the order decides
    assert np.array_equal(got, np.tile(want, n // 6))
    units, _, psi_pad = OI.plan(w)
    ref = OI.rank_shards_to_padded(units, O.reduce_scatter(
        dtype, 3, units, [G.bits16(g) for g in dev_g]))
    assert np.array_equal(G.f32(out).view(np.uint32), ref.view(np.uint32))
