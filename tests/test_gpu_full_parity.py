"""Element-by-element GPU parity at the workloads' full sizes, in the launch
configuration the bench times: every element compared with the CPU oracle
after every step of
  - the 73M decoder at N = 8 (ten steps; its sums split around the
    memory-side cache window),
  - the 654M decoder at N = 2 (five steps),
  - the 4.06B decoder at N = 2 (four steps, the second skipped by an
    injected +inf),
  - the 2.1B decoder under ZeRO-3 and under FSDP2 (three steps each, every
    unit gather),
  - a 120M plan of three ragged FlatParameter units at N = 5 whose
    materialised sums lie past the cache window (three steps),
  - the 654M decoder in Megatron's gradient buckets over four micro-batches,
    reduced every micro-batch or (no_sync) accumulated locally and reduced
    once (three steps each),
  - the 654M decoder under ZeRO-Offload (fp32 state and CPU-Adam on the
    host), with fp32 or 16-bit sums going down (three steps each).

The oracle side holds the full state on the host, in logical order.
FullOracle carries every element through the oracle's own functions, split
into index ranges over a thread pool (each range is independent: the
generator is keyed by logical index and the update is per element): the
master from the oracle's generator, the exact global squared norm and
overflow flag by regeneration (range partials added in order), the
fixed-order reduce-scatter sums -- accumulated over the micro-batches in the
workload's scheme -- by regeneration, the binary32 AdamW update and the
nearest-even cast.  The device arrays are in the padded flat layout: each
unit's real elements are compared with the oracle's logical range and its
padding must be bit-zero.  test_full_oracle_matches_single_threaded pins the
harness to the plain single-threaded oracle step on the CPU.

Bars: the reduce-scatter sums bit for bit; master, exp_avg, exp_avg_sq
within 4 ulp (relative 1e-6); the 16-bit parameters and every gathered unit
within 1 ulp; padding bit-zero everywhere; the step result (overflow, skip,
t, loss scale) exactly and the norm within 1e-5.  Each step reports the
share of elements that match bit for bit, and beyond those bars every
element must be bit-identical: the kernels and the oracle do the same IEEE
binary32 operations in the same order (no contraction, correctly rounded
division and square root, nearest-even casts), which is the notes'
condition for identical bits (Lecture 13, 3.4).  The one input that may
differ is the binary32 gradient scale, rounded from a norm that the device
sums in another fixed fp64 order; the two norms would have to straddle a
binary32 rounding boundary of coef/(S*N) to move it (their relative gap,
about sqrt(Psi) * 2^-53, over binary32's 2^-23 spacing: odds of order 1e-5
per clipped step at these sizes), and for these seeds they do not.  So a difference here is a
change of arithmetic order that the ulp bars alone would let through.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle as O
from fsdp_sharded_mixed_amd import workloads as W
from tests import gpu_common as G
from tests import oracle_inputs as OI

CHUNK = 1 << 21        # elements per host task
CMP_CHUNK = 1 << 25    # elements per device-to-host comparison slice


class FullOracle:
    """The full state of a workload in logical order, stepped element by
    element by the oracle over a thread pool."""

    def __init__(self, w, threads=None):
        self.w = w
        self.units, self.psi, self.psi_pad = OI.plan(w)
        assert self.psi == w.psi
        self.edges = list(range(0, w.psi, CHUNK)) + [w.psi]
        self.pool = ThreadPoolExecutor(threads or G.POOL_THREADS)
        self.p = np.empty(w.psi, np.float32)

        def init(c):
            a, b = self.edges[c], self.edges[c + 1]
            self.p[a:b] = O.gen32(b - a, w.seed, W.STREAM_MASTER, a, w.master_sigma)

        list(self.pool.map(init, range(len(self.edges) - 1)))
        if w.norm_weights_one:
            for a, b in w.norm_ranges():
                self.p[a:b] = 1.0
        self.m = np.zeros(w.psi, np.float32)
        self.v = np.zeros(w.psi, np.float32)
        self.hp = OI.hparams(w)
        self.st = OI.scale_state(w)
        self.step_no = 0

    def close(self):
        self.pool.shutdown()

    def step(self, inject_index=None, keep_sums=False):
        """One step: returns (result, sums or None).  keep_sums keeps every
        reduce-scatter sum of the step (accumulated over the micro-batches),
        in logical order, also of a skipped step."""
        w = self.w
        self.step_no += 1
        scale = self.st.loss_scale
        inj = None
        if inject_index is not None:
            inj = O.Inject(step=self.step_no, replica=w.inject_replica, index=int(inject_index),
                           bits=OI.inf_bits(w.grad_dtype))
        if w.offload_down16:
            return self._step_rounded(scale, inj, keep_sums)
        ss, bad = G.regen_sumsq_threaded(w, self.step_no, scale, self.psi, inj)
        sc, res = O.finish(ss, bad, w.n_ranks, self.hp, self.st)
        sums = np.empty(self.psi, np.float32) if keep_sums else None
        if res.skipped and not keep_sums:
            return res, None

        def part(c):
            a, b = self.edges[c], self.edges[c + 1]
            acc = O.regen_accum_acc(w.grad_dtype, w.n_ranks, w.n_micro, w.accum_mode, w.seed,
                                    self.step_no, w.sigma, scale, np.arange(a, b, dtype=np.int64),
                                    inj)
            if sums is not None:
                sums[a:b] = acc
            if not res.skipped:
                O.adamw_array(acc, sc, self.p[a:b], self.m[a:b], self.v[a:b])

        list(self.pool.map(part, range(len(self.edges) - 1)))
        return res, sums

    def _step_rounded(self, scale, inj, keep_sums):
        """The offload step with 16-bit sums down: the sums rounded to the
        gradient dtype and widened back, the squared norm and the overflow
        flag taken on those values (range partials added in order), then
        the update from them.  The returned sums are the rounded values."""
        w = self.w
        rounded = np.empty(self.psi, np.float32)

        def part(c):
            a, b = self.edges[c], self.edges[c + 1]
            acc = O.regen_accum_acc(w.grad_dtype, w.n_ranks, w.n_micro, w.accum_mode, w.seed,
                                    self.step_no, w.sigma, scale, np.arange(a, b, dtype=np.int64),
                                    inj)
            rounded[a:b] = O.widen(w.grad_dtype, O.narrow(w.grad_dtype, acc))
            return O.sumsq_array(rounded[a:b])

        ss, bad = 0.0, 0
        for s_c, b_c in self.pool.map(part, range(len(self.edges) - 1)):
            ss += s_c
            bad |= b_c
        sc, res = O.finish(ss, bad, w.n_ranks, self.hp, self.st)
        if not res.skipped:
            def upd(c):
                a, b = self.edges[c], self.edges[c + 1]
                O.adamw_array(rounded[a:b], sc, self.p[a:b], self.m[a:b], self.v[a:b])

            list(self.pool.map(upd, range(len(self.edges) - 1)))
        return res, (rounded if keep_sums else None)


def _chunks(pool, n, fn):
    """fn(a, b) over [0, n) in slices of CMP_CHUNK elements, on the pool."""
    return list(pool.map(lambda a: fn(a, min(n, a + CMP_CHUNK)), range(0, n, CMP_CHUNK)))


class Tally:
    """Bit-identical element counts per array over the units of a step."""

    def __init__(self):
        self.exact, self.total, self.worst = {}, {}, 0

    def add(self, name, exact, total, worst=0):
        self.exact[name] = self.exact.get(name, 0) + exact
        self.total[name] = self.total.get(name, 0) + total
        self.worst = max(self.worst, worst)

    def shares(self):
        out = {k: round(self.exact[k] / self.total[k], 6) for k in self.exact}
        out["worst_ulp"] = self.worst
        return out

    def assert_identical(self, what):
        """Every compared element bit-identical to the oracle."""
        off = {k: self.total[k] - self.exact[k] for k in self.exact
               if self.exact[k] != self.total[k]}
        assert not off, f"{what}: elements within the ulp bars but not bit-identical: {off}"


def compare_f32(pool, t, ref, what, max_ulp=4):
    """Every element of fp32 array t (device or host) against ref: within
    max_ulp ulp.  Returns (bit-identical count, worst ulp)."""
    def one(a, b):
        got = t[a:b].cpu().numpy()
        want = ref[a:b]
        diff = got.view(np.uint32) != want.view(np.uint32)
        nd = int(diff.sum())
        worst = 0
        if nd:
            d = G.ulp_distance(got[diff], want[diff])
            k = int(d.argmax())
            worst = int(d[k])
            assert worst <= max_ulp, \
                f"{what}: {worst} ulp at {a + int(np.flatnonzero(diff)[k])}"
        return (b - a) - nd, worst

    parts = _chunks(pool, ref.size, one)
    return sum(x[0] for x in parts), max([0] + [x[1] for x in parts])


def compare_bits32(pool, t, ref, what):
    """Every element bit for bit (NaN payloads included)."""
    def one(a, b):
        bad = np.flatnonzero(t[a:b].cpu().numpy().view(np.uint32) != ref[a:b].view(np.uint32))
        assert bad.size == 0, f"{what}: {bad.size} elements differ, first at {a + int(bad[0])}"

    _chunks(pool, ref.size, one)


def compare_16(pool, t, p_ref, dtype, what):
    """Every 16-bit element of t within 1 ulp of RNE16 of the oracle's fp32
    values p_ref; returns the bit-identical count."""
    def one(a, b):
        got = t[a:b].view(torch.int16).cpu().numpy().view(np.uint16)
        want = O.narrow(dtype, p_ref[a:b])
        diff = got != want
        nd = int(diff.sum())
        if nd:
            assert G.ulp16_distance(got[diff], want[diff]).max() <= 1, what
        return (b - a) - nd

    return sum(_chunks(pool, p_ref.size, one))


def assert_zero(t, what):
    if t.numel():
        assert int(torch.count_nonzero(G.bits_view(t))) == 0, f"{what}: padding is not zero"


def check_state(dev, orc, units, what):
    """Master, exp_avg, exp_avg_sq and the 16-bit parameters: each unit's
    real range against the oracle's logical range, its padding zero."""
    tally = Tally()
    arrays = [("master", dev.master, orc.p), ("exp_avg", dev.exp_avg, orc.m),
              ("exp_avg_sq", dev.exp_avg_sq, orc.v)]
    for u in units:
        o, L, P, lam = int(u["O"]), int(u["L"]), int(u["P"]), int(u["lam"])
        for name, t, ref in arrays:
            ex, worst = compare_f32(orc.pool, t[o:o + L], ref[lam:lam + L], f"{what} {name}")
            tally.add(name, ex, L, worst)
            assert_zero(t[o + L:o + P], f"{what} {name}")
        if dev.params is not None:
            ex = compare_16(orc.pool, dev.params[o:o + L], orc.p[lam:lam + L],
                            dev.w.param_dtype, f"{what} params")
            tally.add("params", ex, L)
            assert_zero(dev.params[o + L:o + P], f"{what} params")
    return tally


def check_sums(orc, t, units, sums, what):
    """Reduce-scatter sums (padded flat t) against the oracle's logical
    sums, bit for bit; padding zero."""
    for u in units:
        o, L, P, lam = int(u["O"]), int(u["L"]), int(u["P"]), int(u["lam"])
        compare_bits32(orc.pool, t[o:o + L], sums[lam:lam + L], what)
        assert_zero(t[o + L:o + P], what)


def check_sums16(orc, t16, units, rounded, dtype, what):
    """16-bit sums (the first Psi' 16-bit words of the device's fp32
    gradient-shard buffer) against the oracle's rounded sums, bit for bit;
    padding zero."""
    for u in units:
        o, L, P, lam = int(u["O"]), int(u["L"]), int(u["P"]), int(u["lam"])

        def one(a, b, o=o, lam=lam):
            got = t16[o + a:o + b].cpu().numpy().view(np.uint16)
            bad = np.flatnonzero(got != O.narrow(dtype, rounded[lam + a:lam + b]))
            assert bad.size == 0, f"{what}: {bad.size} differ, first at {o + a + int(bad[0])}"

        _chunks(orc.pool, L, one)
        assert_zero(t16[o + L:o + P], what)


def check_gathers(dev, orc, tally, what):
    """ZeRO-3: every unit gathered into the reused unit buffer; FSDP2: every
    FSDP unit cast-gathered into the reused group buffer.  Each against
    RNE16 of the oracle's master over the unit's logical range; a ZeRO-3
    unit's padding zero."""
    w = dev.w
    if w.fp32_params:
        for g, info in enumerate(dev.plan.groups):
            buf = dev.gather_cast(g)
            lam0 = dev.plan.units[info.first_unit].lam
            tally.add("gathers", compare_16(orc.pool, buf, orc.p[lam0:lam0 + info.numel],
                                            w.param_dtype, f"{what} group {g}"), info.numel)
    elif w.stage == 3:
        for u, info in enumerate(dev.plan.units):
            buf = dev.gather(u)
            tally.add("gathers", compare_16(orc.pool, buf[:info.L],
                                            orc.p[info.lam:info.lam + info.L], w.param_dtype,
                                            f"{what} unit {u}"), info.L)
            assert_zero(buf[info.L:info.P], f"{what} unit {u}")


def test_full_oracle_matches_single_threaded(orc):
    """CPU pin of the harness: FullOracle (range-parallel regeneration and
    update) tracks the oracle's own single-threaded step (O.zero_step, and
    O.step_reduced after the backward-side reduction, via OracleRun) for
    three steps: at N = 4 on a 5,000,004-element flat with a norm weight
    range and clipping active, at N = 3 on three ragged units (padding)
    whose gradients are reduce-scattered in buckets over three
    micro-batches, in both accumulation schemes, and at N = 2 with the sums
    rounded to bf16 on their way to an offloaded update.  The same results, the
    norm to within rounding, the sums bit for bit, the state within 4 ulp
    and almost all bit for bit."""
    segs = [W.Segment("w", 4_000_000, 0), W.Segment("n", 4, 0, W.KIND_NORM),
            W.Segment("b", 1_000_000, 0)]
    flat = W.Workload(name="flat-5m-n4", description="", segments=segs, n_ranks=4,
                      layout=W.GLOBAL_FLAT, stage=2, grad_dtype=W.BF16, param_dtype=W.BF16,
                      sigma=2e-3, loss_scale=1.0, dynamic=False, lr=1e-3, steps=3, seed=13,
                      norm_weights_one=True, max_norm=1.0)
    cases = [flat]
    for mode in (W.ACCUM_REDUCE_EACH, W.ACCUM_NO_SYNC):
        cases.append(W.Workload(
            name=f"units-acc-m{mode}", description="",
            segments=[W.Segment("a", 700_001, 0), W.Segment("b", 300_002, 1),
                      W.Segment("c", 99_998, 2)],
            n_ranks=3, layout=W.PER_UNIT, stage=2, grad_dtype=W.F16, param_dtype=W.F16,
            sigma=1e-3, loss_scale=1024.0, dynamic=True, lr=1e-3, steps=3, seed=17,
            max_norm=0.5, n_micro=3, accum_mode=mode, bucket_numel=400_000))
    cases.append(W.Workload(
        name="flat-offload16", description="", segments=[W.Segment("f", 2_000_002, 0)],
        n_ranks=2, layout=W.GLOBAL_FLAT, stage=2, grad_dtype=W.BF16, param_dtype=W.BF16,
        sigma=1e-3, loss_scale=1.0, dynamic=False, lr=1e-3, steps=3, seed=19, max_norm=0.5,
        offload=True, offload_down16=True))
    for w in cases:
        full = FullOracle(w, threads=4)
        ref = OI.OracleRun(w)
        try:
            for k in range(1, 4):
                if w.backward_rs:
                    r_ref = ref.step()
                    sums_ref = OI.rank_shards_to_logical(ref.units, ref.grad_shards)
                else:
                    grads = OI.replicas(w, ref.units, ref.psi_pad, k, ref.st.loss_scale)
                    sums_ref = OI.rank_shards_to_logical(
                        ref.units, O.reduce_scatter(w.grad_dtype, w.n_ranks, ref.units, grads))
                    if w.offload_down16:  # the sums as they go down: rounded to bf16
                        sums_ref = O.widen(w.grad_dtype, O.narrow(w.grad_dtype, sums_ref))
                    r_ref = ref.step(grads)
                r_full, sums = full.step(keep_sums=True)
                assert (r_full.skipped, r_full.t, r_full.scale_next) == \
                    (r_ref.skipped, r_ref.t, r_ref.scale_next), w.name
                assert abs(r_full.norm - r_ref.norm) <= 1e-12 * r_ref.norm and r_ref.coef < 1.0
                assert np.array_equal(sums.view(np.uint32), sums_ref.view(np.uint32)), w.name
                for mine, theirs in ((full.p, ref.master), (full.m, ref.m), (full.v, ref.v)):
                    logical = OI.rank_shards_to_logical(ref.units, theirs)
                    share = G.assert_state_close(f"full oracle {w.name}", mine, logical)
                    assert share > 0.999
        finally:
            full.close()


def host_available_bytes():
    """MemAvailable of the host, or None where /proc/meminfo is absent."""
    try:
        with open("/proc/meminfo") as f:
            for ln in f:
                if ln.startswith("MemAvailable:"):
                    return int(ln.split()[1]) * 1024
    except OSError:
        pass
    return None


@pytest.fixture(scope="module")
def R():
    from fsdp_sharded_mixed_amd import runner
    assert torch.cuda.is_available()
    return runner


def flat120m_n5():
    """Three ragged FlatParameter units at N = 5: 480 MB of materialised
    sums, past the size up to which pass 1 keeps a share of them in the
    memory-side cache, so every sum goes out non-temporal and the update
    pass walks its tiles forward."""
    return W.Workload(name="flat-120m-n5", description="three ragged units past the cache window",
                      segments=[W.Segment("a", 50_000_001, 0), W.Segment("b", 40_000_003, 1),
                                W.Segment("c", 30_000_007, 2)],
                      n_ranks=5, layout=W.PER_UNIT, stage=2, grad_dtype=W.BF16,
                      param_dtype=W.BF16, sigma=1e-3, loss_scale=1.0, dynamic=False, lr=1e-4,
                      steps=3, seed=7)


def run_full(R, w, twin_sums=False, rs_first_step=True):
    """Every step of workload w on the device against FullOracle: every
    element of the state, the 16-bit parameters (padding zero) and every
    gathered unit.

    Sums: with twin_sums a second device run steps in lockstep on the same
    replicas with fp32 gradient shards given, where the same kernels write
    the sums that the first run keeps in its workspace; its sums are
    compared every step and its state with the first run's.  Workloads
    that keep fp32 gradient shards (FSDP2, the backward-side reduction,
    ZeRO-Offload) are compared there every step.  Otherwise, with
    rs_first_step, the reduce-scatter alone (zf_reduce_scatter) at step 1."""
    from fsdp_sharded_mixed_amd import inputs as I
    from fsdp_sharded_mixed_amd import zf
    torch.cuda.empty_cache()
    w = W.get(w) if isinstance(w, str) else w
    # the host holds master, m and v (12 B per parameter) and one step's sums
    # (4 B), plus the comparison slices in flight
    need = 16 * w.psi + 2 * G.POOL_THREADS * CMP_CHUNK * 4
    avail = host_available_bytes()
    if avail is not None and avail < need:
        pytest.skip(f"{w.name} needs about {need / 2**30:.0f} GiB of host memory for the "
                    f"full oracle state; {avail / 2**30:.0f} GiB available")
    G.say(f"full parity {w.name}: Psi={w.psi:,} N={w.n_ranks} stage={w.stage} "
          f"micro={w.n_micro} offload={w.offload}, {w.steps} steps")
    dev = R.DeviceRun(w)
    twin = None
    if twin_sums:
        twin = R.DeviceRun(w, grads=False)
        twin.grads = dev.grads
        twin.grad_shards = torch.zeros(dev.psi_pad, dtype=torch.float32, device=dev.device)
        twin.init_state()
    dev.init_state()
    inj = I.inject_index(w, w.psi) if w.inject_step else None
    orc = FullOracle(w)
    units = orc.units
    assert [(u.O, u.L, u.P, u.lam) for u in dev.plan.units] == \
        [(int(u["O"]), int(u["L"]), int(u["P"]), int(u["lam"])) for u in units]
    resident_sums = dev.grad_shards is not None
    trace = []
    try:
        for u in units:  # the initial master, bit for bit
            o, L, lam = int(u["O"]), int(u["L"]), int(u["lam"])
            compare_bits32(orc.pool, dev.master[o:o + L], orc.p[lam:lam + L], "initial master")
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
            rs = None
            if rs_first_step and k == 1 and not (resident_sums or twin is not None):
                rs = torch.empty(dev.psi_pad, dtype=torch.float32, device=dev.device)
                zf.reduce_scatter(dev.plan, w.grad_dtype, dev.grads, rs)
            dev.step()
            if twin is not None:
                twin.step()
            res_d = dev.result()
            dev.loss_scale = res_d.scale_next
            keep = twin is not None or resident_sums or rs is not None
            res_o, sums = orc.step(inject_index=inj if w.inject_step == k else None,
                                   keep_sums=keep)
            G.assert_result_matches(res_d, res_o, f"{w.name} step {k}")
            if sums is not None and w.offload_down16:
                check_sums16(orc, dev.grad_shards.view(torch.int16)[:dev.psi_pad], units, sums,
                             w.grad_dtype, f"{w.name} step {k} 16-bit reduce-scatter sums")
            elif sums is not None:
                src = twin.grad_shards if twin is not None else \
                    (dev.grad_shards if resident_sums else rs)
                check_sums(orc, src, units, sums, f"{w.name} step {k} reduce-scatter sums")
            del rs, sums
            if twin is not None:
                for nm in ("master", "exp_avg", "exp_avg_sq", "params"):
                    assert torch.equal(G.bits_view(getattr(dev, nm)),
                                       G.bits_view(getattr(twin, nm))), f"step {k} {nm}"
            tally = check_state(dev, orc, units, f"{w.name} step {k}")
            check_gathers(dev, orc, tally, f"{w.name} step {k}")
            trace.append((k, res_d.skipped, res_d.t, res_d.scale_used, res_d.scale_next,
                          res_d.norm, res_d.coef))
            G.say(f"  step {k}: skipped={res_d.skipped} t={res_d.t} S={res_d.scale_used}->"
                  f"{res_d.scale_next} norm={res_d.norm:.6f} (oracle {res_o.norm:.6f}) "
                  f"coef={res_d.coef:.6f} sums {'bit-exact' if keep else '-'}; "
                  f"bit-identical shares {tally.shares()}")
            tally.assert_identical(f"{w.name} step {k}")
    finally:
        orc.close()
    return dev, trace


@pytest.mark.gpu
def test_llama73m_n8_every_element(R):
    """73M decoder, N = 8 (the sums materialised, the last 256 MiB of them
    in the memory-side cache window: pass 1's tiles split between
    non-temporal and cache-allocating stores, the update pass walking
    backward), ten steps, clipped each step; a twin run with fp32 gradient
    shards exposes the sums of every step."""
    _, trace = run_full(R, "llama-73m-n8", twin_sums=True)
    assert all(t[1] == 0 and abs(t[5] - 3.03) < 0.1 and t[6] < 1.0 for t in trace)


@pytest.mark.gpu
def test_llama654m_n2_every_element(R):
    """654M decoder, N = 2 (the update pass recomputes the sums from the
    replicas), five steps with clipping active."""
    _, trace = run_full(R, "llama-654m-n2")
    assert all(t[1] == 0 and abs(t[5] - 3.0) < 0.1 and t[6] < 1.0 for t in trace)


@pytest.mark.gpu
def test_flat120m_n5_past_cache_window_every_element(R):
    """120M parameters in three ragged units at N = 5 (padding in every
    unit), the materialised sums past the cache window; a twin run exposes
    the sums of every step."""
    from fsdp_sharded_mixed_amd import zf
    w = flat120m_n5()
    s = zf.plan_flat(w.segments, w.n_ranks, w.layout, w.stage).summary
    assert s.policy == 1 and s.cached_sums_bytes == 0 and s.psi_pad > s.psi
    _, trace = run_full(R, w, twin_sums=True)
    assert all(t[1] == 0 for t in trace)


@pytest.mark.gpu
def test_llama2b_zero3_every_element(R):
    """2.1B decoder as 34 FSDP units, N = 2, stage 3: resident 16-bit shards
    and every unit gathered into one reused buffer every step."""
    _, trace = run_full(R, "llama-2.1b-n2-zero3")
    assert all(t[1] == 0 and t[6] < 1.0 for t in trace)


@pytest.mark.gpu
def test_llama2b_fsdp2_every_element(R):
    """2.1B decoder under FSDP2: per-parameter dim-0 shards over N = 2, fp32
    parameters, the sums in resident fp32 gradient shards (every step, bit
    for bit), all 34 FSDP units cast-gathered every step."""
    dev, trace = run_full(R, "llama-2.1b-n2-fsdp2")
    assert len(dev.plan.groups) == 34 and len(dev.plan.units) == 291
    assert all(t[1] == 0 for t in trace)


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["llama-654m-n2-buckets-a4", "llama-654m-n2-nosync-a4"])
def test_llama654m_bucketed_accumulation_every_element(R, name):
    """654M decoder in Megatron's gradient buffer (12 buckets of >= 40M
    elements, last layer first, each padded to a multiple of N), N = 2,
    four micro-batches per step: every bucket reduce-scattered into the fp32
    gradient shards each micro-batch, or (no_sync) fp32 local accumulation
    and one reduction; the accumulated shards bit for bit every step; global
    norm about 3, so clipping is active."""
    dev, trace = run_full(R, name)
    assert len(dev.plan.groups) == 12
    assert all(t[1] == 0 and abs(t[5] - 3.0) < 0.1 and t[6] < 1.0 for t in trace)


@pytest.mark.gpu
def test_llama654m_offload_every_element(R):
    """654M decoder under ZeRO-Offload: the GPU reduces into fp32 gradient
    shards (bit for bit every step), the fp32 state and CPU-Adam live on
    the host (every element), bf16 parameters come back in chunks."""
    dev, trace = run_full(R, "llama-654m-n2-offload")
    assert dev.master.device.type == "cpu"
    assert all(t[1] == 0 and abs(t[5] - 3.0) < 0.1 and t[6] < 1.0 for t in trace)


@pytest.mark.gpu
def test_llama654m_offload16_every_element(R):
    """The same with 16-bit sums down: the GPU rounds the sums to bf16
    (bit for bit every step), the norm and overflow are taken on the rounded
    values and CPU-Adam updates from them (every element of the host
    state)."""
    dev, trace = run_full(R, "llama-654m-n2-offload16")
    assert dev.w.offload_down16 and dev.master.device.type == "cpu"
    assert all(t[1] == 0 and abs(t[5] - 3.0) < 0.1 and t[6] < 1.0 for t in trace)


@pytest.mark.gpu
def test_llama4b_n2_every_element(R):
    """4.06B decoder, N = 2, fp16 under dynamic loss scaling with +inf in
    replica 1 at step 2: step 2 is skipped (state untouched, every element)
    and S halves 32768 -> 16384; steps 1, 3, 4 applied."""
    _, trace = run_full(R, "llama-4.06b-n2")
    assert [(t[1], t[2]) for t in trace] == [(0, 1), (1, 1), (0, 2), (0, 3)]
    assert trace[1][3] == 32768.0 and trace[1][4] == 16384.0 and trace[2][3] == 16384.0
