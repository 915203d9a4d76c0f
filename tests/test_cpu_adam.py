"""CPU-Adam (zf_cpu_adam, the host side of ZeRO-Offload) against the oracle.

Runs on the CPU: the call touches no GPU.  Given the same step scalars (gs
and the bias corrections, here from the oracle's own finish), the host
update must reproduce the oracle's element update bit for bit -- fp32
master, exp_avg, exp_avg_sq and the 16-bit parameters -- for every length
(ragged vector tails), thread count and element offset.
"""
import numpy as np
import pytest

import oracle as O
from fsdp_sharded_mixed_amd import workloads as W


@pytest.fixture(scope="module")
def zf():
    from fsdp_sharded_mixed_amd import zf as Z
    return Z


def _hp(lr=1e-3, wd=0.01):
    return O.Hparams(lr=lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=wd, max_norm=1.0)


def _zhp(zf, h):
    return zf.hparams(h.lr, h.beta1, h.beta2, h.eps, h.weight_decay, h.max_norm)


def _scalars(acc, t, hp, n_ranks=4, scale=1024.0):
    st = O.ScaleState(loss_scale=scale, t=t, growth_ctr=0, growth_interval=2000, dynamic=1)
    sc, res = O.finish(float(np.sum(acc.astype(np.float64) ** 2)), 0, n_ranks, hp, st)
    assert res.skipped == 0
    return sc


def _state(rng, n):
    """Values over many binades, zeros and subnormal moments included."""
    acc = (rng.standard_normal(n) * 10.0 ** rng.integers(-3, 4, n)).astype(np.float32)
    acc[::97] = 0.0
    p = (rng.standard_normal(n) * 10.0 ** rng.integers(-6, 1, n)).astype(np.float32)
    m = (rng.standard_normal(n) * 10.0 ** rng.integers(-8, -1, n)).astype(np.float32)
    v = np.abs(rng.standard_normal(n) * 10.0 ** rng.integers(-12, -3, n)).astype(np.float32)
    v[::53] = np.float32(1e-44)  # subnormal
    return acc, p, m, v


def _bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


@pytest.mark.parametrize("dtype", [W.BF16, W.F16])
@pytest.mark.parametrize("n,threads", [(0, 1), (1, 1), (15, 2), (16, 1), (17, 3), (1000, 4),
                                       (100003, 0), (300017, 7)])
def test_matches_oracle_update(zf, dtype, n, threads):
    rng = np.random.default_rng(n + threads)
    acc, p, m, v = _state(rng, max(n, 1))
    acc, p, m, v = acc[:n], p[:n], m[:n], v[:n]
    hp = _hp()
    sc = _scalars(acc, 5, hp) if n else _scalars(np.ones(1, np.float32), 5, hp)
    ref = [p.copy(), m.copy(), v.copy()]
    O.adamw_array(acc, sc, *ref)
    got = [p.copy(), m.copy(), v.copy()]
    out = np.full(n, 0xDEAD, np.uint16)
    zf.cpu_adam(_zhp(zf, hp), acc, *got, sc.gs, sc.bc1, sc.bc2, params=out, param_dtype=dtype,
                n_threads=threads)
    for g, r in zip(got, ref):
        assert np.array_equal(_bits(g), _bits(r))
    assert np.array_equal(out, O.narrow(dtype, ref[0]))


def test_offsets_and_no_param_output(zf):
    """Arrays starting at any 4-byte offset (not vector aligned), and no
    16-bit output."""
    rng = np.random.default_rng(5)
    n = 4099
    hp = _hp()
    for off in (1, 2, 3):
        acc, p, m, v = _state(rng, n + off)
        sc = _scalars(acc, 2, hp)
        ref = [x[off:].copy() for x in (p, m, v)]
        O.adamw_array(acc[off:].copy(), sc, *ref)
        zf.cpu_adam(_zhp(zf, hp), acc[off:], p[off:], m[off:], v[off:], sc.gs, sc.bc1, sc.bc2,
                    n_threads=3)
        for g, r in zip((p[off:], m[off:], v[off:]), ref):
            assert np.array_equal(_bits(np.ascontiguousarray(g)), _bits(r))


def _patterns():
    """binary32 bit patterns: every sign/exponent with structured mantissas
    (rounding ties and their neighbours for both 16-bit formats), plus
    infinities and NaNs."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x0FFF, 0x1000, 0x1001, 0x1FFF, 0x2000, 0x2001, 0x3000, 0x7FFF,
                     0x8000, 0x8001, 0xBFFF, 0xC000, 0xFFFF], np.uint32)
    return (hi[:, None] | lows[None, :]).ravel()


@pytest.mark.parametrize("dtype", [W.BF16, W.F16])
def test_cast_every_exponent(zf, dtype):
    """With lr = 0 the master is unchanged (p*1 - 0), so the 16-bit output
    is the rounding of arbitrary binary32 patterns: equal to the oracle's
    round-to-nearest-even everywhere; NaNs stay NaN."""
    bits = _patterns()
    p = bits.view(np.float32).copy()
    n = p.size
    z = np.zeros(n, np.float32)
    hp = _hp(lr=0.0, wd=0.0)
    out = np.empty(n, np.uint16)
    zf.cpu_adam(_zhp(zf, hp), z, p, z.copy(), z.copy(), 1.0, 0.1, 0.001, params=out,
                param_dtype=dtype, n_threads=4)
    nan = np.isnan(bits.view(np.float32))
    # every non-NaN value is unchanged (signalling NaNs come back quieted)
    assert np.array_equal(p.view(np.uint32)[~nan], bits[~nan]) and np.isnan(p[nan]).all()
    ref = O.narrow(dtype, bits.view(np.float32))
    exp_mask, man_mask = (0x7C00, 0x03FF) if dtype == W.F16 else (0x7F80, 0x007F)
    assert np.array_equal(out[~nan], ref[~nan])
    assert np.all((out[nan] & exp_mask) == exp_mask) and np.all((out[nan] & man_mask) != 0)


def test_argument_errors(zf):
    import ctypes as C
    hp = zf.hparams(1e-3)
    ok = np.zeros(64, np.float32)
    a = ok.ctypes.data

    def call(**kw):
        d = dict(n=16, grad=a, master=a, exp_avg=a, exp_avg_sq=a, params=None, param_dtype=2,
                 n_threads=1, gs=1.0, bc1=0.1, bc2=0.001, grad_dtype=0)
        d.update(kw)
        args = zf.CpuAdamArgs(*[d[f] for f, _ in zf.CpuAdamArgs._fields_])
        return zf.lib.zf_cpu_adam(C.byref(hp), C.byref(args))

    assert call() == 0
    assert call(n=-1) == -1
    assert call(grad=None) == -1
    assert call(grad_dtype=5) == -3
    assert call(grad_dtype=1, grad=a + 2) == 0     # 16-bit sums: 2-byte alignment
    assert call(grad_dtype=3, grad=a + 2) == -2
    assert call(params=a, param_dtype=3) == -3
    assert call(master=a + 2) == -2
    assert call(params=a + 1, param_dtype=1) == -2
    assert call(n=0, grad=None) == 0
    assert zf.lib.zf_cpu_adam(None, None) == -1


@pytest.mark.parametrize("gdt", [W.F16, W.BF16])
def test_16bit_gradients(zf, gdt):
    """16-bit gradient sums (the offload step's 16-bit download): the host
    update equals the oracle's on the exactly widened values."""
    rng = np.random.default_rng(11)
    n = 40003
    acc32, p, m, v = _state(rng, n)
    g16 = O.narrow(gdt, acc32)
    acc = O.widen(gdt, g16)
    acc[~np.isfinite(acc)] = 0.0
    g16 = O.narrow(gdt, acc)
    hp = _hp()
    sc = _scalars(acc, 3, hp)
    ref = [p.copy(), m.copy(), v.copy()]
    O.adamw_array(acc, sc, *ref)
    got = [p.copy(), m.copy(), v.copy()]
    out = np.empty(n, np.uint16)
    zf.cpu_adam(_zhp(zf, hp), g16, *got, sc.gs, sc.bc1, sc.bc2, params=out, param_dtype=W.BF16,
                n_threads=5, grad_dtype=gdt)
    for g, r in zip(got, ref):
        assert np.array_equal(_bits(g), _bits(r))
    assert np.array_equal(out, O.narrow(W.BF16, ref[0]))
