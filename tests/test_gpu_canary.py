"""Canary regions around every buffer the device calls write.

Each buffer sits between two 4 KiB guard bands of a fixed byte pattern and
is passed at its exact size, with no slack:
- Psi' elements for the per-element arrays;
- zf_workspace_bytes for the workspace, zf_state_bytes for the state block;
- P_u or the group's element count for the gather buffers.
After the calls, and a synchronisation, both bands must still hold the
pattern byte for byte.

The plans have ragged ends: Psi' not a multiple of 4, units shorter than a
quad, odd unit offsets. The cases cover every launch path:
- the step with recomputed sums (N <= 4), materialised sums (N > 4) and the
  run-time rank count (N = 12);
- stage-3 unit gathers, and FSDP2 with its cast-gathers;
- bucketed reduce-scatter with accumulation, and no_sync accumulation at odd
  offsets;
- the reduce-scatter alone, and resharding of fp32 and 16-bit arrays.
"""
import pytest
import torch

from fsdp_sharded_mixed_amd import workloads as W
from tests import gpu_common as G

pytestmark = pytest.mark.gpu

GUARD = 4096
PATTERN = 0xA5


@pytest.fixture(scope="module")
def zf():
    from fsdp_sharded_mixed_amd import zf as Z
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return Z


class Guarded:
    """A device buffer of `numel` elements between two guard bands."""
    all = []

    def __init__(self, numel, dtype, what, byte_offset=0):
        es = torch.tensor([], dtype=dtype).element_size()
        assert GUARD % es == 0 and byte_offset % es == 0
        self.g = (GUARD + byte_offset) // es
        self.numel, self.what = numel, what
        self.full = torch.empty(numel + self.g + GUARD // es, dtype=dtype, device="cuda")
        self.full.view(torch.uint8).fill_(PATTERN)
        self.t = self.full[self.g:self.g + numel]
        Guarded.all.append(self)

    def check(self):
        b = self.full.view(torch.uint8)
        es = self.full.element_size()
        head, tail = b[:self.g * es], b[(self.g + self.numel) * es:]
        assert bool((head == PATTERN).all()), f"{self.what}: guard before the buffer written"
        assert bool((tail == PATTERN).all()), f"{self.what}: guard after the buffer written"


@pytest.fixture(autouse=True)
def _checked():
    Guarded.all = []
    yield
    torch.cuda.synchronize()
    for b in Guarded.all:
        b.check()
    Guarded.all = []


def _zero_padding(t, plan, n):
    """Rank r's chunk of unit u holds clamp(L_u - r*S_u, 0, S_u) real
    elements, then padding (every layout)."""
    for u in plan.units:
        for r in range(n):
            real = min(max(u.L - r * u.S, 0), u.S)
            t[u.O + r * u.S + real:u.O + (r + 1) * u.S].zero_()


def _grads(plan, n, dtype, seed):
    """N replicas with seeded values in the real elements, zeros in the padding."""
    gen = torch.Generator(device="cuda").manual_seed(seed)
    td = {W.BF16: torch.bfloat16, W.F16: torch.float16}[dtype]
    psi_pad = plan.summary.psi_pad
    out = []
    for q in range(n):
        b = Guarded(psi_pad, td, f"grad replica {q}")
        b.t.copy_((torch.randn(psi_pad, generator=gen, device="cuda") * 1e-2).to(td))
        _zero_padding(b.t, plan, n)
        out.append(b.t)
    return out


def _state_arrays(plan, seed, params_dtype=torch.bfloat16, fp32_params=False):
    gen = torch.Generator(device="cuda").manual_seed(seed)
    psi_pad = plan.summary.psi_pad
    master = Guarded(psi_pad, torch.float32, "master")
    master.t.copy_(torch.randn(psi_pad, generator=gen, device="cuda") * 0.02)
    _zero_padding(master.t, plan, plan.summary.n_ranks)
    m = Guarded(psi_pad, torch.float32, "exp_avg")
    v = Guarded(psi_pad, torch.float32, "exp_avg_sq")
    m.t.zero_()
    v.t.zero_()
    params = None
    if not fp32_params:
        params = Guarded(psi_pad, params_dtype, "params").t
        params.copy_(master.t.to(params_dtype))
    return master.t, m.t, v.t, params


def _step(zf, plan, n, dtype, grads, arrays, grad_shards=None, grads_reduced=False):
    master, m, v, params = arrays
    ws = Guarded(max(1, plan.summary.workspace_bytes), torch.uint8, "workspace")
    st = Guarded(zf.state_bytes(), torch.uint8, "state block")
    zf.state_init(st.t, 1.0, 0)
    hp = zf.hparams(1e-3)
    for _ in range(2):
        zf.shard_step(plan, hp, dtype, dtype, grads, master, m, v, params, ws.t, st.t,
                      grad_shards=grad_shards, grads_reduced=grads_reduced)
    res = zf.read_result(st.t)
    assert res.t == 2 and res.skipped == 0


RAGGED = [40001, 17, 3, 9000, 1, 2051]  # Psi = 51073


@pytest.mark.parametrize("n", [3, 8, 12])
def test_step_global_flat(zf, n):
    """Stage 2 on one global flat: recomputed (N = 3), materialised (8) and
    run-time N (12) sums; the workspace is exactly zf_workspace_bytes."""
    G.say(f"canary step N={n}")
    plan = zf.plan_flat([(L, 0) for L in RAGGED], n, W.GLOBAL_FLAT, 2)
    grads = _grads(plan, n, W.BF16, 10 + n)
    _step(zf, plan, n, W.BF16, grads, _state_arrays(plan, n))


@pytest.mark.parametrize("n", [2, 5])
def test_stage3_unit_gathers(zf, n):
    """Per-unit FlatParameters at stage 3, then every unit gathered into a
    buffer of exactly P_u elements."""
    plan = zf.plan_flat([(L, u) for u, L in enumerate(RAGGED)], n, W.PER_UNIT, 3)
    grads = _grads(plan, n, W.F16, 20 + n)
    arrays = _state_arrays(plan, n, params_dtype=torch.float16)
    _step(zf, plan, n, W.F16, grads, arrays)
    params = arrays[3]
    for u, info in enumerate(plan.units):
        buf = Guarded(info.P, torch.float16, f"unit buffer {u}")
        shards = [params.data_ptr() + 2 * (info.O + r * info.S) for r in range(n)]
        zf.gather(plan, u, W.F16, shards, buf.t)


def test_fsdp2_step_and_cast_gathers(zf):
    """FSDP2: fp32 gradient shards written by pass 1, fp32 parameters, and
    each group cast-gathered into a buffer of exactly its element count."""
    shapes = [(33, 101), (7, 1), (5, 3), (64, 65), (1, 17), (129, 3)]
    segs = [(r * c, g, 0, r if c > 1 else 0)
            for (r, c), g in zip(shapes, [0, 0, 1, 1, 2, 2])]
    n = 3
    plan = zf.plan_flat(segs, n, W.PER_PARAM_DIM0, 3)
    grads = _grads(plan, n, W.BF16, 31)
    shards = Guarded(plan.summary.psi_pad, torch.float32, "fp32 gradient shards")
    arrays = _state_arrays(plan, 32, fp32_params=True)
    _step(zf, plan, n, W.BF16, grads, arrays, grad_shards=shards.t)
    for g, info in enumerate(plan.groups):
        out = Guarded(info.numel, torch.bfloat16, f"group buffer {g}")
        zf.gather_cast(plan, g, W.BF16, arrays[0], out.t)


def test_buckets_accumulation_and_reduced_step(zf):
    """Buckets reduce-scattered and accumulated over two micro-batches, the
    no_sync accumulation at odd offsets, then the step on the reduced shards."""
    n = 4
    ids, nb = zf.plan_buckets(RAGGED, n, 3000)
    plan = zf.plan_flat([(L, b) for L, b in zip(RAGGED, ids)], n, W.PER_UNIT, 2)
    assert nb >= 3
    grads = _grads(plan, n, W.BF16, 41)
    shards = Guarded(plan.summary.psi_pad, torch.float32, "fp32 gradient shards")
    for micro in range(2):
        for g in range(nb):
            zf.bucket_reduce_scatter(plan, g, W.BF16, grads, shards.t, micro > 0)
    # no_sync: a replica's fp32 accumulation, over sub-ranges at odd offsets
    acc = Guarded(1001, torch.float32, "no_sync accumulator", byte_offset=4)
    src = grads[0][3:3 + 1001]
    zf.accumulate(W.BF16, src, acc.t, accumulate=False)
    zf.accumulate(W.BF16, src, acc.t, accumulate=True)
    _step(zf, plan, n, W.BF16, None, _state_arrays(plan, 42), grad_shards=shards.t,
          grads_reduced=True)


def test_reduce_scatter_alone(zf):
    n = 6
    plan = zf.plan_flat([(L, u) for u, L in enumerate(RAGGED)], n, W.PER_UNIT, 2)
    grads = _grads(plan, n, W.F16, 51)
    out = Guarded(plan.summary.psi_pad, torch.float32, "reduce-scatter output")
    zf.reduce_scatter(plan, W.F16, grads, out.t)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_reshard(zf, dtype):
    """A per-element array re-laid from N = 3 per-unit to N = 5 global flat
    and back into destinations of exactly Psi'(to) elements."""
    a = zf.plan_flat([(L, u) for u, L in enumerate(RAGGED)], 3, W.PER_UNIT, 2)
    b = zf.plan_flat([(L, 0) for L in RAGGED], 5, W.GLOBAL_FLAT, 2)
    src = Guarded(a.summary.psi_pad, dtype, "reshard source")
    src.t.copy_(torch.arange(a.summary.psi_pad, device="cuda").to(dtype))
    mid = Guarded(b.summary.psi_pad, dtype, "reshard destination")
    back = Guarded(a.summary.psi_pad, dtype, "reshard round trip")
    zf.reshard(a, b, src.t, mid.t)
    zf.reshard(b, a, mid.t, back.t)


def test_guard_detects_a_write(zf):
    """The harness itself: a byte changed just past a buffer, or just before
    it, is reported (written through torch into the guard band, which is
    part of the same allocation)."""
    for where in ("after", "before"):
        b = Guarded(1000, torch.float32, "probe")
        Guarded.all.remove(b)
        byte = (b.g + b.numel) * 4 if where == "after" else b.g * 4 - 1
        b.full.view(torch.uint8)[byte] = 0
        torch.cuda.synchronize()
        with pytest.raises(AssertionError, match=where):
            b.check()
