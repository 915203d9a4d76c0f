"""zf_shard_step_noalloc (the step with the library's static scratch as its
workspace) against zf_shard_step (a caller workspace) on the GPU, through
the C ABI.

The two entry points run the same kernels on the same grids, so the bar is
bit-for-bit equality of everything the step writes: fp32 master, exp_avg,
exp_avg_sq, the 16-bit parameters, the fp32 gradient shards when given,
and the step result in the state block.  Each case runs several steps on
twin runs fed the same replicas; the calls come in a row on one GPU, a
larger plan first and then a smaller one, so the second reuses a scratch
that still holds the first one's contents.
"""
import pytest
import torch

from fsdp_sharded_mixed_amd import workloads as W
from fsdp_sharded_mixed_amd import zf
from tests import gpu_common as G

pytestmark = pytest.mark.gpu

RESULT_FIELDS = ("overflow", "skipped", "t", "sumsq", "norm", "coef", "scale_used",
                 "scale_next", "gs", "growth_ctr", "bc1", "bc2")


@pytest.fixture(scope="module")
def R():
    from fsdp_sharded_mixed_amd import runner
    assert torch.cuda.is_available()
    return runner


def flat_workload(n, psi, gdt=W.BF16, seed=41, steps=3):
    dyn = gdt == W.F16
    return W.Workload(name=f"flat-{psi}-n{n}", description="", n_ranks=n,
                      segments=[W.Segment("flat", psi, 0)], layout=W.GLOBAL_FLAT, stage=2,
                      grad_dtype=gdt, param_dtype=gdt, sigma=1e-3,
                      loss_scale=4096.0 if dyn else 1.0, dynamic=dyn, lr=1e-3, steps=steps,
                      seed=seed, max_norm=0.5)


def fsdp2_workload():
    shapes = [(37, 64), (64, 1), (101, 48), (48, 1), (5, 7)]
    segs = [W.Segment(f"p{i}", r * c, i // 2, rows=r if c > 1 else 0)
            for i, (r, c) in enumerate(shapes)]
    return W.Workload(name="fsdp2-small-n3", description="", segments=segs, n_ranks=3,
                      layout=W.PER_PARAM_DIM0, stage=3, grad_dtype=W.BF16, param_dtype=W.BF16,
                      sigma=1e-2, loss_scale=1.0, dynamic=False, lr=1e-3, steps=3, seed=43,
                      max_norm=0.5, fp32_params=True)


def bits(t):
    return t.view(torch.int32 if t.element_size() == 4 else torch.int16)


def run_twins(R, w, with_shards=False, side_stream=False):
    """Twin runs of w: `a` steps with zf_shard_step and its workspace, `b`
    with zf_shard_step_noalloc; every output compared bit for bit."""
    G.say(f"noalloc case {w.name}: Psi={w.psi:,} N={w.n_ranks} shards={with_shards} "
          f"side_stream={side_stream}")
    a, b = R.DeviceRun(w), R.DeviceRun(w)
    plan = b.plan
    assert plan.summary.workspace_bytes <= zf.NOALLOC_SCRATCH_BYTES or with_shards
    for run in (a, b):
        run.init_state()
        if with_shards:
            run.grad_shards = torch.zeros(run.psi_pad, dtype=torch.float32, device=run.device)
    s = torch.cuda.Stream() if side_stream else None
    for k in range(1, w.steps + 1):
        a.fill_grads(k, a.loss_scale)
        for ga, gb in zip(a.grads, b.grads):
            gb.copy_(ga)
        if w.inject_step == k:
            a.inject_inf()
            b.inject_inf()
        a.step()
        if s is not None:
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                zf.shard_step_noalloc(plan, b.hp, w.grad_dtype, w.param_dtype, b.grads, b.master,
                                      b.exp_avg, b.exp_avg_sq, b.params, b.state, stream=s,
                                      grad_shards=b.grad_shards)
            torch.cuda.current_stream().wait_stream(s)
        else:
            zf.shard_step_noalloc(plan, b.hp, w.grad_dtype, w.param_dtype, b.grads, b.master,
                                  b.exp_avg, b.exp_avg_sq, b.params, b.state,
                                  grad_shards=b.grad_shards)
        ra, rb = a.result(), b.result()
        for f in RESULT_FIELDS:
            assert getattr(ra, f) == getattr(rb, f), f"{w.name} step {k}: {f}"
        a.loss_scale = b.loss_scale = ra.scale_next
        for name in ("master", "exp_avg", "exp_avg_sq", "params", "grad_shards"):
            ta, tb = getattr(a, name), getattr(b, name)
            if ta is None:
                continue
            assert torch.equal(bits(ta), bits(tb)), f"{w.name} step {k}: {name} differs"
        G.say(f"  step {k}: skipped={rb.skipped} t={rb.t} norm={rb.norm:.6f} equal")
    torch.cuda.synchronize()
    return a, b


def test_noalloc_equals_step_large_then_small(R):
    """Two plans in a row: N = 8 materialising its sums in the scratch (a
    ragged 3,000,011-element flat, 12 MB of sums), then the smaller tiny
    MLP at N = 4 recomputing them (fp16 under a dynamic loss scale)."""
    big = flat_workload(8, 3_000_011)
    pb = zf.plan_flat(big.segments, big.n_ranks, big.layout, big.stage)
    assert pb.summary.policy == 1 and pb.summary.workspace_bytes > 12_000_000
    run_twins(R, big)
    small = W.tiny(stage=3)
    small.steps = 3
    run_twins(R, small)


def test_noalloc_sums_in_grad_shards(R):
    """A plan whose sums do not fit the scratch (N = 8, 20M elements: 80 MB
    of sums) runs when the caller gives fp32 gradient shards, which then
    hold the sums; then a smaller plan of the same kind."""
    w = flat_workload(8, 20_000_003, steps=2)
    assert zf.plan_flat(w.segments, 8, w.layout, w.stage).summary.workspace_bytes > \
        zf.NOALLOC_SCRATCH_BYTES
    run_twins(R, w, with_shards=True)
    run_twins(R, flat_workload(6, 1_000_001, steps=2), with_shards=True)


def test_noalloc_fsdp2_and_skip_on_a_side_stream(R):
    """FSDP2 (the sums into the resident fp32 gradient shards, no 16-bit
    copy), then N = 2 fp16 with +inf injected at step 2 (skipped, loss scale
    halved), both launched on a non-default stream."""
    run_twins(R, fsdp2_workload(), side_stream=True)
    w = flat_workload(2, 500_003, gdt=W.F16, steps=3)
    w.inject_step, w.inject_replica = 2, 1
    a, b = run_twins(R, w, side_stream=True)
    assert b.result().t == 2 and b.loss_scale == 2048.0


def test_noalloc_in_a_captured_graph(R):
    """Code under HIP graph capture is one of the callers the entry point is
    for.  Step 1 runs eagerly (the first call on the device looks up the
    scratch's address); steps 2.. replay one captured call.  An eager twin
    steps with zf_shard_step on the same replicas; after every replay the
    two agree bit for bit.  N = 8 with the sums in the scratch, then N = 3
    in fp16 with +inf at step 3, skipped inside a replay."""
    for w, inject in ((flat_workload(8, 1_000_003, steps=4), None),
                      (flat_workload(3, 300_007, gdt=W.F16, steps=5), 3)):
        G.say(f"noalloc graph case {w.name}")
        a, b = R.DeviceRun(w), R.DeviceRun(w)
        a.init_state()
        b.init_state()

        def noalloc_step():
            zf.shard_step_noalloc(b.plan, b.hp, w.grad_dtype, w.param_dtype, b.grads, b.master,
                                  b.exp_avg, b.exp_avg_sq, b.params, b.state)

        graph = None
        for k in range(1, w.steps + 1):
            a.fill_grads(k, a.loss_scale)
            if inject == k:
                a.grads[w.inject_replica][17] = float("inf")
            for ga, gb in zip(a.grads, b.grads):
                gb.copy_(ga)
            a.step()
            if k == 1:
                noalloc_step()
            else:
                if graph is None:
                    torch.cuda.synchronize()
                    graph = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(graph):
                        noalloc_step()
                graph.replay()
            torch.cuda.synchronize()
            ra, rb = a.result(), b.result()
            for f in RESULT_FIELDS:
                assert getattr(ra, f) == getattr(rb, f), f"{w.name} step {k}: {f}"
            a.loss_scale = ra.scale_next
            for name in ("master", "exp_avg", "exp_avg_sq", "params"):
                assert torch.equal(bits(getattr(a, name)), bits(getattr(b, name))), \
                    f"{w.name} step {k}: {name}"
            G.say(f"  step {k}: skipped={rb.skipped} t={rb.t} equal "
                  f"({'eager' if k == 1 else 'replay'})")
        assert b.result().t == w.steps - (1 if inject else 0)
        del graph
