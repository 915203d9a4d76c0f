"""Shared helpers of the GPU parity tests: oracle-vs-device comparisons.

The device side runs only through the C ABI (runner.DeviceRun ->
fsdp_sharded_mixed_amd.zf).  The oracle side computes its own inputs with
its own generator; expected values come only from the oracle.
"""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle as O
from tests import oracle_inputs as OI

POOL_THREADS = min(16, os.cpu_count() or 1)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits16(t):
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def bits32(t):
    return t.detach().view(torch.int32).cpu().numpy().view(np.uint32)


def bits_view(t):
    """A device tensor's bits as integers of its element size (bitwise
    comparison with torch.equal: NaN payloads and signed zeros count)."""
    return t.view(torch.int32 if t.element_size() == 4 else torch.int16)


def f32(t):
    return t.detach().cpu().numpy()


def ulp_distance(a, b):
    """|a - b| in units in the last place of binary32 (sign-magnitude order)."""
    ia = a.view(np.int32).astype(np.int64)
    ib = b.view(np.int32).astype(np.int64)
    ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
    ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
    return np.abs(ia - ib)


def ulp16_distance(a, b):
    ia = a.astype(np.int64)
    ib = b.astype(np.int64)
    ia = np.where(ia & 0x8000, -(ia & 0x7FFF), ia)
    ib = np.where(ib & 0x8000, -(ib & 0x7FFF), ib)
    return np.abs(ia - ib)


def assert_state_close(name, dev, ref, max_ulp=4):
    """fp32 arrays: within max_ulp ulp (relative ~1e-6), and report exact share."""
    d = ulp_distance(dev, ref)
    worst = int(d.max()) if d.size else 0
    assert worst <= max_ulp, f"{name}: {worst} ulp apart at {int(d.argmax())}"
    return float((d == 0).mean()) if d.size else 1.0


def assert_result_matches(res_dev, res_orc, what=""):
    assert res_dev.overflow == res_orc.overflow, what
    assert res_dev.skipped == res_orc.skipped, what
    assert res_dev.t == res_orc.t, what
    assert res_dev.scale_next == res_orc.scale_next, what
    if not res_orc.skipped:
        assert res_dev.scale_used == res_orc.scale_used, what
        rel = abs(res_dev.norm - res_orc.norm) / max(abs(res_orc.norm), 1e-300)
        assert rel <= 1e-5, f"{what}: norm {res_dev.norm} vs {res_orc.norm}"
        assert abs(res_dev.coef - res_orc.coef) <= 1e-5 * max(res_orc.coef, 1e-300)


def oracle_padded_state(run):
    """Oracle per-rank shard buffers -> padded-flat arrays (the device layout)."""
    u = run.units
    return (OI.rank_shards_to_padded(u, run.master), OI.rank_shards_to_padded(u, run.m),
            OI.rank_shards_to_padded(u, run.v))


def oracle_padded_params(run):
    if run.full is not None:
        return run.full
    return OI.rank_shards_to_padded(run.units, run.shards)


def regen_sumsq_threaded(w, step, scale, psi, inject=None, chunks=None):
    """Exact global sum of squared reduced (and, over the workload's
    micro-batches, accumulated) gradients and the overflow flag by
    regeneration, split over a thread pool; partials added in order."""
    chunks = chunks or max(POOL_THREADS * 4, 1)
    edges = np.linspace(0, psi, chunks + 1).astype(np.int64)

    def part(k):
        return O.regen_accum_sumsq(w.grad_dtype, w.n_ranks, w.n_micro, w.accum_mode, w.seed,
                                   step, w.sigma, scale, int(edges[k]), int(edges[k + 1]),
                                   inject)

    with ThreadPoolExecutor(POOL_THREADS) as ex:
        parts = list(ex.map(part, range(chunks)))
    ss = 0.0
    bad = 0
    for s, b in parts:
        ss += s
        bad |= b
    return ss, bad
