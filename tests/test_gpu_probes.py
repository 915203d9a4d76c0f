"""The bandwidth probes compute what they claim, so that their GB/s figures
count bytes really moved: every output element is checked against numpy's
binary32 arithmetic, and a guard band after every array stays untouched.

* zfi_stream_probe / zfi_stream_probe_shaped: every destination holds the
  sum of the sources in order from 0 (binary32), for several source and
  destination counts, quads per lane and occupancy caps.
* zfi_update_mix_probe: p, m and v each gain x (bf16(g0[i]) + bf16(g1[i]),
  or sums[i]) and out16[i] is the top half of the new p[i], for both block
  sizes and two caps.

Sizes are ragged against every tile (a quad count that no block size
divides).
"""
import numpy as np
import pytest
import torch

from fsdp_sharded_mixed_amd import inputs as I

pytestmark = pytest.mark.gpu

N = 4 * 3001   # 3001 quads: no block of 128 or 256 threads, or 2-4 quads, divides it
GUARD = 1024   # elements after every array
SENT32 = 0x7FC0DEAD
SENT16 = 0x7FAB


def _guarded(vals, dtype):
    """A device array of len(vals) + GUARD elements: vals, then a sentinel."""
    bits = torch.int32 if dtype == torch.float32 else torch.int16
    t = torch.empty(len(vals) + GUARD, dtype=dtype, device="cuda")
    t[:len(vals)] = torch.as_tensor(vals).to(device="cuda", dtype=dtype)
    t.view(bits)[len(vals):] = SENT32 if bits == torch.int32 else np.int16(np.uint16(SENT16))
    return t


def _guard_intact(t):
    if t.dtype == torch.float32:
        return bool((t.view(torch.int32)[-GUARD:] == SENT32).all())
    return bool((t.view(torch.int16)[-GUARD:] == int(np.int16(np.uint16(SENT16)))).all())


def _f32(t, n=N):
    return t[:n].cpu().numpy()


@pytest.mark.parametrize("r,w", [(1, 1), (2, 2), (4, 4), (8, 1)])
def test_stream_probes_write_the_ordered_sum(r, w):
    rng = np.random.default_rng(100 + 10 * r + w)
    srcs_np = [rng.standard_normal(N).astype(np.float32) for _ in range(r)]
    want = np.zeros(N, dtype=np.float32)
    for x in srcs_np:
        want = want + x
    srcs = [_guarded(x, torch.float32) for x in srcs_np]
    runs = [("fixed", lambda d: I.stream_probe(srcs, d, n=N))]
    runs += [(f"q{q}c{c}", lambda d, q=q, c=c: I.stream_probe_shaped(srcs, d, q, c, n=N))
             for q in (1, 2, 4) for c in (0, 4)]
    for name, run in runs:
        dsts = [_guarded(np.zeros(N, dtype=np.float32), torch.float32) for _ in range(w)]
        run(dsts)
        torch.cuda.synchronize()
        for k, d in enumerate(dsts):
            assert np.array_equal(_f32(d).view(np.uint32), want.view(np.uint32)), (name, k)
            assert _guard_intact(d), (name, k)
        for s in srcs:
            assert _guard_intact(s)


def _bf16_to_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("replicas", [True, False])
def test_update_mix_probe_moves_and_adds_every_element(replicas):
    rng = np.random.default_rng(7 if replicas else 8)
    p0, m0, v0 = (rng.standard_normal(N).astype(np.float32) for _ in range(3))
    if replicas:
        g0b, g1b = (torch.randn(N, dtype=torch.float32).to(torch.bfloat16)
                    .view(torch.int16).numpy().view(np.uint16) for _ in range(2))
        x = _bf16_to_f32(g0b) + _bf16_to_f32(g1b)
        g = tuple(_guarded(torch.from_numpy(b.view(np.int16)).view(torch.bfloat16), torch.bfloat16)
                  for b in (g0b, g1b))
    else:
        x = rng.standard_normal(N).astype(np.float32)
        g = _guarded(x, torch.float32)
    for t in (128, 256):
        for c in (0, 3):
            p, m, v = (_guarded(a, torch.float32) for a in (p0, m0, v0))
            o = _guarded(np.zeros(N, dtype=np.float32), torch.bfloat16)
            I.update_mix_probe(g, p, m, v, o, N, t, c)
            torch.cuda.synchronize()
            for name, dev, ref in (("p", p, p0), ("m", m, m0), ("v", v, v0)):
                assert np.array_equal(_f32(dev).view(np.uint32), (ref + x).view(np.uint32)), \
                    (t, c, name)
                assert _guard_intact(dev), (t, c, name)
            got16 = o[:N].view(torch.int16).cpu().numpy().view(np.uint16)
            want16 = ((p0 + x).view(np.uint32) >> 16).astype(np.uint16)
            assert np.array_equal(got16, want16), (t, c)
            assert _guard_intact(o), (t, c)
            for a in (g if replicas else (g,)):
                assert _guard_intact(a)
