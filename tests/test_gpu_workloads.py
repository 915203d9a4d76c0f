"""Full-size determinism of every workload: two independent runs from
fresh state on the same seeded inputs leave every buffer bitwise identical
and report the same squared norm.  (Full-size parity against the oracle,
element by element, is test_gpu_full_parity.py.)
"""
import pytest
import torch

from fsdp_sharded_mixed_amd import workloads as W
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def R():
    from fsdp_sharded_mixed_amd import runner
    assert torch.cuda.is_available()
    return runner


def _device_buffers(dev):
    out = {n: getattr(dev, n) for n in ("master", "exp_avg", "exp_avg_sq", "params", "state",
                                        "grad_shards", "unit_buf", "group_buf")}
    if dev.main_grads is not None:
        out.update({f"main_grad{q}": t for q, t in enumerate(dev.main_grads)})
    return {k: v for k, v in out.items() if v is not None}


@pytest.mark.parametrize("name", ["llama-73m-n8", "llama-654m-n2", "llama-2.1b-n2-zero3",
                                  "llama-2.1b-n2-fsdp2", "llama-4.06b-n2",
                                  "llama-654m-n2-buckets-a4", "llama-654m-n2-nosync-a4",
                                  "llama-654m-n2-offload"])
def test_full_size_determinism(R, name):
    """Two independent runs of the workload's first two steps (fresh state,
    the same seeded inputs, gathers included) leave every buffer bitwise
    identical, and report the same squared norm: the grids and the
    reduction trees are fixed by the plan, never by timing."""
    G.say(f"determinism {name}")
    torch.cuda.empty_cache()
    w = W.get(name)
    runs, norms = [], []
    for _ in range(2):
        dev = R.DeviceRun(w)
        dev.init_state()
        norms.append([dev.run_workload_step().sumsq for _ in range(2)])
        dev.gather_all()
        runs.append(dev)
    torch.cuda.synchronize()
    assert norms[0] == norms[1]
    a, b = _device_buffers(runs[0]), _device_buffers(runs[1])
    assert a.keys() == b.keys()
    for k in a:
        ta, tb = a[k], b[k]
        if ta.dtype.is_floating_point:
            ta, tb = ta.view(torch.int32 if ta.element_size() == 4 else torch.int16), \
                tb.view(torch.int32 if tb.element_size() == 4 else torch.int16)
        assert torch.equal(ta, tb), f"{name}: {k} differs between two runs"
    del runs, a, b
    torch.cuda.empty_cache()
