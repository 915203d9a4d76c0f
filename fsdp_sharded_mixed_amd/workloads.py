"""The synthetic workloads: parameter segments, sharding, dtypes and hyperparameters.

Pure input description -- no step arithmetic lives here.  The tests, the bench
and the smoke check read it to drive both the HIP library and the CPU oracle
with the same seeded inputs.

Shapes:
  * tiny: a 5-layer MLP of Psi = 32,656 parameters with one W||b FlatParameter
    per Linear layer (CMU 15-779 Lecture 13 notes, 0.4: the simulator's MLP
    and its per-layer units), flats of 5248, 16512, 8256, 2080 and 560.
  * Llama-style decoders with the two model shapes of Femtotron dev log #10's
    memory tables: hidden 1024 / intermediate 2048 / 16 heads / 4 KV heads /
    vocab 1024, and hidden 2048 / intermediate 8192 / 32 heads / 8 KV heads /
    vocab 40960 (head_dim 64 in both), untied embedding and LM head.
    Parameter order: embedding, then per layer q, k, v, o, gate, up, down,
    input norm, post-attention norm (Femtotron dev log #7 lists nine tensors
    per layer, q/k/v/o first), then the final norm and the LM head; each
    Linear weight is row-major [out, in].
  * FSDP units for the ZeRO-3 and FSDP2 workloads: {embedding}, one unit
    per decoder layer, {final norm, LM head} (the torchtitan FSDP2 wrapping
    of the Megatron / DeepSpeed / torchtitan source guide, ch. 五.4).
  * Gradient buckets for the accumulation workloads: Megatron's buffer holds
    the parameters last layer first and cuts it into buckets of
    max(40M, 1M * N) elements (source guide, ch. 三.3).

Inputs are a pure function of (seed, stream, logical index): a replica's
gradient for element i at step k (micro-batch a) comes from stream
grad_stream(k, replica, a),
the fp32 master initialisation from STREAM_MASTER, and the index that receives
an injected +inf from the first output of STREAM_INJECT.  The generator is
splitmix64 feeding an Irwin-Hall(12) normal; both the HIP input library and
the CPU oracle implement it from that definition.
"""
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

F16, BF16 = 1, 2
GLOBAL_FLAT, PER_UNIT, PER_PARAM_DIM0 = 0, 1, 2

KIND_WEIGHT, KIND_BIAS, KIND_NORM = 0, 1, 2

STREAM_MASTER = 1 << 40
STREAM_INJECT = 2 << 40


ACCUM_REDUCE_EACH, ACCUM_NO_SYNC = 0, 1


def grad_stream(step: int, replica: int, micro: int = 0) -> int:
    """Stream id of replica `replica`'s gradient in micro-batch `micro` of
    step `step` (steps count from 1, micro-batches from 0; a step without
    accumulation is micro-batch 0)."""
    assert 1 <= step < (1 << 20) and 0 <= replica < 256 and 0 <= micro < 4096
    return (step << 20) | (micro << 8) | replica


@dataclass
class Segment:
    name: str
    numel: int
    unit: int
    kind: int = KIND_WEIGHT
    rows: int = 0  # dim-0 size ([out, in] weights: out); 0 for 1-D tensors


@dataclass
class Workload:
    name: str
    description: str
    segments: List[Segment]
    n_ranks: int
    layout: int
    stage: int
    grad_dtype: int
    param_dtype: int
    sigma: float                 # per-replica gradient standard deviation
    loss_scale: float            # initial loss scale S
    dynamic: bool                # dynamic loss scaling (halve on overflow)
    lr: float
    steps: int
    seed: int
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.01
    max_norm: float = 1.0
    growth_interval: int = 2000
    master_sigma: float = 0.02
    norm_weights_one: bool = False
    inject_step: Optional[int] = None      # +inf injected into one replica at this step
    inject_replica: int = 1
    fp32_params: bool = False              # FSDP2: the fp32 shard is the parameter
    # gradient accumulation over n_micro micro-batches: ACCUM_REDUCE_EACH
    # reduce-scatters every micro-batch into the fp32 gradient shard,
    # ACCUM_NO_SYNC accumulates each replica locally in fp32 and reduces once
    n_micro: int = 1
    accum_mode: int = ACCUM_REDUCE_EACH
    # None: FSDP units from the segments' unit ids.  Otherwise Megatron
    # gradient buckets over the segments in the given order (0: the default
    # bucket size max(40M, 1M * N)); each side computes the bucket ids itself
    bucket_numel: Optional[int] = None
    # ZeRO-Offload: fp32 master / moments and the update on the host
    # (CPU-Adam), 16-bit parameters on the GPU
    offload: bool = False
    # ZeRO-Offload with 16-bit gradients down (the sums rounded to the
    # gradient dtype; norm and overflow on the rounded values)
    offload_down16: bool = False
    extra: dict = field(default_factory=dict)

    @property
    def backward_rs(self) -> bool:
        """The gradients are reduce-scattered bucket by bucket during backward
        and the step consumes the reduced fp32 gradient shards."""
        return self.bucket_numel is not None or self.n_micro > 1

    @property
    def psi(self) -> int:
        return sum(s.numel for s in self.segments)

    def seg_arrays(self) -> Tuple[List[int], List[int]]:
        return [s.numel for s in self.segments], [s.unit for s in self.segments]

    def norm_ranges(self) -> List[Tuple[int, int]]:
        """Logical [start, end) ranges of RMSNorm weight segments."""
        out, pos = [], 0
        for s in self.segments:
            if s.kind == KIND_NORM:
                out.append((pos, pos + s.numel))
            pos += s.numel
        return out


def llama_segments(hidden, inter, heads, kv_heads, layers, vocab, head_dim=64,
                   per_layer_units=False) -> List[Segment]:
    q = heads * head_dim
    kv = kv_heads * head_dim
    segs = [Segment("embed", vocab * hidden, 0, rows=vocab)]
    for i in range(layers):
        u = i + 1 if per_layer_units else 0
        segs += [
            Segment(f"l{i}.q", q * hidden, u, rows=q),
            Segment(f"l{i}.k", kv * hidden, u, rows=kv),
            Segment(f"l{i}.v", kv * hidden, u, rows=kv),
            Segment(f"l{i}.o", hidden * q, u, rows=hidden),
            Segment(f"l{i}.gate", inter * hidden, u, rows=inter),
            Segment(f"l{i}.up", inter * hidden, u, rows=inter),
            Segment(f"l{i}.down", hidden * inter, u, rows=hidden),
            Segment(f"l{i}.input_norm", hidden, u, KIND_NORM),
            Segment(f"l{i}.post_norm", hidden, u, KIND_NORM),
        ]
    last = layers + 1 if per_layer_units else 0
    segs += [Segment("final_norm", hidden, last, KIND_NORM),
             Segment("lm_head", vocab * hidden, last, rows=vocab)]
    return segs


def tiny_segments() -> List[Segment]:
    return [Segment(f"fc{i}", n, i) for i, n in enumerate([5248, 16512, 8256, 2080, 560])]


def _h1024(layers):
    return llama_segments(1024, 2048, 16, 4, layers, 1024)


def _h2048(layers, per_layer_units=False):
    return llama_segments(2048, 8192, 32, 8, layers, 40960, per_layer_units=per_layer_units)


def tiny(stage=2) -> Workload:
    return Workload(
        name=f"tiny-mlp-n4-z{stage}",
        description="5-layer MLP, Psi=32,656, per-layer W||b units, N=4, fp16 grads "
                    "N(0,1e-3)*65536 under dynamic loss scaling",
        segments=tiny_segments(), n_ranks=4, layout=PER_UNIT, stage=stage,
        grad_dtype=F16, param_dtype=F16, sigma=1e-3, loss_scale=65536.0, dynamic=True,
        lr=1e-3, steps=10, seed=1)


def llama73m() -> Workload:
    return Workload(
        name="llama-73m-n8",
        description="Llama-style decoder h1024/i2048/16h/4kv/8L/V1024, Psi=73,417,728, "
                    "one global flat, N=8, bf16 grads N(0,1e-3), norm weights 1.0",
        segments=_h1024(8), n_ranks=8, layout=GLOBAL_FLAT, stage=2,
        grad_dtype=BF16, param_dtype=BF16, sigma=1e-3, loss_scale=1.0, dynamic=False,
        lr=1e-4, steps=10, seed=2, norm_weights_one=True)


def llama654m() -> Workload:
    n = 2
    psi = sum(s.numel for s in _h2048(8))
    return Workload(
        name="llama-654m-n2",
        description="Llama-style decoder h2048/i8192/32h/8kv/8L/V40960, Psi=654,346,240, "
                    "one global flat, N=2, bf16 grads scaled so the global norm is about 3",
        segments=_h2048(8), n_ranks=n, layout=GLOBAL_FLAT, stage=2,
        grad_dtype=BF16, param_dtype=BF16, sigma=3.0 * (n / psi) ** 0.5, loss_scale=1.0,
        dynamic=False, lr=1e-4, steps=5, seed=3)


def llama2b_z3() -> Workload:
    return Workload(
        name="llama-2.1b-n2-zero3",
        description="Llama-style decoder h2048/i8192/32h/8kv/32L/V40960, Psi=2,114,062,336, "
                    "34 FSDP units, N=2, ZeRO-3 per-unit bf16 gather into a reused buffer",
        segments=_h2048(32, per_layer_units=True), n_ranks=2, layout=PER_UNIT, stage=3,
        grad_dtype=BF16, param_dtype=BF16, sigma=1e-3, loss_scale=1.0, dynamic=False,
        lr=1e-4, steps=3, seed=4)


def llama2b_fsdp2() -> Workload:
    """The 2.1B decoder under FSDP2 as torchtitan runs it by default (source
    guide 五.4 and 五.6): every parameter sharded along dim 0, fp32 shards
    that are the parameters, fp32 reduce-scatter into resident fp32 gradient
    shards, bf16 only when a unit (a decoder layer) is gathered."""
    return Workload(
        name="llama-2.1b-n2-fsdp2",
        description="Llama-style decoder h2048/i8192/32h/8kv/32L/V40960, Psi=2,114,062,336, "
                    "FSDP2 per-parameter dim-0 shards over N=2, fp32 parameters and grad "
                    "shards, bf16 cast at the 34 unit gathers",
        segments=_h2048(32, per_layer_units=True), n_ranks=2, layout=PER_PARAM_DIM0, stage=3,
        grad_dtype=BF16, param_dtype=BF16, sigma=1e-3, loss_scale=1.0, dynamic=False,
        lr=1e-4, steps=3, seed=4, fp32_params=True)


def llama4b() -> Workload:
    return Workload(
        name="llama-4.06b-n2",
        description="Llama-style decoder h2048/i8192/32h/8kv/64L/V40960, Psi=4,060,350,464, "
                    "one global flat, N=2, fp16 grads N(0,1e-3)*32768 under dynamic loss "
                    "scaling, +inf injected into replica 1 at step 2",
        segments=_h2048(64), n_ranks=2, layout=GLOBAL_FLAT, stage=2,
        grad_dtype=F16, param_dtype=F16, sigma=1e-3, loss_scale=32768.0, dynamic=True,
        lr=1e-4, steps=4, seed=5, inject_step=2, inject_replica=1)


def _h2048_buckets(layers):
    """Megatron's buffer order: parameters last layer first (the order in
    which backward produces their gradients); bucket ids assigned later."""
    return list(reversed(_h2048(layers)))


def llama654m_buckets(mode=ACCUM_REDUCE_EACH) -> Workload:
    """The 654M decoder in Megatron's gradient buffer (reverse order, default
    40M-element buckets padded to N) with four accumulated micro-batches:
    every bucket is reduce-scattered as its gradients arrive, into fp32
    gradient shards (or, no_sync, each replica accumulates in fp32 and the
    buckets are reduced once after the last micro-batch); then the step."""
    n, a = 2, 4
    psi = sum(s.numel for s in _h2048(8))
    tag = "buckets" if mode == ACCUM_REDUCE_EACH else "nosync"
    how = ("reduce-scatter of every micro-batch into fp32 grad shards"
           if mode == ACCUM_REDUCE_EACH else
           "no_sync fp32 local accumulation, one reduce-scatter at the last micro-batch")
    return Workload(
        name=f"llama-654m-n2-{tag}-a4",
        description="Llama-style decoder h2048/i8192/32h/8kv/8L/V40960, Psi=654,346,240, "
                    "Megatron buffer order with 40M-element gradient buckets, N=2, 4 "
                    f"micro-batches of bf16 grads, {how}, global norm about 3",
        segments=_h2048_buckets(8), n_ranks=n, layout=PER_UNIT, stage=2,
        grad_dtype=BF16, param_dtype=BF16, sigma=3.0 * (n / (psi * a)) ** 0.5, loss_scale=1.0,
        dynamic=False, lr=1e-4, steps=3, seed=6 if mode == ACCUM_REDUCE_EACH else 7,
        n_micro=a, accum_mode=mode, bucket_numel=0)


def llama654m_offload() -> Workload:
    """The 654M decoder under ZeRO-Offload: the GPU keeps the replicas, the
    reduce-scatter and norm passes and the bf16 parameters; the fp32 state
    and the AdamW update live on the host (lecture notes 7.1-7.2)."""
    w = llama654m()
    w.name = "llama-654m-n2-offload"
    w.description = ("Llama-style decoder h2048/i8192/32h/8kv/8L/V40960, Psi=654,346,240, "
                     "one global flat, N=2, bf16 grads (global norm about 3), ZeRO-Offload: "
                     "fp32 state and CPU-Adam on the host, bf16 params uploaded in chunks")
    w.offload, w.seed, w.steps = True, 8, 3
    return w


def llama654m_offload16() -> Workload:
    """The offload workload with the pages' 16-bit gradient edge: the
    reduce-scatter sums go down PCIe rounded to bf16 (2 B per parameter)."""
    w = llama654m_offload()
    w.name = "llama-654m-n2-offload16"
    w.description = w.description.replace("ZeRO-Offload:", "ZeRO-Offload with bf16 sums down:")
    w.offload_down16, w.seed = True, 9
    return w


ALL = {
    "tiny": tiny,
    "llama-73m-n8": llama73m,
    "llama-654m-n2": llama654m,
    "llama-2.1b-n2-zero3": llama2b_z3,
    "llama-2.1b-n2-fsdp2": llama2b_fsdp2,
    "llama-4.06b-n2": llama4b,
    "llama-654m-n2-buckets-a4": llama654m_buckets,
    "llama-654m-n2-nosync-a4": lambda: llama654m_buckets(ACCUM_NO_SYNC),
    "llama-654m-n2-offload": llama654m_offload,
    "llama-654m-n2-offload16": llama654m_offload16,
}


def get(name: str) -> Workload:
    return ALL[name]()
