"""Device buffers and the step sequence for one workload on one GPU.

torch supplies device memory and the stream; libzf_inputs fills the seeded
inputs; every step runs through the libzf C ABI (fsdp_sharded_mixed_amd.zf).

All per-element arrays use the padded flat index p of include/zf.h: the N
ranks' shards of unit u sit side by side at [O_u, O_u + P_u).
"""
import torch

from . import inputs as I
from . import workloads as W
from . import zf

TORCH_16 = {W.F16: torch.float16, W.BF16: torch.bfloat16}


def plan_workload(w):
    """The library's plan of a workload: its FSDP units, or Megatron gradient
    buckets from zf_plan_buckets when the workload is bucketed."""
    segs = w.segments
    if w.bucket_numel is not None:
        ids, _ = zf.plan_buckets([sg.numel for sg in segs], w.n_ranks, w.bucket_numel)
        segs = [(sg.numel, ids[i], sg.kind, sg.rows) for i, sg in enumerate(segs)]
    return zf.plan_flat(segs, w.n_ranks, w.layout, w.stage)


class DeviceRun:
    """A workload's device state: N replicas, fp32 master/m/v, 16-bit params,
    workspace and state block, plus a reused unit buffer for stage 3."""

    def __init__(self, w, device="cuda:0", grads=True, resident_micro=False):
        """resident_micro: keep all n_micro micro-batches' replicas resident
        (the bench's inputs), instead of refilling one set per micro-batch."""
        self.w = w
        self.device = torch.device(device)
        self.plan = plan_workload(w)
        s = self.plan.summary
        self.psi, self.psi_pad = s.psi, s.psi_pad
        n, dev = s.psi_pad, self.device
        gdt, pdt = TORCH_16[w.grad_dtype], TORCH_16[w.param_dtype]
        n_sets = w.n_micro if (resident_micro and w.backward_rs) else 1
        self.micro_grads = [[torch.zeros(n, dtype=gdt, device=dev) for _ in range(w.n_ranks)]
                            if grads else [] for _ in range(n_sets)]
        self.grads = self.micro_grads[0]
        # no_sync: every replica's fp32 local accumulation buffer (main_grad)
        self.main_grads = ([torch.zeros(n, dtype=torch.float32, device=dev)
                            for _ in range(w.n_ranks)]
                           if w.backward_rs and w.accum_mode == W.ACCUM_NO_SYNC else None)
        # ZeRO-Offload keeps the fp32 state on the host: the master and both
        # moments in host memory, pinned staging for the sums coming down and
        # the 16-bit parameters going up
        sdev = torch.device("cpu") if w.offload else dev
        self.master = torch.zeros(n, dtype=torch.float32, device=sdev)
        self.exp_avg = torch.zeros(n, dtype=torch.float32, device=sdev)
        self.exp_avg_sq = torch.zeros(n, dtype=torch.float32, device=sdev)
        if w.offload:
            self.h_grad = torch.empty(n, dtype=torch.float32, pin_memory=True)
            self.h_params = torch.empty(n, dtype=pdt, pin_memory=True)
            self.h_state = torch.empty(zf.state_bytes(), dtype=torch.uint8, pin_memory=True)
        self.n_threads = 0   # CPU-Adam threads (0: every hardware thread)
        self.n_chunks = 8    # offload pipeline chunks
        self.last_result = None
        # FSDP2 keeps fp32 parameters (no 16-bit copy) and resident fp32
        # gradient shards; the other layouts keep a 16-bit copy
        self.params = None if w.fp32_params else torch.zeros(n, dtype=pdt, device=dev)
        self.grad_shards = (torch.zeros(n, dtype=torch.float32, device=dev)
                            if s.policy == 2 or w.backward_rs or w.offload else None)
        self.workspace = torch.empty(max(1, s.workspace_bytes), dtype=torch.uint8, device=dev)
        self.state = torch.empty(zf.state_bytes(), dtype=torch.uint8, device=dev)
        self.unit_buf = (torch.empty(s.max_unit_pad, dtype=pdt, device=dev)
                         if w.stage == 3 and not w.fp32_params else None)
        self.group_buf = (torch.empty(s.max_group_numel, dtype=pdt, device=dev)
                          if w.fp32_params else None)
        self.hp = zf.hparams(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay, w.max_norm)
        self.step_no = 0
        self.loss_scale = w.loss_scale

    # ---- inputs ------------------------------------------------------------
    def logical_to_padded(self, i):
        for u in self.plan.units:
            if u.lam <= i < u.lam + u.L:
                return u.O + (i - u.lam)
        raise IndexError(i)

    def init_state(self):
        """fp32 master from the seeded stream (norm weights 1.0 where the
        workload says so), m = v = 0, 16-bit params = RNE(master), t = 0."""
        w = self.w
        master = (torch.zeros(self.psi_pad, dtype=torch.float32, device=self.device)
                  if w.offload else self.master)
        master.zero_()
        for u in self.plan.units:
            I.fill_normal32(master, u.L, w.seed, W.STREAM_MASTER, u.lam, w.master_sigma,
                            offset=u.O)
        if w.norm_weights_one:
            for a, b in w.norm_ranges():
                pa = self.logical_to_padded(a)
                master[pa:pa + (b - a)] = 1.0
        self.exp_avg.zero_()
        self.exp_avg_sq.zero_()
        if self.params is not None:
            self.params.copy_(master.to(self.params.dtype))
        if w.offload:
            self.master.copy_(master.cpu())
            del master
        zf.state_init(self.state, w.loss_scale, w.dynamic, w.growth_interval)
        self.step_no = 0
        self.loss_scale = w.loss_scale

    def fill_grads(self, step, scale, sigma=None, micro=0, bufs=None):
        """Replica q's gradient for `step` (micro-batch `micro`) into bufs
        (default self.grads), keyed by logical index (pads stay 0)."""
        w = self.w
        sigma = w.sigma if sigma is None else sigma
        for q, g in enumerate(self.grads if bufs is None else bufs):
            for u in self.plan.units:
                I.fill_normal16(g, u.L, w.grad_dtype, w.seed, W.grad_stream(step, q, micro),
                                u.lam, sigma, scale, offset=u.O)
                if u.P > u.L:  # the padding must be zero (a test may have poisoned it)
                    g[u.O + u.L:u.O + u.P].zero_()

    def fill_micro(self, step, scale):
        """Every micro-batch of `step` into the resident sets (and the
        injection into micro-batch 0 when it is due)."""
        for a, bufs in enumerate(self.micro_grads):
            self.fill_grads(step, scale, micro=a, bufs=bufs)
        if self.w.inject_step == step:
            self.inject_inf(self.micro_grads[0])

    def inject_inf(self, bufs=None):
        """+inf into the workload's inject replica at its inject index."""
        i = I.inject_index(self.w, self.psi)
        p = self.logical_to_padded(i)
        (self.grads if bufs is None else bufs)[self.w.inject_replica][p] = float("inf")
        return i

    # ---- backward-side reduction -------------------------------------------
    def backward(self, micro, bufs=None, stream=None):
        """Micro-batch `micro`'s share of the backward-side reduction: every
        bucket reduce-scattered into the fp32 gradient shards (accumulating
        after the first micro-batch), or, no_sync, every replica accumulated
        into its fp32 main_grad and the buckets reduced at the last one.
        Buckets go in plan order, which is the order backward fills them."""
        w, bufs = self.w, (self.grads if bufs is None else bufs)
        ng = len(self.plan.groups)
        if w.accum_mode == W.ACCUM_REDUCE_EACH:
            for g in range(ng):
                zf.bucket_reduce_scatter(self.plan, g, w.grad_dtype, bufs, self.grad_shards,
                                         micro > 0, stream=stream)
            return
        for q in range(w.n_ranks):
            zf.accumulate(w.grad_dtype, bufs[q], self.main_grads[q], n=self.psi_pad,
                          accumulate=micro > 0, stream=stream)
        if micro == w.n_micro - 1:
            for g in range(ng):
                zf.bucket_reduce_scatter(self.plan, g, zf.F32, self.main_grads,
                                         self.grad_shards, False, stream=stream)

    def backward_all(self, stream=None):
        """All micro-batches from the resident sets."""
        for a in range(self.w.n_micro):
            self.backward(a, self.micro_grads[a % len(self.micro_grads)], stream=stream)

    # ---- the step ------------------------------------------------------------
    def step(self, stream=None, phase_events=None):
        self.step_no += 1
        reduced = self.w.backward_rs
        if self.w.offload:
            self.last_result = zf.offload_step(
                self.plan, self.hp, self.w.grad_dtype, self.w.param_dtype,
                None if reduced else self.grads, self.grad_shards, self.params,
                self.workspace, self.state, self.h_state, self.h_grad, self.master,
                self.exp_avg, self.exp_avg_sq, self.h_params, stream=stream,
                grads_reduced=reduced, n_threads=self.n_threads, n_chunks=self.n_chunks,
                phase_events=phase_events, down16=self.w.offload_down16)
            return
        zf.shard_step(self.plan, self.hp, self.w.grad_dtype, self.w.param_dtype,
                      None if reduced else self.grads, self.master, self.exp_avg,
                      self.exp_avg_sq, self.params, self.workspace, self.state, stream=stream,
                      phase_events=phase_events, grad_shards=self.grad_shards,
                      grads_reduced=reduced)

    def result(self):
        return zf.read_result(self.state)

    # ---- resharding and checkpoints ------------------------------------------
    def replan(self, w_new):
        """A DeviceRun for workload w_new (same model, another layout or rank
        count) holding this run's state, re-laid out by logical index with
        zf_reshard; the state block (loss scale, t, beta powers) is copied."""
        assert not (self.w.offload or w_new.offload), "reshards device-resident state"
        new = DeviceRun(w_new, device=self.device)
        for name in ("master", "exp_avg", "exp_avg_sq"):
            zf.reshard(self.plan, new.plan, getattr(self, name), getattr(new, name))
        if self.params is not None and new.params is not None:
            zf.reshard(self.plan, new.plan, self.params, new.params)
        elif new.params is not None:  # fp32 parameters before: cast them
            new.params.copy_(new.master.to(new.params.dtype))
        new.state.copy_(self.state)
        new.step_no, new.loss_scale = self.step_no, self.loss_scale
        return new

    def checkpoint(self):
        """Host copies of everything a resumed run needs: the fp32 state, the
        16-bit parameters and the state block (no file format)."""
        keep = {n: getattr(self, n).detach().cpu().clone()
                for n in ("master", "exp_avg", "exp_avg_sq", "state")}
        if self.params is not None:
            keep["params"] = self.params.detach().cpu().clone()
        keep["step_no"], keep["loss_scale"] = self.step_no, self.loss_scale
        return keep

    def restore(self, ckpt):
        for n in ("master", "exp_avg", "exp_avg_sq", "state", "params"):
            if n in ckpt:
                getattr(self, n).copy_(ckpt[n])
        self.step_no, self.loss_scale = ckpt["step_no"], ckpt["loss_scale"]

    def unit_shards(self, u):
        """Rank r's 16-bit shard of unit u: params[O_u + r*S_u : +S_u]."""
        info = self.plan.units[u]
        base = self.params.data_ptr()
        return [base + 2 * (info.O + r * info.S) for r in range(self.w.n_ranks)]

    def gather(self, u, stream=None):
        zf.gather(self.plan, u, self.w.param_dtype, self.unit_shards(u), self.unit_buf,
                  stream=stream)
        return self.unit_buf[:self.plan.units[u].P]

    def gather_cast(self, g, stream=None):
        """FSDP2 unshard of group g: the group's parameters, unpadded, 16-bit."""
        zf.gather_cast(self.plan, g, self.w.param_dtype, self.master, self.group_buf,
                       stream=stream)
        return self.group_buf[:self.plan.groups[g].numel]

    def gather_all(self, stream=None):
        """Every unit's gather, in forward order (the per-unit stand-in for the
        next forward's all-gathers)."""
        if self.w.fp32_params:
            for g in range(len(self.plan.groups)):
                self.gather_cast(g, stream=stream)
        elif self.w.stage == 3:
            for u in range(len(self.plan.units)):
                self.gather(u, stream=stream)

    def run_workload_step(self):
        """One step of the workload's own sequence: fresh grads for step k at
        the current loss scale (every micro-batch, each reduced bucket by
        bucket as it is filled, when the workload accumulates), the
        injection if due, then the step."""
        k = self.step_no + 1
        if self.w.backward_rs:
            for a in range(self.w.n_micro):
                bufs = self.micro_grads[a % len(self.micro_grads)]
                self.fill_grads(k, self.loss_scale, micro=a, bufs=bufs)
                if self.w.inject_step == k and a == 0:
                    self.inject_inf(bufs)
                self.backward(a, bufs)
        else:
            self.fill_grads(k, self.loss_scale)
            if self.w.inject_step == k:
                self.inject_inf()
        self.step()
        res = self.result()
        self.loss_scale = res.scale_next
        return res
