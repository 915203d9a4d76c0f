/*
 * zf.h -- C ABI of the sharded mixed-precision AdamW step for MI355X (gfx950).
 *
 * The library emulates N data-parallel ranks on one GPU.  One zf_shard_step
 * call is one training step's optimizer side for all N ranks:
 *   1. reduce-scatter: the N replicas' 16-bit gradients are summed in binary32
 *      in the fixed order r = 0..N-1, each rank owning its shard of every
 *      FlatParameter unit;
 *   2. the loss scale is removed, a non-finite sum anywhere skips the step,
 *      and the gradient is clipped by its global L2 norm;
 *   3. AdamW updates every rank's fp32 master / exp_avg / exp_avg_sq shard;
 *   4. each shard is cast to fp16/bf16 and written into the full gathered
 *      parameter buffer (stages 0-2) or kept as the rank's resident shard
 *      (stage 3, gathered per unit by zf_gather before use).
 *
 * Pages the operations follow (cited by title and section):
 *   [L13] CMU 15-779 Lecture 13 notes, "Zero Redundancy and PyTorch FSDP":
 *         2.1 Adam, 2.2 fp32 master weights, 3.1-3.3 the three ZeRO stages,
 *         3.4 bit-exactness, 3.6 padding, 4.1 communication, 5.1 FSDP's
 *         per-unit all-gather, 5.2 FlatParameter (flatten, pad, split),
 *         5.6 gradient accumulation, 7.1-7.2 ZeRO-Offload and CPU-Adam.
 *   [F5]  Femtotron dev log #5 (Data Parallelism): resharding when the DP
 *         size changes.
 *   [F6]  Femtotron dev log #6 (ZeRO-1 and ZeRO-2): the sharding protocol
 *         make_master / reduce_grads / gather_weights / post_step, and the
 *         master as one 1-D vector.
 *   [F7]  Femtotron dev log #7 (ZeRO-3): the gradient hook pads with zeros
 *         and reduce-scatters with AVG into a shard of shard_size.
 *   [F9]  Femtotron dev log #9: ZeRO-3 unshard = all-gather of the flat shard
 *         into a padded_size full buffer.
 *   [MDT] Megatron / DeepSpeed / torchtitan architecture and source guide,
 *         ch. 四.3 (step: check fp16 overflow -> clip -> Adam per fp32
 *         partition -> copy to the 16-bit partition -> all-gather), 五.4 and
 *         五.6 (FSDP2: per-parameter dim-0 shards, the fp32 shard is the
 *         parameter, fp32 reduce-scatter into the shard's gradient, cast to
 *         the parameter dtype at all-gather time), 六.2 (Stage 3 vs FSDP1 vs
 *         FSDP2), 六.4 (checkpoint formats and resharding), 三.3 (Megatron's
 *         gradient buffer and buckets, no_sync
 *         accumulation in fp32) and 五.7 (global gradient-norm clipping;
 *         gradient accumulation on the shard).
 *
 * Conventions for every call:
 *   - Sizes are element counts unless a name ends in _bytes.
 *   - Device buffers are owned by the caller.  They must stay alive until
 *     the stream has passed the call; the library keeps no reference after
 *     returning and allocates no memory in zf_shard_step, zf_reduce_scatter,
 *     zf_gather or zf_state_init.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).
 *   - Every argument is validated before anything is enqueued: a call that
 *     returns an error leaves the stream untouched.  A launch failure is
 *     reported as ZF_EHIP (the stream may then hold part of the step).
 *   - An overflow (skipped step) is a result, not an error.
 *   - No call aborts or throws.
 *   - HIP graphs: zf_shard_step, zf_shard_step_noalloc (after its first
 *     call on the device), zf_reduce_scatter, zf_gather, zf_gather_cast,
 *     zf_bucket_reduce_scatter, zf_accumulate and
 *     zf_state_init enqueue kernels only (no memset, copy, allocation or
 *     synchronisation; every pointer travels by value in the kernel
 *     arguments), so a caller may capture them on a stream and replay the
 *     graph.  The state block carries t, the loss scale and the skip
 *     decision from one replay to the next.  The hyperparameters (and every
 *     pointer) are those of the capture, so a learning-rate schedule needs a
 *     new capture.  zf_read_result and zf_offload_step synchronise and
 *     cannot be captured.
 *
 * Device data layout (the padded flat index p):
 *   A plan's units are laid end to end, unit u at offset O_u with P_u =
 *   N*ceil(L_u/N) elements (its L_u real elements, then P_u - L_u zeros).
 *   Rank r owns, in unit u, the S_u = P_u/N elements [O_u + r*S_u, +S_u).
 *   EVERY per-element device array of the step -- each gradient replica,
 *   the fp32 master / exp_avg / exp_avg_sq, the 16-bit parameters and the
 *   fp32 reduce-scatter output -- holds Psi' = sum_u P_u elements indexed by
 *   p.  So rank r's fp32 shard of unit u is master[O_u + r*S_u .. +S_u): the
 *   N ranks' shards of a unit sit side by side, as one rank's shards of all
 *   units would in FSDP's per-unit FlatParameter shards.  Padding elements
 *   must be zero in the gradients and stay zero everywhere.
 *   Base pointers must be 16-byte aligned (torch allocations are 256-byte
 *   aligned).
 */
#ifndef ZF_H
#define ZF_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZF_MAX_RANKS 64

enum zf_status {
  ZF_OK = 0,
  ZF_EINVAL = -1,  /* bad argument: NULL pointer, bad count, bad plan, bad unit */
  ZF_EALIGN = -2,  /* a base pointer is not 16-byte aligned                    */
  ZF_EDTYPE = -3,  /* unknown dtype                                            */
  ZF_ESIZE = -4,   /* a size overflows or exceeds a limit                      */
  ZF_EHIP = -5,    /* the HIP runtime reported an error                        */
  ZF_ENOMEM = -6,  /* host allocation for a plan failed                        */
  ZF_EUNSUP = -7   /* the host CPU lacks an instruction set a call needs        */
};

/* ZF_F32 is accepted only where a call says so (the fp32 replicas of
 * zf_bucket_reduce_scatter). */
enum zf_dtype { ZF_F16 = 1, ZF_BF16 = 2, ZF_F32 = 3 };
/* Layouts:
 *   ZF_GLOBAL_FLAT    all parameters form one FlatParameter ([F6]);
 *   ZF_PER_UNIT       one FlatParameter per FSDP unit ([L13] 5.2, FSDP1);
 *   ZF_PER_PARAM_DIM0 FSDP2 ([MDT] 五.4): every parameter is cut along dim 0
 *                     into N chunks of ceil(R/N) rows (torch.chunk; short or
 *                     empty last chunks), each rank's chunk padded with zero
 *                     rows, so a parameter of R x C elements takes
 *                     P = N*ceil(R/N)*C elements in the padded flat; the FSDP
 *                     unit ids group parameters for zf_gather_cast. */
enum zf_layout { ZF_GLOBAL_FLAT = 0, ZF_PER_UNIT = 1, ZF_PER_PARAM_DIM0 = 2 };

/* One parameter tensor, in model order.  `unit` is its FSDP unit id (ids run
 * 0,0,..,1,1,..; ignored for ZF_GLOBAL_FLAT); `kind` is informational (0
 * weight, 1 bias, 2 norm weight); `dim0` is its number of rows, used by
 * ZF_PER_PARAM_DIM0 (<= 0: a 1-D tensor; must divide numel). */
typedef struct {
  int64_t numel;
  int32_t unit;
  int32_t kind;
  int64_t dim0;
} zf_segment;

typedef struct zf_plan zf_plan;  /* opaque, immutable once made */

typedef struct {
  int64_t psi;                 /* real parameters */
  int64_t psi_pad;             /* Psi' = sum_u P_u */
  int64_t n_units;
  int64_t max_unit_pad;        /* max_u P_u: elements of a ZeRO-3 unit buffer */
  int64_t n_groups;            /* FSDP units (== n_units except ZF_PER_PARAM_DIM0) */
  int64_t max_group_numel;     /* max unpadded elements of a group (zf_gather_cast) */
  int32_t n_ranks, layout, stage;
  int32_t policy;              /* where pass 2 finds the sums: 0 recomputed from
                                  the replicas, 1 the workspace's fp32 copy,
                                  2 the caller's fp32 gradient shard (FSDP2) */
  int64_t workspace_bytes;
  /* bytes of model state per rank once backward has finished ([L13] 2.3 and
   * 3.5): [0..3] stages 0..3 = 16*Psi, 4*Psi' + 12*Psi'/N, 2*Psi' + 14*Psi'/N,
   * 16*Psi'/N; [4] FSDP2 with fp32 parameters ([MDT] 五.6: fp32 shard +
   * fp32 grad shard + m + v) = 16*Psi'/N; and the stage-3 peak while
   * backward holds one unit's full params and grads ([L13] exercise 5). */
  int64_t state_bytes[5];
  int64_t stage3_peak_bytes;
  /* bytes one rank would send per step with ring collectives ([L13] 4.1,
   * 4.2): [0] DP all-reduce, [1] stage 1, [2] stage 2, [3] stage 3,
   * [4] the slides' stage 1 (all-reduce of grads + all-gather of params). */
  double comm_bytes[5];
  /* bytes of the materialised fp32 sums (policy 1 or 2) that pass 1 stores
   * with cache-allocating stores and the update pass reads first, from the
   * chip's memory-side cache (Infinity Cache): the last 256 MiB of the sums
   * when all of them take at most 448 MiB, else 0.  The step on already
   * reduced gradients (grads_reduced) and the offload step do not use it.
   * A performance detail only: no result depends on it. */
  int64_t cached_sums_bytes;
} zf_plan_summary;

typedef struct {
  int64_t L;    /* real elements */
  int64_t P;    /* padded elements, a multiple of N */
  int64_t S;    /* shard elements, P / N */
  int64_t O;    /* offset in the padded flat */
  int64_t lam;  /* offset of its first element in the unpadded model order */
} zf_unit_info;

/* Plan the FlatParameter layout ([L13] 5.2; [F6] for the global flat):
 * ZF_PER_UNIT flattens each unit's segments end to end and pads it to a
 * multiple of n_ranks; ZF_GLOBAL_FLAT treats the whole model as one unit.
 * n_ranks in [1, ZF_MAX_RANKS]; stage in [0, 3] selects the output of
 * zf_shard_step (0-2: full buffer; 3: resident shards) and the ledger row.
 * Host only; *out receives a plan to release with zf_plan_free.
 * Errors: ZF_EINVAL (NULL, nseg < 1, numel < 1, unit ids not 0,0,..,1,..),
 * ZF_ESIZE (n_ranks out of range, Psi' >= 2^62, or a step kernel's grid
 * above 2^31 - 1 blocks: Psi' above about 2^40), ZF_ENOMEM. */
int zf_plan_flat(const zf_segment* segs, int64_t nseg, int32_t n_ranks, int32_t layout,
                 int32_t stage, zf_plan** out);

/* Copy the plan's summary.  Errors: ZF_EINVAL. */
int zf_plan_info(const zf_plan* plan, zf_plan_summary* out);

/* Copy unit u's offsets and sizes.  Errors: ZF_EINVAL (u out of range).
 * Under ZF_PER_PARAM_DIM0 the units are the parameters. */
int zf_plan_unit(const zf_plan* plan, int64_t u, zf_unit_info* out);

typedef struct {
  int64_t first_unit;  /* its units are first_unit .. first_unit + n_units - 1 */
  int64_t n_units;
  int64_t numel;       /* unpadded elements: sum of the units' L */
  int64_t padded;      /* padded elements: sum of the units' P */
} zf_group_info;

/* Copy FSDP unit (group) g's extent.  Errors: ZF_EINVAL. */
int zf_plan_group(const zf_plan* plan, int64_t g, zf_group_info* out);

/* Release a plan (NULL is allowed).  Only after the stream has passed every
 * call that used it. */
void zf_plan_free(zf_plan* plan);

/* Device workspace one zf_shard_step needs: per-block partial sums of the
 * squared norm, plus, when 2N > 8, the fp32 reduce-scatter output (Psi' x
 * 4 bytes), which is cheaper than re-reading N replicas.  < 0 on error. */
int64_t zf_workspace_bytes(const zf_plan* plan);

/* Bytes of the device state block (loss scale, growth counter, Adam step
 * count, running beta powers, and the last step's result). */
int64_t zf_state_bytes(void);

/* Initialise a state block (device memory, zf_state_bytes() bytes, 16-byte
 * aligned): loss scale S > 0, dynamic scaling on/off (halve on overflow;
 * double after growth_interval applied steps in a row, never if <= 0),
 * t = 0; every byte of the block is written.  The block is plain data with
 * no pointers and does not depend on N or the layout: copying it to the
 * host and back (a checkpoint) or to another plan's run (zf_reshard)
 * resumes the step sequence exactly.  Enqueued on `stream`.  Errors:
 * ZF_EINVAL, ZF_EALIGN, ZF_EHIP. */
int zf_state_init(void* d_state, double loss_scale, int32_t dynamic, int32_t growth_interval,
                  void* stream);

/* AdamW's hyperparameters as doubles; every binary32 constant of the
 * update is rounded once from them.  beta1 and beta2 must lie in [0, 1)
 * (ZF_EINVAL otherwise); lr, eps and weight_decay are used as given.  With
 * eps = 0 an element whose updated exp_avg and exp_avg_sq are both zero (the
 * zero padding, or a zero gradient on zero state) becomes NaN, as the
 * formula says (0/0): pass eps > 0 to keep the padding zero. */
typedef struct {
  double lr, beta1, beta2, eps, weight_decay;
  double max_norm;  /* global L2 clip threshold; <= 0 disables clipping */
} zf_hparams;

typedef struct {
  int32_t grad_dtype;         /* ZF_F16 or ZF_BF16 */
  int32_t param_dtype;        /* ZF_F16 or ZF_BF16 */
  const void* const* grads;   /* host array of N device pointers: replica q's
                                 padded-flat gradient, Psi' 16-bit values, loss-
                                 scaled by the state's current S */
  float* master;              /* Psi' fp32, padded-flat order, updated in place */
  float* exp_avg;             /* Psi' fp32 */
  float* exp_avg_sq;          /* Psi' fp32 */
  void* params;               /* Psi' 16-bit: stages 0-2 the gathered full
                                 buffer; stage 3 the N resident shards; or
                                 NULL: no 16-bit copy (fp32 parameters, as
                                 FSDP2 keeps them) */
  float* grad_shards;         /* NULL, or Psi' fp32: the ranks' resident fp32
                                 gradient shards; pass 1 writes the sums
                                 there and pass 2 reads them (required by
                                 ZF_PER_PARAM_DIM0 plans and by
                                 grads_reduced) */
  int32_t grads_reduced;      /* 0: reduce-scatter `grads` in pass 1.
                                 1: grad_shards already hold the reduced
                                 (and accumulated) gradients, as left by
                                 zf_bucket_reduce_scatter; `grads` and
                                 grad_dtype are ignored (grads may be NULL)
                                 and pass 1 only reads grad_shards for the
                                 overflow flag and the norm partials */
  int32_t reserved;           /* must be 0 */
  int64_t numel;              /* elements of each per-element array above
                                 (grads[q], master, exp_avg, exp_avg_sq,
                                 params, grad_shards); must be >= Psi' */
  void* workspace;            /* device workspace (may be NULL only if
                                 zf_workspace_bytes(plan) is 0) */
  int64_t workspace_size;     /* its size in bytes; must be >=
                                 zf_workspace_bytes(plan) */
  void* state;                /* a state block set up by zf_state_init */
  void* const* phase_events;  /* NULL, or 4 hipEvent_t recorded on `stream`:
                                 before pass 1, after pass 1, after the norm
                                 reduction and finish, after the update pass */
} zf_step_args;

/* One emulated step for all N ranks ([L13] 3.1 steps 3-6, 3.2, 3.3; [F6]
 * reduce_grads + step + gather_weights; [MDT] 四.3 order).  Enqueues four
 * kernels on `stream` (three when the partials fit one reduce block: reduce
 * and finish are then one launch, with the same bits) and returns without
 * synchronising:
 *   pass 1  reduce-scatter sums, overflow flag, per-tile squared-norm
 *           partials (fp64), and the fp32 sums when the plan materialises;
 *   reduce  fixed contiguous ranges of the partials, in order;
 *   finish  one block: fixed-order total, skip decision, clip coefficient,
 *           bias corrections, next loss scale -> state block;
 *   pass 2  unless skipped: g = sum * f32(coef/(S*N)); AdamW; RNE cast to
 *           param_dtype into params[p].
 * The skip decision and clip coefficient stay on the device.
 * Errors: ZF_EINVAL, ZF_EALIGN, ZF_EDTYPE, ZF_ESIZE (numel < Psi' or
 * workspace_size < zf_workspace_bytes(plan)), ZF_EHIP. */
int zf_shard_step(const zf_plan* plan, const zf_hparams* hp, const zf_step_args* args,
                  void* stream);

/* Bytes of the library's static device scratch array (64 MiB), the
 * workspace of zf_shard_step_noalloc. */
#define ZF_NOALLOC_SCRATCH_BYTES (64ll << 20)

/* zf_shard_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same kernels on the same grids, so the same results bit
 * for bit, but the workspace is the library's static device array of
 * ZF_NOALLOC_SCRATCH_BYTES instead of a caller buffer.  The caller still
 * passes every input and output; args->workspace must be NULL and
 * args->workspace_size 0.  The call allocates nothing (no hipMalloc, no
 * host allocation): the array is part of the library's code object, held
 * on every GPU that runs the library from its load until the process ends,
 * each GPU its own copy.  The first call on a device looks up the array's
 * address there (a query, not an allocation); a caller that captures the
 * call in a graph makes one call on that device before capturing.
 * Scratch needed: zf_workspace_bytes(plan), less the fp32 sums' share
 * (Psi' * 4 bytes rounded up to 256) when the plan materialises the sums
 * (zf_plan_summary.policy 1) and args->grad_shards is given, since pass 1
 * then writes the sums there; a plan that needs more than
 * ZF_NOALLOC_SCRATCH_BYTES (policy 1 without grad_shards above about 16.7M
 * elements, or any plan above about 8.5e9 elements) gets ZF_ESIZE before
 * anything is enqueued.  Every scratch byte a call reads it first writes
 * in the same call, so nothing needs clearing, but every call on one GPU
 * shares that GPU's one array: calls that overlap on a GPU (two streams,
 * two threads) race and must be serialised by the caller.  Errors: as
 * zf_shard_step, plus ZF_EINVAL (workspace given; a device ordinal >= 64)
 * and ZF_ESIZE (scratch too small). */
int zf_shard_step_noalloc(const zf_plan* plan, const zf_hparams* hp, const zf_step_args* args,
                          void* stream);

/* The reduce-scatter alone ([L13] 3.2; [F7] gradient hook): rs_out[p] is
 * the fixed-order binary32 sum of the N replicas at p, for every p < Psi'
 * (each rank's shard in its padded-flat place).  numel: elements of every
 * grads[q] and of rs_out, >= Psi'.  Errors as zf_shard_step. */
int zf_reduce_scatter(const zf_plan* plan, int32_t grad_dtype, const void* const* grads,
                      float* rs_out, int64_t numel, void* stream);

/* Megatron gradient buckets ([MDT] 三.3): assign a bucket id to every
 * parameter, in buffer order.  Megatron lays the buffer out last layer
 * first, so that gradients fill it from the head as backward runs; callers
 * that follow it pass the segments in that order.  A bucket closes as soon
 * as it holds at least bucket_numel elements; a parameter is never split;
 * the last bucket takes the rest.  bucket_numel <= 0 selects the default
 * max(40,000,000, 1,000,000 * n_ranks).  unit_out[s] receives segment s's
 * bucket id (0, 0, .., 1, ..), usable as zf_segment.unit with ZF_PER_UNIT:
 * each bucket is then a FlatParameter padded to a multiple of n_ranks and
 * split evenly, as the distributed optimizer pads its buckets.  Host only.
 * Errors: ZF_EINVAL (NULL, nseg < 1, numel < 1), ZF_ESIZE (n_ranks out of
 * range). */
int zf_plan_buckets(const int64_t* numel, int64_t nseg, int32_t n_ranks, int64_t bucket_numel,
                    int32_t* unit_out, int64_t* n_buckets);

/* Backward-side reduce-scatter of one bucket as its gradients become ready
 * ([L13] 3.2: one reduce-scatter per bucket during backward; [MDT] 三.3 and
 * 四.3), accumulating over micro-batches ([L13] 5.6 and [MDT] 五.7: each
 * micro-batch reduce-scattered and added to the sharded gradient).  For
 * every p in group g's padded range [O, O + padded) -- a bucket or unit of a
 * ZF_PER_UNIT plan, the whole flat of a ZF_GLOBAL_FLAT plan, an FSDP unit
 * of a ZF_PER_PARAM_DIM0 plan:
 *   sum = f32(grads[0][p]) + f32(grads[1][p]) + ... + f32(grads[N-1][p])
 *   grad_shards[p] = accumulate ? grad_shards[p] + sum : sum
 * each + one binary32 addition, in rank order.  grad_dtype: ZF_F16 or
 * ZF_BF16 replicas, or ZF_F32 for fp32 replicas (the no_sync scheme: every
 * replica accumulates locally with zf_accumulate and is reduced once, at
 * the last micro-batch).  grads: host array of N device pointers to padded-
 * flat replicas, 16-byte aligned, of numel elements (only the group's range
 * is read); grad_shards: numel fp32, 16-byte aligned; numel >= Psi'.
 * Distinct groups touch disjoint ranges: they may run in any order or on
 * different streams.  A zf_shard_step with grads_reduced = 1 then consumes
 * grad_shards.  Errors: ZF_EINVAL, ZF_EALIGN, ZF_EDTYPE, ZF_ESIZE,
 * ZF_EHIP. */
int zf_bucket_reduce_scatter(const zf_plan* plan, int64_t group, int32_t grad_dtype,
                             const void* const* grads, float* grad_shards, int64_t numel,
                             int32_t accumulate, void* stream);

/* Local gradient accumulation under no_sync ([MDT] 三.3: the backward hook
 * adds each micro-batch's gradient into the parameter's fp32 main_grad and
 * nothing is communicated until the last micro-batch):
 *   acc[i] = accumulate ? acc[i] + f32(grad[i]) : f32(grad[i]),  i < n.
 * grad: n ZF_F16 / ZF_BF16 values (2-byte aligned); acc: n fp32 (4-byte
 * aligned); any offsets, e.g. one bucket's range of a replica.  n >= 0.
 * Errors: ZF_EINVAL, ZF_EALIGN, ZF_EDTYPE, ZF_EHIP. */
int zf_accumulate(int32_t grad_dtype, const void* grad, float* acc, int64_t n, int32_t accumulate,
                  void* stream);

/* FSDP2 unshard of group g ([MDT] 五.4: each rank's fp32 shards are cast to
 * the parameter dtype, all-gathered and copied out into the full
 * parameters): out holds the group's parameters end to end, unpadded, in
 * model order; element e of parameter u is RNE16(master[O_u + e]) -- rank
 * e / S_u's shard, offset e % S_u.  master: the padded-flat fp32 array of
 * zf_shard_step (master_numel >= Psi', 16-byte aligned); out: out_numel >=
 * the group's numel, 2-byte aligned.  Errors: ZF_EINVAL, ZF_EALIGN,
 * ZF_EDTYPE, ZF_ESIZE, ZF_EHIP. */
int zf_gather_cast(const zf_plan* plan, int64_t group, int32_t dtype, const float* master,
                   int64_t master_numel, void* out, int64_t out_numel, void* stream);

/* ZeRO-3 / FSDP unit gather ([L13] 3.3 and 5.1; [F9] unshard):
 * unit_buf[r*S_u + j] = shards[r][j] for every rank r < N and j < S_u, i.e.
 * the N ranks' 16-bit shards of unit u concatenated in rank order into the
 * unit's padded FlatParameter (P_u elements; the caller reuses one buffer of
 * max_unit_pad elements for every unit).  `shards` is a host array of N
 * device pointers (any 2-byte alignment; with stage-3 zf_shard_step output
 * they are params + O_u + r*S_u), each of S_u elements.  unit_buf_numel:
 * elements of unit_buf, >= P_u.  Errors: ZF_EINVAL, ZF_EALIGN, ZF_EDTYPE,
 * ZF_ESIZE, ZF_EHIP. */
int zf_gather(const zf_plan* plan, int64_t unit, int32_t dtype, const void* const* shards,
              void* unit_buf, int64_t unit_buf_numel, void* stream);

typedef struct {
  int32_t overflow;     /* a reduced gradient was inf or NaN */
  int32_t skipped;      /* the update was skipped (== overflow) */
  int64_t t;            /* applied Adam steps so far */
  double sumsq;         /* sum of squared reduced (still scaled) gradients */
  double norm;          /* sqrt(sumsq) / (S*N): the clipped-against norm */
  double coef;          /* min(1, max_norm / (norm + 1e-6)), 1 if disabled */
  double scale_used;    /* loss scale of this step's gradients */
  double scale_next;    /* loss scale for the next step */
  float gs;             /* binary32 factor applied to the sums */
  int32_t growth_ctr;
  float bc1, bc2;       /* binary32 bias corrections 1 - beta^t of the update */
} zf_step_result;

/* Resharding ([F5]: a checkpoint saved at one DP size loaded at another
 * needs the state redistributed; [MDT] 六.4: universal checkpoints, DCP):
 * re-lay one per-element array from plan `from` to plan `to` by logical
 * index.  Every real element moves from its padded-flat place under `from`
 * to its place under `to`; every padding element of `dst` becomes zero.
 * The plans may differ in layout and rank count but must describe the same
 * model (the same segments in the same order; Psi is checked).  Rank r's
 * real part of unit u is the logical run [lam_u + r*S_u, +clamp(L_u -
 * r*S_u, 0, S_u)) in every layout.  src / dst: device arrays of src_numel
 * >= Psi'(from) and dst_numel >= Psi'(to) elements of elem_bytes (2: 16-bit
 * parameters, 4: fp32 master / moments), aligned to elem_bytes, not
 * overlapping.  The device state block needs no change (it does not depend
 * on N).  Errors: ZF_EINVAL, ZF_EALIGN, ZF_ESIZE, ZF_ENOMEM, ZF_EHIP. */
int zf_reshard(const zf_plan* from, const zf_plan* to, const void* src, int64_t src_numel,
               void* dst, int64_t dst_numel, int32_t elem_bytes, void* stream);

/* Name of the HIP runtime error behind the calling thread's last ZF_EHIP
 * ("hipSuccess" if there was none).  The string is static. */
const char* zf_hip_error_name(void);

/* Copy the last step's result from a device state block to the host.
 * Synchronises `stream`.  Errors: ZF_EINVAL, ZF_EHIP. */
int zf_read_result(const void* d_state, zf_step_result* out, void* stream);

/* ---- ZeRO-Offload ([L13] 7.1-7.2) --------------------------------------
 * The offload partition keeps the 16-bit parameters (and forward/backward)
 * on the GPU; the fp32 master, exp_avg, exp_avg_sq and the Adam update live
 * on the CPU.  Gradients go down PCIe, updated 16-bit parameters come back
 * up in chunks that overlap the CPU update of the next chunk. */

typedef struct {
  int64_t n;                /* elements */
  const void* grad;         /* n reduced gradient sums, still loss-scaled, of
                               grad_dtype */
  float* master;            /* n fp32, updated in place */
  float* exp_avg;           /* n fp32 */
  float* exp_avg_sq;        /* n fp32 */
  void* params;             /* NULL, or n 16-bit outputs RNE16(master) */
  int32_t param_dtype;      /* ZF_F16 or ZF_BF16 (when params is given) */
  int32_t n_threads;        /* worker threads; <= 0: every hardware thread */
  float gs, bc1, bc2;       /* the step's scalars, from zf_step_result */
  int32_t grad_dtype;       /* 0 or ZF_F32: binary32 sums (4-byte aligned);
                               ZF_F16 / ZF_BF16: 16-bit sums (2-byte aligned),
                               widened exactly */
} zf_cpu_adam_args;

/* CPU-Adam ([L13] 7.2: a SIMD, multithreaded Adam on the CPU): the same
 * element update as zf_shard_step's update pass, in the same binary32
 * operations and order (so given the same gs, bc1, bc2 it gives the same
 * bits), on host memory, split over n_threads threads in contiguous ranges
 * of 8-lane AVX2 vectors; the 16-bit outputs are rounded to nearest-even
 * (F16C for fp16, integer rounding for bf16).  The caller skips the call
 * for a skipped step.  Host pointers: 4-byte aligned (params 2-byte).  Runs
 * on the calling thread plus n_threads - 1 workers and returns when done.
 * Errors: ZF_EINVAL, ZF_EALIGN, ZF_EDTYPE, ZF_EUNSUP (the CPU lacks AVX2 or
 * F16C). */
int zf_cpu_adam(const zf_hparams* hp, const zf_cpu_adam_args* args);

typedef struct {
  int32_t grad_dtype;         /* as zf_step_args */
  int32_t param_dtype;        /* dtype of the device 16-bit parameters */
  const void* const* grads;   /* as zf_step_args (ignored with grads_reduced) */
  float* grad_shards;         /* device Psi' fp32: pass 1 leaves the sums here
                                 (or they are already reduced) */
  void* params;               /* device Psi' 16-bit parameters: the upload's
                                 destination (padded-flat, as zf_shard_step) */
  int64_t numel;              /* elements of every per-element array, >= Psi' */
  void* workspace;            /* device workspace, zf_workspace_bytes(plan) */
  int64_t workspace_size;
  void* state;                /* device state block */
  void* h_state;              /* pinned host, zf_state_bytes() */
  float* h_grad;              /* pinned host Psi' fp32: the sums come down here */
  float* h_master;            /* host Psi' fp32 state, padded-flat order */
  float* h_exp_avg;
  float* h_exp_avg_sq;
  void* h_params;             /* pinned host Psi' 16-bit staging of the upload */
  int32_t grads_reduced;      /* as zf_step_args */
  int32_t n_threads;          /* CPU-Adam threads (<= 0: every hardware thread) */
  int32_t n_chunks;           /* pipeline chunks, 1 .. 4096 */
  int32_t down16;             /* 0: the fp32 sums go down (4 B per element;
                                 the result equals zf_shard_step's bit for
                                 bit).  1: the sums are rounded to the
                                 gradient dtype on the GPU and go down in 16
                                 bits (2 B per element, the pages' fp16
                                 gradient edge); the overflow check and the
                                 norm are taken on the rounded values, as
                                 the host would see them.  1 needs
                                 grads_reduced = 0. */
  void* const* phase_events;  /* NULL, or 4 hipEvent_t recorded on `stream`:
                                 before pass 1, after the finish kernel, after
                                 the last download, after the last upload */
} zf_offload_args;

/* One ZeRO-Offload step for all N ranks ([L13] 7.1: only the fp16
 * parameters stay on the GPU; 7.2: gradients down, CPU-Adam, 16-bit
 * parameters back up in chunks pipelined with the CPU update):
 *   GPU   pass 1 (reduce-scatter sums into grad_shards, overflow, norm
 *         partials), norm reduction, finish -- as zf_shard_step;
 *   PCIe  the state block and the sums, chunk by chunk, into h_state and
 *         h_grad;
 *   CPU   unless the step is skipped, zf_cpu_adam chunk by chunk on
 *         h_master / h_exp_avg / h_exp_avg_sq, writing RNE16 into h_params;
 *   PCIe  each chunk of h_params into params as soon as it is ready.
 * The uploads run on a library-owned stream per device (created on first
 * use, kept until the process ends), so both PCIe directions are busy at
 * once.  Blocks until the step is complete and fills *result (may be
 * NULL).  With down16 = 0 the state and parameters equal zf_shard_step's
 * bit for bit; with down16 = 1 they follow the 16-bit gradients.
 * Calls that overlap on one device must not share host buffers.  Errors:
 * ZF_EINVAL, ZF_EALIGN, ZF_EDTYPE, ZF_ESIZE, ZF_EHIP, ZF_EUNSUP. */
int zf_offload_step(const zf_plan* plan, const zf_hparams* hp, const zf_offload_args* args,
                    void* stream, zf_step_result* result);

/* Text for a status code (static storage). */
const char* zf_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif /* ZF_H */
