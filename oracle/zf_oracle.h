/*
 * zf_oracle.h -- CPU oracle for the sharded mixed-precision AdamW step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this code; only the test suite, the package smoke check and
 * the bench's CPU-baseline leg do.  It shares no source, header, table or
 * helper with the HIP library.
 *
 * Plain, slow, single-threaded C99, built with -O2 -ffp-contract=off and no
 * fast-math, so every float expression below is one IEEE binary32 operation
 * rounded to nearest-even (x86-64 SSE scalar arithmetic).
 *
 * Sources (the pages are cited by title and section):
 *  [L13]  CMU 15-779 Lecture 13 notes, "Zero Redundancy and PyTorch FSDP":
 *         2.1 (Adam), 2.2 (fp32 master weights), 2.3 (bytes per parameter),
 *         2.4-2.5 (ZeRO tables 1 and 2), 3.1-3.3 (the three stages),
 *         3.4 (bit-exactness conditions), 3.5 (memory), 3.6 (padding),
 *         4.1-4.2 (communication volume), 5.2 (FlatParameter), 5.6 (the two
 *         gradient-accumulation schemes), exercises 1-5.
 *  [F5]   Femtotron dev log #5 (Data Parallelism): gradient accumulation with
 *         no_sync, resharding when the DP size changes.
 *  [F6]   Femtotron dev log #6 (ZeRO-1 and ZeRO-2): the master as one 1-D vector.
 *  [F7]   Femtotron dev log #7 (ZeRO-3): the ZeRO-2 gradient hook (pad, then
 *         reduce-scatter with AVG), ZeRO-3 is not bit-exact (reduction tree).
 *  [F9]   Femtotron dev log #9: ZeRO-3 unshard into a padded full buffer.
 *  [MDT]  Megatron / DeepSpeed / torchtitan architecture and source guide,
 *         ch. 四.3 (DeepSpeed stage 1/2 flat partitions; "check overflow ->
 *         clip -> step"), 五.4 and 五.6 (FSDP2: per-parameter dim-0 shards,
 *         fp32 shard is the parameter, cast at all-gather time, fp32
 *         reduce-scatter), 六.2 (Stage 3 vs FSDP1 vs FSDP2), 三.3 (Megatron
 *         gradient buckets, fp32 gradient accumulation) and 五.7
 *         (gradient-norm clipping and accumulation on the shard), 六.4
 *         (checkpoint formats and resharding).
 *
 * Where the pages leave a step open, the reading taken is stated at the
 * function that takes it.  Parity status: every function is pinned by a
 * CPU test (tests/test_oracle_pins.py) except where marked otherwise.
 */
#ifndef ZF_ORACLE_H
#define ZF_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { OR_F16 = 1, OR_BF16 = 2, OR_F32 = 3 };
enum { OR_GLOBAL_FLAT = 0, OR_PER_UNIT = 1 };

/* One FlatParameter unit ([L13] 5.2).  All counts are elements. */
typedef struct {
  int64_t L;    /* real (unpadded) length                          */
  int64_t P;    /* padded length, N * ceil(L / N)                  */
  int64_t S;    /* shard length, P / N                             */
  int64_t O;    /* offset of the unit in the padded flat            */
  int64_t lam;  /* offset of the unit's first element, unpadded     */
  int64_t M;    /* offset of this unit's shard inside a rank buffer */
} or_unit;

typedef struct { double lr, beta1, beta2, eps, weight_decay, max_norm; } or_hparams;

/* Loss-scale and Adam-step bookkeeping carried from step to step. */
typedef struct {
  double loss_scale;        /* S */
  int64_t t;                /* applied Adam steps */
  int32_t growth_ctr;       /* k */
  int32_t growth_interval;  /* K */
  int32_t dynamic;          /* 1: halve on overflow, double after K clean steps */
  int32_t pad_;
} or_scale_state;

/* fp32 scalars of one applied step (every one rounded once from double). */
typedef struct {
  float gs, dec, b1, c1, b2, c2, bc1, bc2, lrf, ef;
} or_scalars;

typedef struct {
  int32_t overflow, skipped;
  double sumsq, norm, coef, scale_used, scale_next;
  int64_t t;
  float gs;
  int32_t pad_;
} or_result;

/* ---- casts ------------------------------------------------------------- */
float    or_f16_to_f32(uint16_t h);
float    or_bf16_to_f32(uint16_t h);
uint16_t or_f32_to_f16(float f);
uint16_t or_f32_to_bf16(float f);
void     or_cast_array(int32_t dtype, int64_t n, const float* src, uint16_t* dst);
void     or_widen_array(int32_t dtype, int64_t n, const uint16_t* src, float* dst);

/* ---- seeded input generator (splitmix64 + Irwin-Hall-12) --------------- */
uint64_t or_splitmix64_next(uint64_t* state);
uint64_t or_stream_state(uint64_t seed, uint64_t stream);
float    or_normal_z(uint64_t stream_state, int64_t logical_index);
void     or_gen16(uint16_t* dst, int64_t n, int32_t dtype, uint64_t seed, uint64_t stream,
                  int64_t logical_base, double sigma, double scale);
void     or_gen32(float* dst, int64_t n, uint64_t seed, uint64_t stream, int64_t logical_base,
                  double sigma);

/* ---- layout planner and ledger ----------------------------------------- */
int or_layout(const int64_t* seg_numel, const int32_t* seg_unit, int64_t nseg, int32_t n_ranks,
              int32_t layout, or_unit* units_out, int64_t max_units, int64_t* n_units_out,
              int64_t* psi_out, int64_t* psi_pad_out);
int or_ledger(const or_unit* units, int64_t n_units, int32_t n_ranks, int32_t stage,
              int64_t* after_backward_bytes, int64_t* peak_bytes);
/* FSDP2 per-parameter dim-0 sharding: one unit per parameter, padded to a
 * multiple of N rows (rows[s] <= 0 means a 1-D parameter). */
int or_layout_dim0(const int64_t* seg_numel, const int64_t* seg_rows, int64_t nseg,
                   int32_t n_ranks, or_unit* units_out, int64_t max_units, int64_t* n_units_out,
                   int64_t* psi_out, int64_t* psi_pad_out);
double or_comm_bytes(int64_t psi_pad, int32_t n_ranks, int32_t variant);

/* ---- the step ------------------------------------------------------------ */
int or_reduce_scatter(int32_t grad_dtype, int32_t n_ranks, const or_unit* units, int64_t n_units,
                      const uint16_t* const* grads, float* const* rs_out);
int or_finish(double sumsq, int32_t overflow, int32_t n_ranks, const or_hparams* hp,
              or_scale_state* st, or_scalars* sc, or_result* res);
void or_adamw_array(int64_t n, const float* acc, const or_scalars* sc, float* p, float* m, float* v);
int or_step_reduced(int32_t param_dtype, int32_t n_ranks, const or_unit* units, int64_t n_units,
                    int32_t stage, float* const* acc, float* const* master,
                    float* const* exp_avg, float* const* exp_avg_sq, uint16_t* params_full,
                    uint16_t* const* param_shards, const or_hparams* hp, or_scale_state* st,
                    or_result* res);
int or_rs_accumulate(int32_t grad_dtype, int32_t n_ranks, const or_unit* units, int64_t n_units,
                     int64_t u, const void* const* grads, float* const* shards,
                     int32_t accumulate);
int or_local_accumulate(int32_t grad_dtype, int64_t n, const uint16_t* grad, float* acc,
                        int32_t accumulate);
int or_bucket_assign(const int64_t* seg_numel, int64_t nseg, int32_t n_ranks,
                     int64_t bucket_numel, int32_t* unit_out, int64_t* n_buckets);
int or_zero_step(int32_t grad_dtype, int32_t param_dtype, int32_t n_ranks, const or_unit* units,
                 int64_t n_units, int32_t stage, const uint16_t* const* grads,
                 float* const* master, float* const* exp_avg, float* const* exp_avg_sq,
                 uint16_t* params_full, uint16_t* const* param_shards, const or_hparams* hp,
                 or_scale_state* st, or_result* res);
int or_gather_unit(const or_unit* units, int64_t n_units, int32_t n_ranks, int64_t u,
                   const uint16_t* const* param_shards, uint16_t* unit_buf);
int or_fsdp2_step(int32_t grad_dtype, int32_t n_ranks, const or_unit* units, int64_t n_units,
                  const uint16_t* const* grads, float* const* master, float* const* exp_avg,
                  float* const* exp_avg_sq, float* const* grad_shards, const or_hparams* hp,
                  or_scale_state* st, or_result* res);
int or_fsdp2_gather(const or_unit* units, int64_t n_units, int32_t n_ranks, int64_t first,
                    int64_t count, int32_t dtype, const float* const* master, uint16_t* out);
int or_reshard(const or_unit* ua, int64_t nua, int32_t na, const void* const* a,
               const or_unit* ub, int64_t nub, int32_t nb, void* const* b, int32_t elem_bytes);
int or_dp_step(int32_t grad_dtype, int32_t param_dtype, int32_t n_ranks, int64_t psi,
               const uint16_t* const* grads, float* master, float* exp_avg, float* exp_avg_sq,
               uint16_t* params, const or_hparams* hp, or_scale_state* st, or_result* res);

/* ---- full-size checks by regeneration ---------------------------------- */
typedef struct { int64_t step, replica, index; uint16_t bits; uint16_t pad_[3]; } or_inject;
int or_regen_sumsq(int32_t grad_dtype, int32_t n_ranks, uint64_t seed, int64_t step, double sigma,
                   double scale, int64_t i0, int64_t i1, const or_inject* inj, double* sumsq,
                   int32_t* nonfinite);
int or_regen_acc(int32_t grad_dtype, int32_t n_ranks, uint64_t seed, int64_t step, double sigma,
                 double scale, int64_t n, const int64_t* logical_idx, const or_inject* inj,
                 float* acc_out);
/* With gradient accumulation over n_micro micro-batches (mode 0: reduce
 * every micro-batch and add to the shard; mode 1: no_sync, fp32 local
 * accumulation then one reduction). */
int or_regen_accum_sumsq(int32_t grad_dtype, int32_t n_ranks, int32_t n_micro, int32_t mode,
                         uint64_t seed, int64_t step, double sigma, double scale, int64_t i0,
                         int64_t i1, const or_inject* inj, double* sumsq, int32_t* nonfinite);
int or_regen_accum_acc(int32_t grad_dtype, int32_t n_ranks, int32_t n_micro, int32_t mode,
                       uint64_t seed, int64_t step, double sigma, double scale, int64_t n,
                       const int64_t* logical_idx, const or_inject* inj, float* acc_out);
/* Steps 2-3 of the step on n given reduced values in their order: the
 * squared norm sum of (double)x^2 and the overflow flag (any non-finite). */
int or_sumsq_array(int64_t n, const float* x, double* sumsq, int32_t* nonfinite);

#ifdef __cplusplus
}
#endif
#endif
