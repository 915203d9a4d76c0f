/*
 * zf_oracle.c -- CPU oracle for the sharded mixed-precision AdamW step.
 *
 * TEST INFRASTRUCTURE ONLY: see zf_oracle.h.  The product path never loads it.
 *
 * Every float expression is written as the binary32 operation sequence it
 * defines; with -ffp-contract=off and SSE scalar arithmetic each operator
 * rounds once, to nearest-even.  Double is used only where the reading of the
 * pages says so (the squared-norm accumulation and the per-step scalars).
 */
#include "zf_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Casts between binary32 and the two 16-bit formats.  IEEE round-to-nearest-
 * even, written with integer arithmetic so that no library conversion is
 * involved.  NaN maps to a quiet NaN of the same sign (never reached by an
 * applied step: a non-finite gradient skips the step).                      */

static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

float or_bf16_to_f32(uint16_t h) { return u2f((uint32_t)h << 16); }

float or_f16_to_f32(uint16_t h) {
  uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
  uint32_t e = (h >> 10) & 0x1Fu;
  uint32_t f = h & 0x3FFu;
  if (e == 0x1F) return u2f(sign | 0x7F800000u | (f << 13));          /* inf / NaN */
  if (e != 0) return u2f(sign | ((e - 15 + 127) << 23) | (f << 13));   /* normal */
  /* zero or subnormal: value = f * 2^-24, exact in binary32 */
  {
    float mag = (float)f * 5.9604644775390625e-8f;
    return (sign != 0u) ? -mag : mag;
  }
}

uint16_t or_f32_to_bf16(float x) {
  uint32_t u = f2u(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
  /* add just under half an ulp, plus one if the kept lsb is odd (ties to even) */
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

uint16_t or_f32_to_f16(float x) {
  uint32_t u = f2u(x);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  uint32_t a = u & 0x7FFFFFFFu;
  int32_t e;
  uint32_t mant, q, rem, halfway;
  int shift;
  if (a > 0x7F800000u) return (uint16_t)(sign | 0x7E00u);   /* NaN */
  if (a >= 0x47800000u) return (uint16_t)(sign | 0x7C00u);  /* |x| >= 2^16, or inf */
  if (a < 0x00800000u) return sign;                          /* binary32 zero/subnormal */
  e = (int32_t)(a >> 23) - 127;
  mant = (a & 0x7FFFFFu) | 0x800000u;                        /* 24-bit significand */
  if (e >= -14) {
    /* normal binary16: keep 11 significant bits */
    q = mant >> 13;
    rem = mant & 0x1FFFu;
    if (rem > 0x1000u || (rem == 0x1000u && (q & 1u))) q += 1u;
    /* q in [0x400, 0x800]; a carry to 0x800 bumps the exponent, up to inf */
    return (uint16_t)(sign | (uint16_t)((uint32_t)(e + 14) * 1024u + q));
  }
  /* subnormal binary16: units of 2^-24; value / 2^-24 = mant * 2^(e+1) */
  shift = -(e + 1);
  if (shift > 25) return sign;
  q = mant >> shift;
  rem = mant & ((1u << shift) - 1u);
  halfway = 1u << (shift - 1);
  if (rem > halfway || (rem == halfway && (q & 1u))) q += 1u;
  return (uint16_t)(sign | q);
}

void or_cast_array(int32_t dtype, int64_t n, const float* src, uint16_t* dst) {
  int64_t i;
  for (i = 0; i < n; ++i)
    dst[i] = (dtype == OR_BF16) ? or_f32_to_bf16(src[i]) : or_f32_to_f16(src[i]);
}

void or_widen_array(int32_t dtype, int64_t n, const uint16_t* src, float* dst) {
  int64_t i;
  for (i = 0; i < n; ++i)
    dst[i] = (dtype == OR_BF16) ? or_bf16_to_f32(src[i]) : or_f16_to_f32(src[i]);
}

static float widen(int32_t dtype, uint16_t h) {
  return (dtype == OR_BF16) ? or_bf16_to_f32(h) : or_f16_to_f32(h);
}
static uint16_t narrow(int32_t dtype, float f) {
  return (dtype == OR_BF16) ? or_f32_to_bf16(f) : or_f32_to_f16(f);
}

/* ------------------------------------------------------------------------ */
/* Seeded inputs.  splitmix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014) used as a counter-based
 * generator: output j of a generator whose state starts at s is
 * mix(s + (j+1)*gamma).  A stream's starting state is output number `stream`
 * of the generator seeded with `seed`.  Element i of a stream consumes outputs
 * 3i, 3i+1, 3i+2: twelve 16-bit words k, and z = (sum k - 393210) / 65536 is
 * an Irwin-Hall(12) approximation of N(0,1), exact in binary32.            */

#define OR_GAMMA 0x9E3779B97F4A7C15ull

static uint64_t or_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t or_splitmix64_next(uint64_t* state) {
  *state += OR_GAMMA;
  return or_mix64(*state);
}

uint64_t or_stream_state(uint64_t seed, uint64_t stream) {
  return or_mix64(seed + (stream + 1ull) * OR_GAMMA);
}

float or_normal_z(uint64_t st, int64_t logical_index) {
  int64_t sum = 0;
  int c, h;
  for (c = 0; c < 3; ++c) {
    uint64_t w = or_mix64(st + ((uint64_t)logical_index * 3ull + (uint64_t)c + 1ull) * OR_GAMMA);
    for (h = 0; h < 4; ++h) sum += (int64_t)((w >> (16 * h)) & 0xFFFFull);
  }
  return (float)(sum - 393210) / 65536.0f;
}

void or_gen16(uint16_t* dst, int64_t n, int32_t dtype, uint64_t seed, uint64_t stream,
              int64_t logical_base, double sigma, double scale) {
  uint64_t st = or_stream_state(seed, stream);
  float sf = (float)sigma, kf = (float)scale;
  int64_t i;
  for (i = 0; i < n; ++i) {
    float x = or_normal_z(st, logical_base + i) * sf;
    x = x * kf;
    dst[i] = narrow(dtype, x);
  }
}

void or_gen32(float* dst, int64_t n, uint64_t seed, uint64_t stream, int64_t logical_base,
              double sigma) {
  uint64_t st = or_stream_state(seed, stream);
  float sf = (float)sigma;
  int64_t i;
  for (i = 0; i < n; ++i) dst[i] = or_normal_z(st, logical_base + i) * sf;
}

/* Gradient stream of (step, micro-batch, replica); steps count from 1,
 * micro-batches from 0 (a step without accumulation is micro-batch 0),
 * replicas < 256, micro-batches < 4096. */
static uint64_t grad_stream(int64_t step, int64_t micro, int64_t replica) {
  return ((uint64_t)step << 20) | ((uint64_t)micro << 8) | (uint64_t)replica;
}

/* ------------------------------------------------------------------------ */
/* Layout.  [L13] 5.2: the tensors of a unit are flattened end to end into
 * one 1-D FlatParameter, right-padded with zeros to a multiple of the shard
 * count and split into equal shards; shard d belongs to rank d, so the pad
 * (at most N-1 elements) sits in the last shard.  [L13] 0.4 builds one such
 * unit per Linear layer (W then b).  [F6]: ZeRO-1/2 may instead treat all
 * parameters as one giant 1-D vector (the global-flat layout).            */

int or_layout(const int64_t* seg_numel, const int32_t* seg_unit, int64_t nseg, int32_t n_ranks,
              int32_t layout, or_unit* units_out, int64_t max_units, int64_t* n_units_out,
              int64_t* psi_out, int64_t* psi_pad_out) {
  int64_t s, nu = 0, O = 0, lam = 0, M = 0;
  int32_t cur = -1;
  if (n_ranks < 1 || nseg < 1 || !seg_numel || !units_out) return -1;
  if (layout != OR_GLOBAL_FLAT && layout != OR_PER_UNIT) return -1;
  if (layout == OR_PER_UNIT && !seg_unit) return -1;
  for (s = 0; s < nseg; ++s) {
    int32_t uid = (layout == OR_GLOBAL_FLAT) ? 0 : seg_unit[s];
    if (seg_numel[s] < 1) return -1;
    if (uid != cur) {
      if (uid != cur + 1) return -1;  /* unit ids must run 0,0,..,1,1,..,2 */
      if (nu >= max_units) return -1;
      units_out[nu].L = 0;
      units_out[nu].lam = lam;
      nu += 1;
      cur = uid;
    }
    units_out[nu - 1].L += seg_numel[s];
    lam += seg_numel[s];
  }
  for (s = 0; s < nu; ++s) {
    or_unit* u = &units_out[s];
    u->P = ((u->L + n_ranks - 1) / n_ranks) * n_ranks;
    u->S = u->P / n_ranks;
    u->O = O;
    u->M = M;
    O += u->P;
    M += u->S;
  }
  *n_units_out = nu;
  *psi_out = lam;
  *psi_pad_out = O;
  return 0;
}

/* FSDP2 ([MDT] 五.4, 五.6, 六.2): every parameter is its own shard unit,
 * cut along dim 0 into N chunks of ceil(R/N) rows (torch.chunk: the last
 * chunks may be short or empty), each rank's chunk padded with zero rows to
 * ceil(R/N) rows.  In the padded flat the parameter then takes
 * P = N*ceil(R/N)*C elements (C = numel/R), rank r owning [r*S, (r+1)*S)
 * with S = ceil(R/N)*C. */
int or_layout_dim0(const int64_t* seg_numel, const int64_t* seg_rows, int64_t nseg,
                   int32_t n_ranks, or_unit* units_out, int64_t max_units, int64_t* n_units_out,
                   int64_t* psi_out, int64_t* psi_pad_out) {
  int64_t s, O = 0, lam = 0, M = 0;
  if (n_ranks < 1 || nseg < 1 || !seg_numel || !units_out || nseg > max_units) return -1;
  for (s = 0; s < nseg; ++s) {
    int64_t R = (seg_rows && seg_rows[s] > 0) ? seg_rows[s] : seg_numel[s];
    int64_t C, c;
    or_unit* u = &units_out[s];
    if (seg_numel[s] < 1 || seg_numel[s] % R != 0) return -1;
    C = seg_numel[s] / R;
    c = (R + n_ranks - 1) / n_ranks;
    u->L = seg_numel[s];
    u->P = (int64_t)n_ranks * c * C;
    u->S = c * C;
    u->O = O;
    u->lam = lam;
    u->M = M;
    O += u->P;
    lam += u->L;
    M += u->S;
  }
  *n_units_out = nseg;
  *psi_out = lam;
  *psi_pad_out = O;
  return 0;
}

/* Bytes of model state one rank holds once backward has finished ([L13] 2.3
 * and 3.5, and its summary): stage 0 (plain DP) 2+2+12 bytes per parameter;
 * stage 1 full 16-bit params and grads plus its 1/N of the fp32
 * master/m/v; stage 2 also keeps only its 1/N of the grads; stage 3 keeps
 * only its 1/N of everything.  With padding, the sharded stages count the
 * padded Psi' ([L13] 3.6).  The stage-3 peak follows exercise 5 of the
 * notes: while backward runs unit b (units run last to first), a rank holds
 * its resident shards, the already reduce-scattered grad shards of units
 * after b, and the full 16-bit params and full grads of unit b.  For stages
 * 0-2 the peak reported is the after-backward figure (the transient fp32
 * gradient of one unit at update time is not modelled).                 */
int or_ledger(const or_unit* units, int64_t n_units, int32_t n_ranks, int32_t stage,
              int64_t* after_backward_bytes, int64_t* peak_bytes) {
  int64_t psi = 0, psi_pad = 0, s_tot = 0, u, b;
  if (!units || n_units < 1 || n_ranks < 1 || stage < 0 || stage > 4) return -1;
  for (u = 0; u < n_units; ++u) {
    psi += units[u].L;
    psi_pad += units[u].P;
    s_tot += units[u].S;
  }
  switch (stage) {
    case 0: *after_backward_bytes = 2 * psi + 2 * psi + 12 * psi; break;
    case 1: *after_backward_bytes = 2 * psi_pad + 2 * psi_pad + 12 * s_tot; break;
    case 2: *after_backward_bytes = 2 * psi_pad + 2 * s_tot + 12 * s_tot; break;
    case 3: *after_backward_bytes = 2 * s_tot + 2 * s_tot + 12 * s_tot; break;
    default:
      /* FSDP2 with fp32 parameters: the fp32 shard is the parameter and the
       * master; fp32 grad shard; m and v -- 4 + 4 + 8 bytes per element
       * ([MDT] 五.6) */
      *after_backward_bytes = 4 * s_tot + 4 * s_tot + 8 * s_tot;
      break;
  }
  *peak_bytes = *after_backward_bytes;
  if (stage == 3) {
    int64_t best = 0;
    for (b = n_units - 1; b >= 0; --b) {
      int64_t reduced = 0, here;
      for (u = b + 1; u < n_units; ++u) reduced += units[u].S;
      here = 2 * s_tot + 12 * s_tot + 2 * reduced + 2 * units[b].P + 2 * units[b].P;
      if (here > best) best = here;
    }
    *peak_bytes = best;
  }
  return 0;
}

/* Bytes one rank sends per step with ring collectives ([L13] 4.1-4.2): a
 * ring reduce-scatter or all-gather of 2*Psi' bytes sends (N-1)/N of it.
 * variant 0: DP all-reduce (RS + AG); 1, 2: stage 1/2 (RS of grads + AG of
 * params); 3: stage 3 (AG in forward, AG in backward, RS); 4: the slides'
 * stage 1 (all-reduce of grads, then AG of params).                      */
double or_comm_bytes(int64_t psi_pad, int32_t n_ranks, int32_t variant) {
  double passes;
  switch (variant) {
    case 0: case 1: case 2: passes = 2.0; break;
    case 3: case 4: passes = 3.0; break;
    default: return -1.0;
  }
  return passes * ((double)(n_ranks - 1) / (double)n_ranks) * 2.0 * (double)psi_pad;
}

/* ------------------------------------------------------------------------ */
/* Reduce-scatter ([L13] 3.1 step 3 and 3.2; [F7] ZeRO-2 hook): rank r
 * receives the element-wise reduction of all N replicas over its own shard of
 * every unit.  Reading taken: the sum is done in binary32, in the fixed rank
 * order 0..N-1 starting from replica 0 widened to binary32; the 1/N of the
 * average is folded into the gradient scale (see or_finish).  A ring would
 * accumulate in a rotating order ([L13] 3.4 condition 2); this is the fixed
 * order.  Output: rs_out[r] has the rank's shard buffer layout (unit-major,
 * unit u at offset M_u, S_u elements, pad included).                      */
int or_reduce_scatter(int32_t grad_dtype, int32_t n_ranks, const or_unit* units, int64_t n_units,
                      const uint16_t* const* grads, float* const* rs_out) {
  int64_t u, j;
  int32_t r, q;
  if (!units || !grads || !rs_out || n_ranks < 1) return -1;
  for (r = 0; r < n_ranks; ++r) {
    for (u = 0; u < n_units; ++u) {
      const or_unit* U = &units[u];
      for (j = 0; j < U->S; ++j) {
        int64_t p = U->O + (int64_t)r * U->S + j;
        float acc = widen(grad_dtype, grads[0][p]);
        for (q = 1; q < n_ranks; ++q) acc = acc + widen(grad_dtype, grads[q][p]);
        rs_out[r][U->M + j] = acc;
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Scalars of one step, from the global squared norm and overflow flag.
 *  - [MDT] 四.3: the optimizer first checks for fp16 overflow, then clips,
 *    then steps.  Reading: any non-finite reduced gradient skips the step;
 *    with dynamic loss scaling the scale halves and the growth counter
 *    resets; m, v, the master, t and the 16-bit params are left untouched.
 *    Otherwise t advances, and after K consecutive applied steps the scale
 *    doubles.
 *  - Global L2 clipping on the fp32 gradient ([MDT] 五.7; Femtotron dev log
 *    #4 and #5).  Reading: the norm is of the unscaled, averaged gradient,
 *    norm = sqrt(sumsq) / (S*N) in double, and the coefficient is
 *    min(1, max_norm / (norm + 1e-6)); max_norm <= 0 disables clipping.
 *  - Unscale, average and clip are one binary32 factor gs = f32(coef/(S*N)).
 *  - Adam's bias corrections ([L13] 2.1) use beta^t formed by t-1 successive
 *    double multiplications; every scalar is rounded to binary32 once.    */
int or_finish(double sumsq, int32_t overflow, int32_t n_ranks, const or_hparams* hp,
              or_scale_state* st, or_scalars* sc, or_result* res) {
  double S, norm, coef, B1, B2;
  int64_t i;
  if (!hp || !st || !sc || !res || n_ranks < 1) return -1;
  memset(res, 0, sizeof(*res));
  memset(sc, 0, sizeof(*sc));
  res->overflow = overflow ? 1 : 0;
  res->sumsq = sumsq;
  res->scale_used = st->loss_scale;
  if (overflow) {
    res->skipped = 1;
    if (st->dynamic) {
      st->loss_scale = st->loss_scale * 0.5;
      st->growth_ctr = 0;
    }
    res->scale_next = st->loss_scale;
    res->t = st->t;
    return 0;
  }
  S = st->loss_scale;
  st->t += 1;
  st->growth_ctr += 1;
  if (st->dynamic && st->growth_interval > 0 && st->growth_ctr >= st->growth_interval) {
    st->loss_scale = S * 2.0;
    st->growth_ctr = 0;
  }
  norm = sqrt(sumsq) / (S * (double)n_ranks);
  coef = 1.0;
  if (hp->max_norm > 0.0) {
    coef = hp->max_norm / (norm + 1e-6);
    if (coef > 1.0) coef = 1.0;
  }
  B1 = hp->beta1;
  B2 = hp->beta2;
  for (i = 1; i < st->t; ++i) {
    B1 = B1 * hp->beta1;
    B2 = B2 * hp->beta2;
  }
  sc->gs = (float)(coef / (S * (double)n_ranks));
  sc->dec = (float)(1.0 - hp->lr * hp->weight_decay);
  sc->b1 = (float)hp->beta1;
  sc->c1 = (float)(1.0 - hp->beta1);
  sc->b2 = (float)hp->beta2;
  sc->c2 = (float)(1.0 - hp->beta2);
  sc->bc1 = (float)(1.0 - B1);
  sc->bc2 = (float)(1.0 - B2);
  sc->lrf = (float)hp->lr;
  sc->ef = (float)hp->eps;
  res->norm = norm;
  res->coef = coef;
  res->gs = sc->gs;
  res->scale_next = st->loss_scale;
  res->t = st->t;
  return 0;
}

/* AdamW on fp32 master/m/v, element by element ([L13] 2.1 for Adam, 2.2 for
 * the fp32 master; 3.1: Adam is element-wise, so a shard updates exactly as
 * the same elements of the whole array would).  Reading: decoupled weight
 * decay applied to the parameter first, then Adam with epsilon outside the
 * square root and bias corrections 1 - beta^t:
 *     g = acc*gs;  p = p*dec;  m = b1*m + c1*g;  v = b2*v + c2*(g*g);
 *     d = sqrt(v/bc2) + eps;   p = p - lr*((m/bc1)/d)                      */
void or_adamw_array(int64_t n, const float* acc, const or_scalars* sc, float* p, float* m,
                    float* v) {
  int64_t i;
  for (i = 0; i < n; ++i) {
    float g = acc[i] * sc->gs;
    float pp = p[i] * sc->dec;
    float mm = sc->b1 * m[i] + sc->c1 * g;
    float vv = sc->b2 * v[i] + sc->c2 * (g * g);
    float d = sqrtf(vv / sc->bc2) + sc->ef;
    float mh = mm / sc->bc1;
    pp = pp - sc->lrf * (mh / d);
    p[i] = pp;
    m[i] = mm;
    v[i] = vv;
  }
}

/* The optimizer side of one step from already reduce-scattered gradients
 * ([L13] 3.1 steps 4-6; [MDT] 四.3 step order): acc[r] is rank r's fp32
 * gradient shard (the fixed-order sums over ranks, accumulated over
 * micro-batches when there are several).
 *   2. overflow: any non-finite value of any shard, padding included;
 *   3. squared norm: sum of (double)acc^2 over the real elements in logical
 *      order (unit by unit, ranks in order), so the value does not depend on
 *      the layout; the padding is zero by contract and would add nothing;
 *   4-6. scalars (or_finish); a skipped step stops here;
 *   7. each rank runs AdamW on its shard (padding included: zero stays zero);
 *   8. each rank casts its shard to 16 bits; stages 0-2 place it in the full
 *      padded buffer (the post-update all-gather, [L13] 3.1 step 6), stage 3
 *      keeps it as the rank's resident shard ([L13] exercise 4), unless
 *      param_shards is NULL: fp32 parameters (FSDP2, [MDT] 五.6), no copy.
 * master/exp_avg/exp_avg_sq/param_shards[r] are rank r's shard buffers:
 * sum_u S_u elements, unit u at offset M_u.                               */
int or_step_reduced(int32_t param_dtype, int32_t n_ranks, const or_unit* units, int64_t n_units,
                    int32_t stage, float* const* acc, float* const* master,
                    float* const* exp_avg, float* const* exp_avg_sq, uint16_t* params_full,
                    uint16_t* const* param_shards, const or_hparams* hp, or_scale_state* st,
                    or_result* res) {
  int64_t s_tot = 0, u, j, k;
  int32_t r, overflow = 0;
  double ss = 0.0;
  or_scalars sc;
  if (!units || n_units < 1 || !acc || !master || !exp_avg || !exp_avg_sq || !hp || !st || !res)
    return -1;
  if (stage < 3 && !params_full) return -1;
  for (u = 0; u < n_units; ++u) s_tot += units[u].S;

  for (r = 0; r < n_ranks; ++r)
    for (k = 0; k < s_tot; ++k)
      if (!isfinite(acc[r][k])) overflow = 1;

  for (u = 0; u < n_units; ++u) {
    const or_unit* U = &units[u];
    for (r = 0; r < n_ranks; ++r)
      for (j = 0; j < U->S; ++j) {
        if ((int64_t)r * U->S + j >= U->L) continue;  /* padding */
        ss += (double)acc[r][U->M + j] * (double)acc[r][U->M + j];
      }
  }

  or_finish(ss, overflow, n_ranks, hp, st, &sc, res);
  if (res->skipped) return 0;

  for (r = 0; r < n_ranks; ++r)
    or_adamw_array(s_tot, acc[r], &sc, master[r], exp_avg[r], exp_avg_sq[r]);

  if (stage == 3 && !param_shards) return 0;  /* fp32 parameters: no 16-bit copy */
  for (r = 0; r < n_ranks; ++r) {
    for (u = 0; u < n_units; ++u) {
      const or_unit* U = &units[u];
      for (j = 0; j < U->S; ++j) {
        uint16_t q = narrow(param_dtype, master[r][U->M + j]);
        if (stage < 3)
          params_full[U->O + (int64_t)r * U->S + j] = q;
        else
          param_shards[r][U->M + j] = q;
      }
    }
  }
  return 0;
}

/* One emulated ZeRO step for all N ranks ([L13] 3.1 steps 3-6, 3.2, 3.3):
 * the reduce-scatter (each rank gets the fixed-order sum over its shard of
 * every unit), then the optimizer side (or_step_reduced). */
int or_zero_step(int32_t grad_dtype, int32_t param_dtype, int32_t n_ranks, const or_unit* units,
                 int64_t n_units, int32_t stage, const uint16_t* const* grads,
                 float* const* master, float* const* exp_avg, float* const* exp_avg_sq,
                 uint16_t* params_full, uint16_t* const* param_shards, const or_hparams* hp,
                 or_scale_state* st, or_result* res) {
  int64_t s_tot = 0, u;
  int32_t r;
  float** acc;
  int rc;
  if (!units || n_units < 1 || !grads) return -1;
  for (u = 0; u < n_units; ++u) s_tot += units[u].S;
  acc = (float**)calloc((size_t)n_ranks, sizeof(float*));
  if (!acc) return -2;
  rc = 0;
  for (r = 0; r < n_ranks && rc == 0; ++r) {
    acc[r] = (float*)malloc((size_t)(s_tot > 0 ? s_tot : 1) * sizeof(float));
    if (!acc[r]) rc = -2;
  }
  if (rc == 0) {
    or_reduce_scatter(grad_dtype, n_ranks, units, n_units, grads, acc);
    rc = or_step_reduced(param_dtype, n_ranks, units, n_units, stage, acc, master, exp_avg,
                         exp_avg_sq, params_full, param_shards, hp, st, res);
  }
  for (r = 0; r < n_ranks; ++r) free(acc[r]);
  free(acc);
  return rc;
}

/* One element of a gradient buffer: 16-bit (widened exactly) or binary32. */
static float grad_at(int32_t dtype, const void* g, int64_t p) {
  if (dtype == OR_F32) return ((const float*)g)[p];
  return widen(dtype, ((const uint16_t*)g)[p]);
}

/* Backward-side reduce-scatter of one bucket as its gradients arrive
 * ([L13] 3.2: with buckets, one reduce-scatter per bucket during backward;
 * [MDT] 三.3: each bucket padded to a multiple of the DP size and split
 * evenly, rank r owning the r-th piece; 四.3: IPG buckets reduced to their
 * owners).  Unit u of the plan is the bucket; shards[r] are rank r's shard
 * buffers (unit u at offset M_u).
 * Gradient accumulation ([L13] 5.6 and [MDT] 五.7: either every micro-batch
 * is reduce-scattered and the result added to the sharded gradient, or the
 * full gradients are accumulated locally and reduced once at the last
 * micro-batch): the micro-batch's fixed-order sum over ranks is formed
 * first and then added to the shard (reading: the reduced tensor is
 * produced by the collective before the shard's gradient accumulates it);
 * accumulate == 0 stores the sum, as the first micro-batch does.
 * grad_dtype OR_F32 takes binary32 replicas: the locally accumulated fp32
 * gradients of the no_sync scheme ([MDT] 三.3: fp32 main_grad buffers
 * reduced in fp32).                                                       */
int or_rs_accumulate(int32_t grad_dtype, int32_t n_ranks, const or_unit* units, int64_t n_units,
                     int64_t u, const void* const* grads, float* const* shards,
                     int32_t accumulate) {
  int64_t j;
  int32_t r, q;
  const or_unit* U;
  if (!units || !grads || !shards || u < 0 || u >= n_units) return -1;
  if (grad_dtype != OR_F16 && grad_dtype != OR_BF16 && grad_dtype != OR_F32) return -1;
  U = &units[u];
  for (r = 0; r < n_ranks; ++r) {
    for (j = 0; j < U->S; ++j) {
      int64_t p = U->O + (int64_t)r * U->S + j;
      float sum = grad_at(grad_dtype, grads[0], p);
      for (q = 1; q < n_ranks; ++q) sum = sum + grad_at(grad_dtype, grads[q], p);
      shards[r][U->M + j] = accumulate ? shards[r][U->M + j] + sum : sum;
    }
  }
  return 0;
}

/* Local gradient accumulation of one replica under no_sync ([MDT] 三.3: the
 * backward hook adds each micro-batch's gradient into the parameter's fp32
 * main_grad; no communication until the last micro-batch): acc[i] =
 * acc[i] + f32(grad[i]), or f32(grad[i]) for the first micro-batch. */
int or_local_accumulate(int32_t grad_dtype, int64_t n, const uint16_t* grad, float* acc,
                        int32_t accumulate) {
  int64_t i;
  if (!grad || !acc || n < 0) return -1;
  if (grad_dtype != OR_F16 && grad_dtype != OR_BF16) return -1;
  for (i = 0; i < n; ++i) {
    float g = widen(grad_dtype, grad[i]);
    acc[i] = accumulate ? acc[i] + g : g;
  }
  return 0;
}

/* Megatron's gradient buckets ([MDT] 三.3): parameters in buffer order
 * are grouped into buckets of bucket_numel elements, by default
 * max(40,000,000, 1,000,000 * dp_size).  Reading: parameters are not split;
 * a bucket is closed as soon as its element count reaches bucket_numel, and
 * the last bucket takes whatever remains.  unit_out[s] receives segment s's
 * bucket id (0, 0, .., 1, ..).                                           */
int or_bucket_assign(const int64_t* seg_numel, int64_t nseg, int32_t n_ranks,
                     int64_t bucket_numel, int32_t* unit_out, int64_t* n_buckets) {
  int64_t s, fill = 0, B;
  int32_t cur = 0;
  if (!seg_numel || !unit_out || !n_buckets || nseg < 1 || n_ranks < 1) return -1;
  B = bucket_numel > 0 ? bucket_numel : 1000000LL * n_ranks;
  if (bucket_numel <= 0 && B < 40000000LL) B = 40000000LL;
  for (s = 0; s < nseg; ++s) {
    if (seg_numel[s] < 1) return -1;
    unit_out[s] = cur;
    fill += seg_numel[s];
    if (fill >= B && s + 1 < nseg) {
      cur += 1;
      fill = 0;
    }
  }
  *n_buckets = (int64_t)cur + 1;
  return 0;
}

/* ZeRO-3 / FSDP gather of one unit before it is used ([L13] 3.3 and 5.1
 * step 3; [F9] unshard): the N ranks' shards of unit u, in rank order, form
 * the unit's padded FlatParameter: unit_buf[r*S_u + j] = shard_r[u][j].    */
int or_gather_unit(const or_unit* units, int64_t n_units, int32_t n_ranks, int64_t u,
                   const uint16_t* const* param_shards, uint16_t* unit_buf) {
  int64_t j;
  int32_t r;
  if (!units || u < 0 || u >= n_units || !param_shards || !unit_buf) return -1;
  for (r = 0; r < n_ranks; ++r)
    for (j = 0; j < units[u].S; ++j)
      unit_buf[(int64_t)r * units[u].S + j] = param_shards[r][units[u].M + j];
  return 0;
}

/* One FSDP2 step for all N ranks ([MDT] 五.4 and 五.6): the reduce-scatter in
 * fp32 writes each rank's fp32 gradient shard (kept, as the shard's .grad);
 * overflow, norm and clip as in or_zero_step; AdamW updates the fp32 shard,
 * which is itself the parameter, so the step writes no 16-bit copy -- the
 * 16-bit values appear only when a unit is gathered (or_fsdp2_gather).
 * Buffers are per-rank shard buffers (sum_u S_u elements, unit u at M_u). */
int or_fsdp2_step(int32_t grad_dtype, int32_t n_ranks, const or_unit* units, int64_t n_units,
                  const uint16_t* const* grads, float* const* master, float* const* exp_avg,
                  float* const* exp_avg_sq, float* const* grad_shards, const or_hparams* hp,
                  or_scale_state* st, or_result* res) {
  int64_t s_tot = 0, u, j, k;
  int32_t r, overflow = 0;
  double ss = 0.0;
  or_scalars sc;
  if (!units || n_units < 1 || !grads || !master || !exp_avg || !exp_avg_sq || !grad_shards ||
      !hp || !st || !res)
    return -1;
  for (u = 0; u < n_units; ++u) s_tot += units[u].S;
  or_reduce_scatter(grad_dtype, n_ranks, units, n_units, grads, grad_shards);
  for (r = 0; r < n_ranks; ++r)
    for (k = 0; k < s_tot; ++k)
      if (!isfinite(grad_shards[r][k])) overflow = 1;
  for (u = 0; u < n_units; ++u) {
    const or_unit* U = &units[u];
    for (r = 0; r < n_ranks; ++r)
      for (j = 0; j < U->S; ++j) {
        if ((int64_t)r * U->S + j >= U->L) continue;  /* padding */
        ss += (double)grad_shards[r][U->M + j] * (double)grad_shards[r][U->M + j];
      }
  }
  or_finish(ss, overflow, n_ranks, hp, st, &sc, res);
  if (res->skipped) return 0;
  for (r = 0; r < n_ranks; ++r)
    or_adamw_array(s_tot, grad_shards[r], &sc, master[r], exp_avg[r], exp_avg_sq[r]);
  return 0;
}

/* FSDP2 unshard of one group of parameters (units first .. first+count-1)
 * before it is used ([MDT] 五.4: each rank's fp32 shards are cast to the
 * parameter dtype, all-gathered, then copied out into each parameter's
 * full tensor): out holds the group's parameters end to end, unpadded, in
 * order; element e of parameter u comes from rank e / S_u, offset e % S_u. */
int or_fsdp2_gather(const or_unit* units, int64_t n_units, int32_t n_ranks, int64_t first,
                    int64_t count, int32_t dtype, const float* const* master, uint16_t* out) {
  int64_t i, e, pos = 0;
  if (!units || !master || !out || first < 0 || count < 1 || first + count > n_units) return -1;
  for (i = first; i < first + count; ++i) {
    const or_unit* U = &units[i];
    for (e = 0; e < U->L; ++e) {
      int64_t r = e / U->S, j = e % U->S;
      if (r >= n_ranks) return -1;
      out[pos + e] = narrow(dtype, master[r][U->M + j]);
    }
    pos += U->L;
  }
  return 0;
}

/* Resharding by logical index ([F5]: when the DP size changes between save
 * and load, the shard offsets lose their meaning and the state has to be
 * redistributed for the new parallelism; [MDT] 六.4: DeepSpeed converts its
 * per-rank ZeRO checkpoints to a universal one, torchtitan's DCP reshards
 * natively).  Every real element keeps its value
 * and moves from its place under layout A (N_a ranks) to its place under
 * layout B (N_b ranks); every padding element of B is zero.  Rank r's real
 * part of unit u is the logical run [lam_u + r*S_u, lam_u + r*S_u +
 * clamp(L_u - r*S_u, 0, S_u)) in every layout, so the element is found by
 * walking both layouts' (unit, rank) runs in logical order.  elem_bytes is
 * 2 or 4; a[r] / b[r] are the ranks' shard buffers (unit u at M_u). */
int or_reshard(const or_unit* ua, int64_t nua, int32_t na, const void* const* a,
               const or_unit* ub, int64_t nub, int32_t nb, void* const* b, int32_t elem_bytes) {
  int64_t psi_a = 0, psi_b = 0, u, i;
  int32_t r;
  char* logical;
  if (!ua || !ub || !a || !b || na < 1 || nb < 1 || (elem_bytes != 2 && elem_bytes != 4))
    return -1;
  for (u = 0; u < nua; ++u) psi_a += ua[u].L;
  for (u = 0; u < nub; ++u) psi_b += ub[u].L;
  if (psi_a != psi_b) return -1;
  logical = (char*)malloc((size_t)(psi_a > 0 ? psi_a : 1) * (size_t)elem_bytes);
  if (!logical) return -2;
  /* A's runs into logical order */
  for (u = 0; u < nua; ++u)
    for (r = 0; r < na; ++r)
      for (i = 0; i < ua[u].S; ++i) {
        int64_t e = (int64_t)r * ua[u].S + i;
        if (e >= ua[u].L) break;
        memcpy(logical + (ua[u].lam + e) * elem_bytes,
               (const char*)a[r] + (ua[u].M + i) * elem_bytes, (size_t)elem_bytes);
      }
  /* logical order into B's runs, zeros in B's padding */
  for (u = 0; u < nub; ++u)
    for (r = 0; r < nb; ++r)
      for (i = 0; i < ub[u].S; ++i) {
        int64_t e = (int64_t)r * ub[u].S + i;
        char* dst = (char*)b[r] + (ub[u].M + i) * elem_bytes;
        if (e < ub[u].L)
          memcpy(dst, logical + (ub[u].lam + e) * elem_bytes, (size_t)elem_bytes);
        else
          memset(dst, 0, (size_t)elem_bytes);
      }
  free(logical);
  return 0;
}

/* Plain data-parallel reference on one unpadded buffer of Psi elements: the
 * same N replicas are summed in the same rank order, and the whole array is
 * updated at once.  ZeRO-1/2 must reproduce it bit for bit ([L13] 3.4: the
 * same summation order and an element-wise Adam make the results identical).
 * grads[q] is replica q's unpadded gradient, logical order.               */
int or_dp_step(int32_t grad_dtype, int32_t param_dtype, int32_t n_ranks, int64_t psi,
               const uint16_t* const* grads, float* master, float* exp_avg, float* exp_avg_sq,
               uint16_t* params, const or_hparams* hp, or_scale_state* st, or_result* res) {
  float* acc;
  int64_t i;
  int32_t q, overflow = 0;
  double ss = 0.0;
  or_scalars sc;
  if (!grads || !master || !exp_avg || !exp_avg_sq || !params || !hp || !st || !res) return -1;
  acc = (float*)malloc((size_t)(psi > 0 ? psi : 1) * sizeof(float));
  if (!acc) return -2;
  for (i = 0; i < psi; ++i) {
    float a = widen(grad_dtype, grads[0][i]);
    for (q = 1; q < n_ranks; ++q) a = a + widen(grad_dtype, grads[q][i]);
    acc[i] = a;
    if (!isfinite(a)) overflow = 1;
    ss += (double)a * (double)a;
  }
  or_finish(ss, overflow, n_ranks, hp, st, &sc, res);
  if (!res->skipped) {
    or_adamw_array(psi, acc, &sc, master, exp_avg, exp_avg_sq);
    for (i = 0; i < psi; ++i) params[i] = narrow(param_dtype, master[i]);
  }
  free(acc);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Full-size checks by regeneration: the reduced gradient of a logical index
 * is recomputed from the seeded generator, so a sample of elements (and the
 * exact global squared norm, range by range) can be checked at any model
 * size without holding the replicas in host memory.  An optional injection
 * overrides one (step, replica, index) with given 16-bit bits.           */

#define OR_MAX_REPLICAS 64
#define OR_MAX_MICRO 16

/* Starting states of the gradient streams of `step`: st[a*N + q] for
 * micro-batch a, replica q. */
static int grad_states(uint64_t seed, int64_t step, int32_t n_micro, int32_t n_ranks,
                       uint64_t* st) {
  int32_t q, a;
  if (n_ranks < 1 || n_ranks > OR_MAX_REPLICAS || n_micro < 1 || n_micro > OR_MAX_MICRO)
    return -1;
  for (a = 0; a < n_micro; ++a)
    for (q = 0; q < n_ranks; ++q)
      st[a * n_ranks + q] = or_stream_state(seed, grad_stream(step, a, q));
  return 0;
}

/* Replica q's widened gradient at index i in micro-batch a (an injection
 * applies to micro-batch 0). */
static float regen_grad(int32_t dtype, int32_t n_ranks, const uint64_t* st, int64_t step,
                        float sf, float kf, int64_t i, int32_t a, int32_t q,
                        const or_inject* inj) {
  uint16_t h;
  if (a == 0 && inj && inj->step == step && inj->replica == q && inj->index == i) {
    h = inj->bits;
  } else {
    float x = or_normal_z(st[a * n_ranks + q], i) * sf;
    x = x * kf;
    h = narrow(dtype, x);
  }
  return widen(dtype, h);
}

/* The reduced (and accumulated) gradient of logical index i.  mode 0:
 * every micro-batch is reduce-scattered and added to the shard
 * (or_rs_accumulate per micro-batch); mode 1: no_sync, each replica
 * accumulates in fp32 (or_local_accumulate) and the fp32 buffers are
 * summed once in rank order.  With one micro-batch both are the plain
 * reduce-scatter sum. */
static float regen_acc_one(int32_t dtype, int32_t n_ranks, int32_t n_micro, int32_t mode,
                           const uint64_t* st, int64_t step, float sf, float kf, int64_t i,
                           const or_inject* inj) {
  float acc = 0.0f;
  int32_t q, a;
  if (mode == 0) {
    for (a = 0; a < n_micro; ++a) {
      float sum = 0.0f;
      for (q = 0; q < n_ranks; ++q) {
        float g = regen_grad(dtype, n_ranks, st, step, sf, kf, i, a, q, inj);
        sum = (q == 0) ? g : sum + g;
      }
      acc = (a == 0) ? sum : acc + sum;
    }
  } else {
    for (q = 0; q < n_ranks; ++q) {
      float loc = 0.0f;
      for (a = 0; a < n_micro; ++a) {
        float g = regen_grad(dtype, n_ranks, st, step, sf, kf, i, a, q, inj);
        loc = (a == 0) ? g : loc + g;
      }
      acc = (q == 0) ? loc : acc + loc;
    }
  }
  return acc;
}

int or_regen_accum_sumsq(int32_t grad_dtype, int32_t n_ranks, int32_t n_micro, int32_t mode,
                         uint64_t seed, int64_t step, double sigma, double scale, int64_t i0,
                         int64_t i1, const or_inject* inj, double* sumsq, int32_t* nonfinite) {
  int64_t i;
  double ss = 0.0;
  int32_t nf = 0;
  float sf = (float)sigma, kf = (float)scale;
  uint64_t st[OR_MAX_REPLICAS * OR_MAX_MICRO];
  if (!sumsq || !nonfinite || i1 < i0 || (mode != 0 && mode != 1)) return -1;
  if (grad_states(seed, step, n_micro, n_ranks, st) != 0) return -1;
  for (i = i0; i < i1; ++i) {
    float a = regen_acc_one(grad_dtype, n_ranks, n_micro, mode, st, step, sf, kf, i, inj);
    if (!isfinite(a)) nf = 1;
    ss += (double)a * (double)a;
  }
  *sumsq = ss;
  *nonfinite = nf;
  return 0;
}

int or_regen_accum_acc(int32_t grad_dtype, int32_t n_ranks, int32_t n_micro, int32_t mode,
                       uint64_t seed, int64_t step, double sigma, double scale, int64_t n,
                       const int64_t* logical_idx, const or_inject* inj, float* acc_out) {
  int64_t k;
  float sf = (float)sigma, kf = (float)scale;
  uint64_t st[OR_MAX_REPLICAS * OR_MAX_MICRO];
  if (!logical_idx || !acc_out || (mode != 0 && mode != 1)) return -1;
  if (grad_states(seed, step, n_micro, n_ranks, st) != 0) return -1;
  for (k = 0; k < n; ++k)
    acc_out[k] = regen_acc_one(grad_dtype, n_ranks, n_micro, mode, st, step, sf, kf,
                               logical_idx[k], inj);
  return 0;
}

/* The squared norm and overflow flag of given reduced values (steps 2-3 of
 * the step, [MDT] 四.3 check overflow then clip by the global norm): used
 * where the values are not the plain sums, e.g. sums rounded to the
 * gradient dtype before an offloaded update ([L13] 7.1's 16-bit gradient
 * edge). */
int or_sumsq_array(int64_t n, const float* x, double* sumsq, int32_t* nonfinite) {
  int64_t i;
  double ss = 0.0;
  int32_t nf = 0;
  if (!sumsq || !nonfinite || n < 0 || (n > 0 && !x)) return -1;
  for (i = 0; i < n; ++i) {
    if (!isfinite(x[i])) nf = 1;
    ss += (double)x[i] * (double)x[i];
  }
  *sumsq = ss;
  *nonfinite = nf;
  return 0;
}

int or_regen_sumsq(int32_t grad_dtype, int32_t n_ranks, uint64_t seed, int64_t step, double sigma,
                   double scale, int64_t i0, int64_t i1, const or_inject* inj, double* sumsq,
                   int32_t* nonfinite) {
  return or_regen_accum_sumsq(grad_dtype, n_ranks, 1, 0, seed, step, sigma, scale, i0, i1, inj,
                              sumsq, nonfinite);
}

int or_regen_acc(int32_t grad_dtype, int32_t n_ranks, uint64_t seed, int64_t step, double sigma,
                 double scale, int64_t n, const int64_t* logical_idx, const or_inject* inj,
                 float* acc_out) {
  return or_regen_accum_acc(grad_dtype, n_ranks, 1, 0, seed, step, sigma, scale, n, logical_idx,
                            inj, acc_out);
}
