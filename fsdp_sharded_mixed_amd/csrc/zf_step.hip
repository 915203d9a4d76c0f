// zf_step.hip -- the step's kernels (pass 1, the norm reduction, the finish,
// the fused update pass) and the C entry points of the step.
//
// The step is a stream over the padded flat index p with under one flop per
// byte, so it is bound by HBM bandwidth and uses no matrix cores.  A lane
// moves 4-element quads (16 bytes of fp32, 8 bytes of a 16-bit stream), so
// every wave instruction covers one contiguous span (zf_device.h), from
// 16-byte aligned bases.
//
// Pages followed (by title and section):
//   CMU 15-779 Lecture 13 notes, "Zero Redundancy and PyTorch FSDP": 2.1
//   (Adam), 2.2 (update in fp32 master weights, then cast down), 3.1-3.3 (the
//   stages: reduce-scatter, update of the own shard, all-gather of 16-bit
//   params, or per-unit gather under stage 3), 3.4 (same summation order =>
//   same bits), 5.2 (FlatParameter padding).
//   Megatron / DeepSpeed / torchtitan architecture and source guide, ch. 四.3
//   (check fp16 overflow, clip, Adam per fp32 partition, copy to the 16-bit
//   partition) and 五.7 (clipping by the global gradient norm).
//
// Arithmetic contract (shared with nothing; checked against the CPU oracle):
//   acc  = f32(g_0) + f32(g_1) + ... + f32(g_{N-1})          in rank order
//   skip = any acc is inf or NaN (padding included)
//   ss   = sum of (double)acc^2; norm = sqrt(ss)/(S*N); coef = min(1,
//          max_norm/(norm+1e-6)); gs = f32(coef/(S*N))
//   g = acc*gs; p = p*dec; m = b1*m + c1*g; v = b2*v + c2*(g*g);
//   p = p - lr*((m/bc1) / (sqrt(v/bc2) + eps)); out = RNE16(p)
// Each operator is one IEEE binary32 operation: built with
// -ffp-contract=off and correctly rounded division and square root.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "zf_device.h"
#include "zf_hip_status.h"
#include "zf_internal.h"

// The workspace of zf_shard_step_noalloc: a static device array that every
// GPU the library runs on holds from the code object's load until the
// process ends, each GPU its own copy at its own address.  In host code the
// name `scratch` only stands for the symbol: its device address comes from
// hipGetSymbolAddress (noalloc_scratch below), never from the name itself.
static __device__ __align__(256) unsigned char scratch[ZF_NOALLOC_SCRATCH_BYTES];

namespace {

using namespace zf::dev;
using zf::hip_ok;
using zf::kThreads;
using zf::DevState;
using zf::kStateBytes;

// ---------------------------------------------------------------------------
// Pass 1: reduce-scatter sums, overflow flag and squared-norm partials, one
// tile per block.  The last block also takes the ragged tail (< 4 elements).
struct Pass1Args {
  GradPtrs g;
  int64_t n;          // Psi'
  float* rs;          // fp32 sums (OUT == 1, 3) or unused
  uint16_t* rs16;     // 16-bit sums (OUT == 2) or unused
  Partial* partials;  // one per tile (NORM) or unused
  int32_t nr;
  int32_t tile_map;   // see tile_of_block
  int64_t plain_from; // OUT == 3: full tiles from this quad on store the sums
                      // cache-allocating (see zf::cached_sums_quads)
};

// OUT: 0 the sums stay in registers; 1 they are stored in fp32,
// non-temporal; 3 as 1, but full tiles from quad plain_from on use plain,
// cache-allocating stores (see zf::cached_sums_quads); 2 they are rounded to
// the gradient dtype and stored in 16 bits, and the overflow flag and the
// norm are taken on the rounded values (the 16-bit gradients an offloaded
// optimizer receives).
constexpr bool stores_fp32(int out) { return out == 1 || out == 3; }

// The quads of one tile.  FULL: every quad of the tile lies below nq (all
// tiles but the last), so no load or store carries a range check: the loads
// issue back to back instead of one predicated branch each.  PLAIN: the fp32
// sums go out with plain stores, in another shape than the non-temporal ones
// (stq32_halves), because the compiler merges two stores of one value to one
// address into one and drops the non-temporal hint.
template <int NR, int DT, int OUT, bool NORM, int Q, bool FULL, bool PLAIN>
__device__ __forceinline__ void pass1_quads(const Pass1Args& a, int nr, int64_t nq, int64_t q0,
                                            double& ss, uint32_t& bad) {
  int64_t qi[Q];
  bool ok[Q];
#pragma unroll
  for (int h = 0; h < Q; ++h) {
    qi[h] = q0 + (int64_t)h * kThreads;
    ok[h] = FULL || qi[h] < nq;
  }
  f32x4 acc[Q];
  sum_quads<NR, DT, true, Q>(a.g, nr, qi, ok, acc);
#pragma unroll
  for (int h = 0; h < Q; ++h) {
    if (!ok[h]) continue;
    if constexpr (stores_fp32(OUT) && PLAIN) stq32_halves(a.rs, qi[h], acc[h]);
    if constexpr (stores_fp32(OUT) && !PLAIN) stq32_nt(a.rs, qi[h], acc[h]);
    if constexpr (OUT == 2) {
      const u32x2 w = (u32x2){pack2<DT>(acc[h].x, acc[h].y), pack2<DT>(acc[h].z, acc[h].w)};
      stq16_nt(a.rs16, qi[h], w);
      acc[h] = widen4<DT>(w);
    }
    if constexpr (NORM) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        bad |= nonfinite(acc[h][k]) ? 1u : 0u;
        ss = ss + (double)acc[h][k] * (double)acc[h][k];
      }
    }
  }
}

// OUT == 3's last tile, which may end inside: one quad at a time, in the
// same order as pass1_quads.  It runs in one block per launch, and as a loop
// the compiler cannot fold the full tiles' straight-line code into it.
template <int NR, int DT, int OUT, bool NORM, int Q>
__device__ __forceinline__ void pass1_last(const Pass1Args& a, int nr, int64_t nq, int64_t q0,
                                           double& ss, uint32_t& bad) {
#pragma unroll 1
  for (int h = 0; h < Q; ++h)
    pass1_quads<NR, DT, OUT, NORM, 1, false, false>(a, nr, nq, q0 + (int64_t)h * kThreads, ss,
                                                     bad);
}

template <int NR, int DT, int OUT, bool NORM, int Q>
__global__ __launch_bounds__(kThreads) void zf_pass1(Pass1Args a) {
  // the occupancy cap: dynamic LDS (see occupancy_lds) that no lane touches
  // (n is never negative)
  extern __shared__ uint32_t zf_occupancy_lds[];
  if (a.n < 0) zf_occupancy_lds[threadIdx.x] = 0u;
  const int nr = NR > 0 ? NR : a.nr;
  const int64_t nq = a.n / kQuad;
  const int64_t tile = tile_of_block(a.tile_map);
  const int64_t q0 = tile * kThreads * Q + threadIdx.x;
  double ss = 0.0;
  uint32_t bad = 0;
  const bool full = (tile + 1) * kThreads * Q <= nq;
  if constexpr (OUT == 3) {
    if (!full)
      pass1_last<NR, DT, OUT, NORM, Q>(a, nr, nq, q0, ss, bad);
    else if (tile * kThreads * Q >= a.plain_from)  // uniform over the block
      pass1_quads<NR, DT, OUT, NORM, Q, true, true>(a, nr, nq, q0, ss, bad);
    else
      pass1_quads<NR, DT, OUT, NORM, Q, true, false>(a, nr, nq, q0, ss, bad);
  } else {
    if (full)
      pass1_quads<NR, DT, OUT, NORM, Q, true, false>(a, nr, nq, q0, ss, bad);
    else
      pass1_quads<NR, DT, OUT, NORM, Q, false, false>(a, nr, nq, q0, ss, bad);
  }
  const int64_t tail0 = nq * kQuad;
  if (tile == gridDim.x - 1 && (int64_t)threadIdx.x < a.n - tail0) {
    const int64_t p = tail0 + threadIdx.x;
    float t = sum1<DT>(a.g, nr, p);
    if constexpr (stores_fp32(OUT)) a.rs[p] = t;
    if constexpr (OUT == 2) {
      const uint16_t q = narrow1<DT>(t);
      a.rs16[p] = q;
      t = widen1<DT>(q);
    }
    if constexpr (NORM) {
      bad |= nonfinite(t) ? 1u : 0u;
      ss = ss + (double)t * (double)t;
    }
  }
  if constexpr (NORM) {
    block_reduce(ss, bad);
    if (threadIdx.x == 0) {
      a.partials[tile].ss = ss;
      a.partials[tile].bad = bad;
    }
  }
}

// Pass 1 over gradients that are already reduced (and accumulated): the
// fp32 gradient shards are only read, for the overflow flag and the
// squared-norm partials, over the same tiles as zf_pass1.  Non-temporal
// loads, as in zf_pass1 (654M bucketed: -14% against plain loads).
template <int Q>
__global__ __launch_bounds__(kThreads) void zf_pass1_reduced(Pass1Args a) {
  const int64_t nq = a.n / kQuad;
  const int64_t tile = tile_of_block(a.tile_map);
  const int64_t q0 = tile * kThreads * Q + threadIdx.x;
  f32x4 acc[Q];
  bool ok[Q];
#pragma unroll
  for (int h = 0; h < Q; ++h) {
    const int64_t q = q0 + (int64_t)h * kThreads;
    ok[h] = q < nq;
    acc[h] = ok[h] ? ldq32<true>(a.rs, q) : (f32x4){0, 0, 0, 0};
  }
  double ss = 0.0;
  uint32_t bad = 0;
#pragma unroll
  for (int h = 0; h < Q; ++h) {
    if (!ok[h]) continue;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      bad |= nonfinite(acc[h][k]) ? 1u : 0u;
      ss = ss + (double)acc[h][k] * (double)acc[h][k];
    }
  }
  const int64_t tail0 = nq * kQuad;
  if (tile == gridDim.x - 1 && (int64_t)threadIdx.x < a.n - tail0) {
    const float t = a.rs[tail0 + threadIdx.x];
    bad |= nonfinite(t) ? 1u : 0u;
    ss = ss + (double)t * (double)t;
  }
  block_reduce(ss, bad);
  if (threadIdx.x == 0) {
    a.partials[tile].ss = ss;
    a.partials[tile].bad = bad;
  }
}

// Level 2: block b reduces the tile partials [b*T/G, (b+1)*T/G) in order.
struct Level2Args {
  const Partial* in;
  Partial* out;
  int64_t n_in;
};

__global__ __launch_bounds__(kThreads) void zf_level2(Level2Args a) {
  const int64_t G = gridDim.x;
  const int64_t lo = a.n_in * (int64_t)blockIdx.x / G;
  const int64_t hi = a.n_in * ((int64_t)blockIdx.x + 1) / G;
  double ss = 0.0;
  uint32_t bad = 0;
  for (int64_t i = lo + threadIdx.x; i < hi; i += kThreads) {
    ss = ss + a.in[i].ss;
    bad = bad | a.in[i].bad;
  }
  block_reduce(ss, bad);
  if (threadIdx.x == 0) {
    a.out[blockIdx.x].ss = ss;
    a.out[blockIdx.x].bad = bad;
  }
}

// ---------------------------------------------------------------------------
// Finish: one block turns the partials into the step's scalars.
struct FinishArgs {
  const Partial* partials;
  DevState* st;
  double beta1, beta2, max_norm;
  int32_t np, n_ranks;
};

// The step's scalars from the total squared norm and the overflow bits
// (one thread).
__device__ __forceinline__ void finish_state(const FinishArgs& a, double ss, uint32_t bad) {
  DevState* s = a.st;
  s->overflow = bad ? 1 : 0;
  s->sumsq = ss;
  s->scale_used = s->loss_scale;
  if (bad) {
    // overflow: skip; a dynamic loss scale halves and its counter restarts
    s->skipped = 1;
    if (s->dynamic) {
      s->loss_scale = s->loss_scale * 0.5;
      s->growth_ctr = 0;
    }
    s->norm = 0.0;
    s->coef = 0.0;
    s->gs = 0.0f;
    return;
  }
  s->skipped = 0;
  const double S = s->loss_scale;
  s->t = s->t + 1;
  s->growth_ctr = s->growth_ctr + 1;
  if (s->dynamic && s->growth_interval > 0 && s->growth_ctr >= s->growth_interval) {
    s->loss_scale = S * 2.0;
    s->growth_ctr = 0;
  }
  const double sn = S * (double)a.n_ranks;
  const double norm = sqrt(ss) / sn;
  double coef = 1.0;
  if (a.max_norm > 0.0) {
    coef = a.max_norm / (norm + 1e-6);
    if (coef > 1.0) coef = 1.0;
  }
  s->beta1_pow = s->beta1_pow * a.beta1;
  s->beta2_pow = s->beta2_pow * a.beta2;
  s->norm = norm;
  s->coef = coef;
  s->gs = (float)(coef / sn);
  s->bc1 = (float)(1.0 - s->beta1_pow);
  s->bc2 = (float)(1.0 - s->beta2_pow);
}

__global__ __launch_bounds__(kThreads) void zf_finish(FinishArgs a) {
  double ss = 0.0;
  uint32_t bad = 0;
  for (int i = threadIdx.x; i < a.np; i += kThreads) {
    ss = ss + a.partials[i].ss;
    bad = bad | a.partials[i].bad;
  }
  block_reduce(ss, bad);
  if (threadIdx.x == 0) finish_state(a, ss, bad);
}

// Level 2 and the finish in one launch, for plans whose norm reduction has
// a single level-2 block: that block reduces every tile partial in the
// order zf_level2 does and finishes.  The result is the same bits as the
// two launches, whose finish would add zeros to the one level-2 partial.
__global__ __launch_bounds__(kThreads) void zf_level2_finish(Level2Args l, FinishArgs a) {
  double ss = 0.0;
  uint32_t bad = 0;
  for (int64_t i = threadIdx.x; i < l.n_in; i += kThreads) {
    ss = ss + l.in[i].ss;
    bad = bad | l.in[i].bad;
  }
  block_reduce(ss, bad);
  if (threadIdx.x == 0) finish_state(a, ss, bad);
}

// ---------------------------------------------------------------------------
// Pass 2: fused unscale/clip + AdamW + RNE cast + gathered write.
struct Pass2Args {
  GradPtrs g;
  const float* rs;
  float* master;
  float* m;
  float* v;
  void* out;
  const DevState* st;
  int64_t n;
  float dec, b1, c1, b2, c2, lrf, ef;
  int32_t nr;
  int32_t reverse;  // MAT: 1 if block b takes tile gridDim.x - 1 - b (cached sums first)
};

struct Coef {
  float gs, dec, b1, c1, b2, c2, bc1, bc2, lrf, ef;
};

__device__ __forceinline__ void adamw1(const Coef& c, float acc, float& p, float& m, float& v) {
  const float g = acc * c.gs;
  float pp = p * c.dec;
  const float mm = c.b1 * m + c.c1 * g;
  const float vv = c.b2 * v + c.c2 * (g * g);
  const float d = sqrtf(vv / c.bc2) + c.ef;
  const float mh = mm / c.bc1;
  pp = pp - c.lrf * (mh / d);
  p = pp;
  m = mm;
  v = vv;
}

template <int NR, int GDT, int PDT, bool MAT, int Q, bool OUT16>
__global__ __launch_bounds__(zf::kThreadsPass2Mat) void zf_pass2(Pass2Args a) {
  constexpr int T = zf::threads_pass2(MAT);  // the block size
  // the occupancy cap: dynamic LDS (see occupancy_lds) that no lane touches
  // (n is never negative)
  extern __shared__ uint32_t zf_occupancy_lds[];
  if (a.n < 0) zf_occupancy_lds[threadIdx.x] = 0u;
  if (a.st->skipped) return;  // the whole grid leaves at once
  Coef c;
  c.gs = a.st->gs;
  c.bc1 = a.st->bc1;
  c.bc2 = a.st->bc2;
  c.dec = a.dec; c.b1 = a.b1; c.c1 = a.c1; c.b2 = a.b2; c.c2 = a.c2;
  c.lrf = a.lrf; c.ef = a.ef;
  const int nr = NR > 0 ? NR : a.nr;
  const int64_t nq = a.n / kQuad;
  const int64_t tile =
      (MAT && a.reverse) ? (int64_t)gridDim.x - 1 - blockIdx.x : (int64_t)blockIdx.x;
  const int64_t q0 = tile * T * Q + threadIdx.x;
  int64_t qi[Q];
  bool ok[Q];
#pragma unroll
  for (int h = 0; h < Q; ++h) {
    qi[h] = q0 + (int64_t)h * T;
    ok[h] = qi[h] < nq;
  }
  f32x4 acc[Q], p[Q], m[Q], v[Q];
  if constexpr (MAT) {
#pragma unroll
    for (int h = 0; h < Q; ++h) acc[h] = ok[h] ? ldq32(a.rs, qi[h]) : (f32x4){0, 0, 0, 0};
  } else {
    sum_quads<NR, GDT, false, Q>(a.g, nr, qi, ok, acc);
  }
#pragma unroll
  for (int h = 0; h < Q; ++h) {
    if (ok[h]) {
      p[h] = ldq32<true>(a.master, qi[h]);
      m[h] = ldq32<true>(a.m, qi[h]);
      v[h] = ldq32<true>(a.v, qi[h]);
    }
  }
#pragma unroll
  for (int h = 0; h < Q; ++h) {
    if (!ok[h]) continue;
    float pp[4] = {p[h].x, p[h].y, p[h].z, p[h].w};
    float mm[4] = {m[h].x, m[h].y, m[h].z, m[h].w};
    float vv[4] = {v[h].x, v[h].y, v[h].z, v[h].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) adamw1(c, acc[h][k], pp[k], mm[k], vv[k]);
    stq32_nt(a.master, qi[h], (f32x4){pp[0], pp[1], pp[2], pp[3]});
    stq32_nt(a.m, qi[h], (f32x4){mm[0], mm[1], mm[2], mm[3]});
    stq32_nt(a.v, qi[h], (f32x4){vv[0], vv[1], vv[2], vv[3]});
    if constexpr (OUT16)
      stq16_nt(a.out, qi[h], (u32x2){pack2<PDT>(pp[0], pp[1]), pack2<PDT>(pp[2], pp[3])});
  }
  const int64_t tail0 = nq * kQuad;
  if (tile == gridDim.x - 1 && (int64_t)threadIdx.x < a.n - tail0) {
    const int64_t e = tail0 + threadIdx.x;
    const float t = MAT ? a.rs[e] : sum1<GDT>(a.g, nr, e);
    float pe = a.master[e], me = a.m[e], ve = a.v[e];
    adamw1(c, t, pe, me, ve);
    a.master[e] = pe;
    a.m[e] = me;
    a.v[e] = ve;
    if constexpr (OUT16) reinterpret_cast<uint16_t*>(a.out)[e] = narrow1<PDT>(pe);
  }
}

// ---------------------------------------------------------------------------
// State initialisation.
// 64 threads: every byte of the 256-byte block is written (the struct's
// fields, then zeros), so a copied block is fully defined.
__global__ void zf_state_init_kernel(DevState* s, double S, int32_t dynamic, int32_t growth) {
  static_assert(kStateBytes == 64 * sizeof(uint32_t), "one word per thread");
  reinterpret_cast<uint32_t*>(s)[threadIdx.x] = 0u;
  __syncthreads();
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  s->loss_scale = S;
  s->beta1_pow = 1.0;
  s->beta2_pow = 1.0;
  s->t = 0;
  s->growth_ctr = 0;
  s->growth_interval = growth;
  s->dynamic = dynamic ? 1 : 0;
  s->pad0 = 0;
  s->overflow = 0;
  s->skipped = 0;
  s->sumsq = 0.0;
  s->norm = 0.0;
  s->coef = 0.0;
  s->scale_used = S;
  s->gs = 0.0f;
  s->bc1 = 0.0f;
  s->bc2 = 0.0f;
  s->pad1 = 0.0f;
}

// ---------------------------------------------------------------------------
// Host side.

template <int OUT, bool NORM, int U>
void launch_pass1_u(int nr, int32_t dt, dim3 grid, uint32_t lds, hipStream_t s,
                    const Pass1Args& a) {
#define ZF_P1(NRV, DTV) \
  hipLaunchKernelGGL((zf_pass1<NRV, DTV, OUT, NORM, zf::kQuadsPerUnr * U>), grid, dim3(kThreads), \
                     lds, s, a)
#define ZF_P1_DT(NRV) \
  do { if (dt == ZF_BF16) ZF_P1(NRV, ZF_BF16); else ZF_P1(NRV, ZF_F16); } while (0)
  switch (nr) {
    case 1: ZF_P1_DT(1); break;
    case 2: ZF_P1_DT(2); break;
    case 3: ZF_P1_DT(3); break;
    case 4: ZF_P1_DT(4); break;
    case 5: ZF_P1_DT(5); break;
    case 6: ZF_P1_DT(6); break;
    case 7: ZF_P1_DT(7); break;
    case 8: ZF_P1_DT(8); break;
    default: ZF_P1_DT(0); break;
  }
#undef ZF_P1_DT
#undef ZF_P1
}

template <int OUT, bool NORM>
int launch_pass1(const zf_plan* plan, int32_t dt, hipStream_t s, const Pass1Args& a) {
  const dim3 grid((uint32_t)plan->pass1_tiles);
  const int nr = plan->summary.n_ranks;
  const uint32_t lds = zf::occupancy_lds(zf::occ_pass1(nr, OUT != 0));
  if (plan->unr1 == 2) launch_pass1_u<OUT, NORM, 2>(nr, dt, grid, lds, s, a);
  else launch_pass1_u<OUT, NORM, 1>(nr, dt, grid, lds, s, a);
  return hip_ok(hipGetLastError()) ? ZF_OK : ZF_EHIP;
}

template <int GDT, int PDT, bool OUT16>
void launch_pass2_nr(int nr, bool mat, dim3 grid, hipStream_t s, const Pass2Args& a) {
  constexpr int Q = zf::kQuadsPass2;
  const uint32_t lds = zf::occupancy_lds(zf::occ_pass2(mat, a.reverse != 0));
  const dim3 block((uint32_t)zf::threads_pass2(mat));
  if (mat) {
    hipLaunchKernelGGL((zf_pass2<0, GDT, PDT, true, Q, OUT16>), grid, block, lds, s, a);
    return;
  }
#define ZF_P2(NRV) \
  hipLaunchKernelGGL((zf_pass2<NRV, GDT, PDT, false, Q, OUT16>), grid, block, lds, s, a)
  switch (nr) {
    case 1: ZF_P2(1); break;
    case 2: ZF_P2(2); break;
    case 3: ZF_P2(3); break;
    case 4: ZF_P2(4); break;
    case 5: ZF_P2(5); break;
    case 6: ZF_P2(6); break;
    case 7: ZF_P2(7); break;
    case 8: ZF_P2(8); break;
    default: ZF_P2(0); break;
  }
#undef ZF_P2
}

void launch_pass2_dt(int nr, int32_t gdt, int32_t pdt, bool mat, bool out16, dim3 grid,
                     hipStream_t s, const Pass2Args& a) {
  if (!out16) {  // fp32 parameters: no 16-bit copy, the param dtype is unused
    if (gdt == ZF_BF16) launch_pass2_nr<ZF_BF16, ZF_BF16, false>(nr, mat, grid, s, a);
    else launch_pass2_nr<ZF_F16, ZF_BF16, false>(nr, mat, grid, s, a);
    return;
  }
  if (gdt == ZF_BF16) {
    if (pdt == ZF_BF16) launch_pass2_nr<ZF_BF16, ZF_BF16, true>(nr, mat, grid, s, a);
    else launch_pass2_nr<ZF_BF16, ZF_F16, true>(nr, mat, grid, s, a);
  } else {
    if (pdt == ZF_BF16) launch_pass2_nr<ZF_F16, ZF_BF16, true>(nr, mat, grid, s, a);
    else launch_pass2_nr<ZF_F16, ZF_F16, true>(nr, mat, grid, s, a);
  }
}

int launch_pass2(const zf_plan* plan, int32_t gdt, int32_t pdt, bool mat, bool out16,
                 hipStream_t s, const Pass2Args& a) {
  const dim3 grid((uint32_t)zf::pass2_tiles(plan, mat));  // fits: checked by the planner
  const int nr = plan->summary.n_ranks;
  launch_pass2_dt(nr, gdt, pdt, mat, out16, grid, s, a);
  return hip_ok(hipGetLastError()) ? ZF_OK : ZF_EHIP;
}

// The device address of `scratch` on the device that runs `s` (the
// current device for the NULL stream), looked up once per device with that
// device current and kept until the process ends.  No allocation: a fixed
// table, one entry per device ordinal.
constexpr int kMaxDevices = 64;

int noalloc_scratch(hipStream_t s, char** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  if (s) {
    hipDevice_t d = 0;
    if (!hip_ok(hipStreamGetDevice(s, &d))) return ZF_EHIP;
    dev = static_cast<int>(d);
  } else if (!hip_ok(hipGetDevice(&dev))) {
    return ZF_EHIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return ZF_EINVAL;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    int cur = 0;
    if (!hip_ok(hipGetDevice(&cur))) return ZF_EHIP;
    if (cur != dev && !hip_ok(hipSetDevice(dev))) return ZF_EHIP;
    void* p = nullptr;
    const bool found = hip_ok(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (cur != dev) (void)hipSetDevice(cur);
    if (!found || !p) return ZF_EHIP;
    addr[dev] = p;
  }
  *out = static_cast<char*>(addr[dev]);
  return ZF_OK;
}

int record(void* const* ev, int i, hipStream_t s) {
  if (!ev || !ev[i]) return ZF_OK;
  return hip_ok(hipEventRecord(static_cast<hipEvent_t>(ev[i]), s)) ? ZF_OK : ZF_EHIP;
}

}  // namespace


thread_local int zf::last_hip_error = 0;

extern "C" const char* zf_hip_error_name(void) {
  return hipGetErrorName(static_cast<hipError_t>(zf::last_hip_error));
}

extern "C" int64_t zf_state_bytes(void) { return kStateBytes; }

extern "C" int zf_state_init(void* d_state, double loss_scale, int32_t dynamic,
                             int32_t growth_interval, void* stream) {
  if (!d_state || !(loss_scale > 0.0) || loss_scale > 1e300) return ZF_EINVAL;
  if (!aligned16(d_state)) return ZF_EALIGN;
  (void)hipGetLastError();
  hipLaunchKernelGGL(zf_state_init_kernel, dim3(1), dim3(64), 0,
                     static_cast<hipStream_t>(stream), static_cast<DevState*>(d_state),
                     loss_scale, dynamic, growth_interval);
  return hip_ok(hipGetLastError()) ? ZF_OK : ZF_EHIP;
}

int zf::step_enqueue(const zf_plan* plan, const zf_hparams* hp, const zf_step_args* args,
                     void* stream, bool update, bool down16, bool noalloc) {
  if (!valid_plan(plan) || !hp || !args) return ZF_EINVAL;
  const zf_plan_summary& sm = plan->summary;
  if (args->grads_reduced != 0 && args->grads_reduced != 1) return ZF_EINVAL;
  if (args->reserved != 0) return ZF_EINVAL;
  const bool reduced = args->grads_reduced == 1;
  if ((!reduced && !valid_dtype(args->grad_dtype)) || !valid_dtype(args->param_dtype))
    return ZF_EDTYPE;
  if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0) || !(hp->beta2 >= 0.0 && hp->beta2 < 1.0))
    return ZF_EINVAL;
  GradPtrs gp;
  int rc = ZF_OK;
  if (reduced) {
    for (int q = 0; q < ZF_MAX_RANKS; ++q) gp.p[q] = nullptr;
    if (!args->grad_shards) return ZF_EINVAL;
  } else if ((rc = grads_ok(plan, args->grads, gp)) != ZF_OK) {
    return rc;
  }
  void* const bufs[] = {args->state, args->master, args->exp_avg, args->exp_avg_sq};
  for (int i = 0; i < (update ? 4 : 1); ++i) {
    if (!bufs[i]) return ZF_EINVAL;
    if (!aligned16(bufs[i])) return ZF_EALIGN;
  }
  if (!update && !args->grad_shards) return ZF_EINVAL;
  if (down16 && (update || reduced)) return ZF_EINVAL;
  if (args->params && !aligned16(args->params)) return ZF_EALIGN;
  if (args->grad_shards && !aligned16(args->grad_shards)) return ZF_EALIGN;
  if (sm.policy == 2 && !args->grad_shards) return ZF_EINVAL;
  if (args->numel < sm.psi_pad) return ZF_ESIZE;
  if (noalloc) {
    // the static scratch holds the partials, and the fp32 sums only when
    // the plan materialises them and the caller gives no grad_shards
    if (args->workspace || args->workspace_size != 0) return ZF_EINVAL;
    const int64_t need = (plan->ws_rs_offset >= 0 && !args->grad_shards)
                             ? sm.workspace_bytes
                             : plan->ws_partials_bytes;
    if (need > ZF_NOALLOC_SCRATCH_BYTES) return ZF_ESIZE;
  } else if (sm.workspace_bytes > 0) {
    if (!args->workspace) return ZF_EINVAL;
    if (!aligned16(args->workspace)) return ZF_EALIGN;
    if (args->workspace_size < sm.workspace_bytes) return ZF_ESIZE;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(args->workspace);
  // every argument is valid: only now touch the runtime for the scratch
  if (noalloc && (rc = noalloc_scratch(s, &ws)) != ZF_OK) return rc;
  Partial* partials = reinterpret_cast<Partial*>(ws + plan->ws_partials_offset);
  // the sums go to the caller's fp32 gradient shard if given, else to the
  // workspace copy if the plan materialises them, else nowhere (recomputed)
  float* rs = args->grad_shards;
  if (!rs && plan->ws_rs_offset >= 0) rs = reinterpret_cast<float*>(ws + plan->ws_rs_offset);
  const bool mat = rs != nullptr;
  const int nr = sm.n_ranks;

  (void)hipGetLastError();
  if ((rc = record(args->phase_events, 0, s)) != ZF_OK) return rc;

  Pass1Args a1;
  a1.g = gp;
  a1.n = sm.psi_pad;
  a1.rs = rs;
  a1.rs16 = down16 ? reinterpret_cast<uint16_t*>(args->grad_shards) : nullptr;
  a1.partials = partials;
  a1.nr = nr;
  a1.tile_map = plan->pass1_map;
  // sums stored by pass 1 and read back by the update pass: the tail of them
  // stays in the memory-side cache and the update pass starts there
  const bool cached = mat && !reduced && !down16 && update && plan->cached_sums_quads > 0;
  a1.plain_from = cached ? sm.psi_pad / 4 - plan->cached_sums_quads : INT64_MAX;
  if (reduced) {
    const dim3 grid((uint32_t)plan->pass1_tiles);
    if (plan->unr1 == 2)
      hipLaunchKernelGGL(zf_pass1_reduced<zf::kQuadsPerUnr * 2>, grid, dim3(kThreads), 0, s, a1);
    else
      hipLaunchKernelGGL(zf_pass1_reduced<zf::kQuadsPerUnr>, grid, dim3(kThreads), 0, s, a1);
    rc = hip_ok(hipGetLastError()) ? ZF_OK : ZF_EHIP;
  } else {
    if (down16) rc = launch_pass1<2, true>(plan, args->grad_dtype, s, a1);
    else if (cached) rc = launch_pass1<3, true>(plan, args->grad_dtype, s, a1);
    else if (mat) rc = launch_pass1<1, true>(plan, args->grad_dtype, s, a1);
    else rc = launch_pass1<0, true>(plan, args->grad_dtype, s, a1);
  }
  if (rc != ZF_OK) return rc;
  if ((rc = record(args->phase_events, 1, s)) != ZF_OK) return rc;

  Partial* partials2 = reinterpret_cast<Partial*>(ws + plan->ws_partials2_offset);
  Level2Args a2l;
  a2l.in = partials;
  a2l.out = partials2;
  a2l.n_in = plan->pass1_tiles;
  FinishArgs af;
  af.partials = partials2;
  af.st = static_cast<DevState*>(args->state);
  af.beta1 = hp->beta1;
  af.beta2 = hp->beta2;
  af.max_norm = hp->max_norm;
  af.np = plan->level2_blocks;
  af.n_ranks = nr;
  if (plan->level2_blocks == 1) {
    hipLaunchKernelGGL(zf_level2_finish, dim3(1), dim3(kThreads), 0, s, a2l, af);
    if (!hip_ok(hipGetLastError())) return ZF_EHIP;
  } else {
    hipLaunchKernelGGL(zf_level2, dim3((uint32_t)plan->level2_blocks), dim3(kThreads), 0, s,
                       a2l);
    if (!hip_ok(hipGetLastError())) return ZF_EHIP;
    hipLaunchKernelGGL(zf_finish, dim3(1), dim3(kThreads), 0, s, af);
    if (!hip_ok(hipGetLastError())) return ZF_EHIP;
  }
  if ((rc = record(args->phase_events, 2, s)) != ZF_OK) return rc;
  if (!update) return ZF_OK;

  // binary32 hyperparameters, each rounded once from its double value
  const zf::UpdateConsts uc = zf::update_consts(hp);
  Pass2Args a2;
  a2.g = gp;
  a2.rs = rs;
  a2.master = args->master;
  a2.m = args->exp_avg;
  a2.v = args->exp_avg_sq;
  a2.out = args->params;
  a2.st = static_cast<const DevState*>(args->state);
  a2.n = sm.psi_pad;
  a2.dec = uc.dec;
  a2.b1 = uc.b1;
  a2.c1 = uc.c1;
  a2.b2 = uc.b2;
  a2.c2 = uc.c2;
  a2.lrf = uc.lrf;
  a2.ef = uc.ef;
  a2.nr = nr;
  a2.reverse = cached ? 1 : 0;
  // with reduced gradients pass 2 reads grad_shards (mat); the gradient
  // dtype then only names an instantiation
  rc = launch_pass2(plan, reduced ? ZF_BF16 : args->grad_dtype, args->param_dtype, mat,
                    args->params != nullptr, s, a2);
  if (rc != ZF_OK) return rc;
  return record(args->phase_events, 3, s);
}

extern "C" int zf_shard_step(const zf_plan* plan, const zf_hparams* hp,
                             const zf_step_args* args, void* stream) {
  return zf::step_enqueue(plan, hp, args, stream, true, false);
}

extern "C" int zf_shard_step_noalloc(const zf_plan* plan, const zf_hparams* hp,
                                     const zf_step_args* args, void* stream) {
  return zf::step_enqueue(plan, hp, args, stream, true, false, true);
}

extern "C" int zf_reduce_scatter(const zf_plan* plan, int32_t grad_dtype,
                                 const void* const* grads, float* rs_out, int64_t numel,
                                 void* stream) {
  if (!valid_plan(plan) || !rs_out) return ZF_EINVAL;
  if (!valid_dtype(grad_dtype)) return ZF_EDTYPE;
  if (!aligned16(rs_out)) return ZF_EALIGN;
  if (numel < plan->summary.psi_pad) return ZF_ESIZE;
  GradPtrs gp;
  int rc = grads_ok(plan, grads, gp);
  if (rc != ZF_OK) return rc;
  Pass1Args a1;
  a1.g = gp;
  a1.n = plan->summary.psi_pad;
  a1.rs = rs_out;
  a1.partials = nullptr;
  a1.plain_from = INT64_MAX;  // the caller's sums are not read back here
  a1.nr = plan->summary.n_ranks;
  a1.tile_map = plan->pass1_map;
  (void)hipGetLastError();
  a1.rs16 = nullptr;
  return launch_pass1<1, false>(plan, grad_dtype, static_cast<hipStream_t>(stream), a1);
}

extern "C" int zf_read_result(const void* d_state, zf_step_result* out, void* stream) {
  if (!d_state || !out) return ZF_EINVAL;
  DevState h;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!hip_ok(hipMemcpyAsync(&h, d_state, sizeof(h), hipMemcpyDeviceToHost, s)))
    return ZF_EHIP;
  if (!hip_ok(hipStreamSynchronize(s))) return ZF_EHIP;
  out->overflow = h.overflow;
  out->skipped = h.skipped;
  out->t = h.t;
  out->sumsq = h.sumsq;
  out->norm = h.norm;
  out->coef = h.coef;
  out->scale_used = h.scale_used;
  out->scale_next = h.loss_scale;
  out->gs = h.gs;
  out->growth_ctr = h.growth_ctr;
  out->bc1 = h.bc1;
  out->bc2 = h.bc2;
  return ZF_OK;
}
