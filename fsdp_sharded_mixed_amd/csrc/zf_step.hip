// zf_step.hip -- gfx950 kernels and C entry points of the sharded AdamW step.
//
// The step is a stream over the padded flat index p with under one flop per
// byte, so it is bound by HBM bandwidth and uses no matrix cores.  Every
// kernel reads and writes 16 bytes per lane per access (eight 16-bit values
// or four fp32 values), wave64-coalesced, from 16-byte aligned bases.
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

#include <algorithm>
#include <cstdint>
#include <new>
#include <vector>

#include "zf_hip_status.h"
#include "zf_internal.h"

namespace {

using zf::hip_ok;

using zf::kThreads;

using zf::DevState;
using zf::kStateBytes;

struct __align__(16) Partial {
  double ss;
  uint32_t bad;
  uint32_t pad;
};

struct GradPtrs {
  const uint16_t* p[ZF_MAX_RANKS];
};

// Element ownership.  A "quad" is 4 consecutive elements: 16 bytes of an
// fp32 stream, 8 bytes of a 16-bit stream.  A block's tile is 256*Q quads and
// lane t owns quads tile*256*Q + h*256 + t (h < Q): every load or store
// instruction of a wave covers one contiguous span (1 KiB of fp32, 512 B of
// 16-bit values), which keeps whole cache lines per instruction and lets the
// non-temporal stores go out as full lines.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kQuad = 4;

template <bool NT>
__device__ __forceinline__ u32x2 ldq16(const uint16_t* base, int64_t q) {
  const u32x2* p = reinterpret_cast<const u32x2*>(base) + q;
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
__device__ __forceinline__ f32x4 ldq32(const float* base, int64_t q) {
  return reinterpret_cast<const f32x4*>(base)[q];
}
__device__ __forceinline__ void stq32_nt(float* base, int64_t q, f32x4 x) {
  __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(base) + q);
}
__device__ __forceinline__ void stq16_nt(void* base, int64_t q, u32x2 x) {
  __builtin_nontemporal_store(x, reinterpret_cast<u32x2*>(base) + q);
}

// ---------------------------------------------------------------------------
// 16-bit <-> binary32.  Widening is exact; narrowing uses the hardware
// round-to-nearest-even conversions (v_cvt_pk_bf16_f32, v_cvt_f16_f32).

template <int DT>
__device__ __forceinline__ float lo16(uint32_t w) {
  if constexpr (DT == ZF_BF16) return __uint_as_float(w << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
template <int DT>
__device__ __forceinline__ float hi16(uint32_t w) {
  if constexpr (DT == ZF_BF16) return __uint_as_float(w & 0xFFFF0000u);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
template <int DT>
__device__ __forceinline__ float widen1(uint16_t h) {
  return lo16<DT>((uint32_t)h);
}
template <int DT>
__device__ __forceinline__ uint16_t narrow1(float x) {
  if constexpr (DT == ZF_BF16) return __builtin_bit_cast(uint16_t, (__bf16)x);
  else return __builtin_bit_cast(uint16_t, (_Float16)x);
}
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return (uint32_t)narrow1<DT>(a) | ((uint32_t)narrow1<DT>(b) << 16);
}
template <int DT>
__device__ __forceinline__ f32x4 widen4(const u32x2& w) {
  return (f32x4){lo16<DT>(w.x), hi16<DT>(w.x), lo16<DT>(w.y), hi16<DT>(w.y)};
}

__device__ __forceinline__ bool nonfinite(float x) {
  return (__float_as_uint(x) & 0x7F800000u) == 0x7F800000u;
}

// Tile of this block.  Blocks are dispatched to the 8 XCDs round-robin
// (block b on XCD b % 8).  map == 0: tile b, so all XCDs share one moving
// window; map == 1: XCD x walks its own contiguous eighth of the tiles in
// order (faster for pass 1 with few replicas, slower with many).  Partials
// are indexed by tile, so the reduction order does not depend on the map.
__device__ __forceinline__ int64_t tile_of_block(int map) {
  const int64_t b = blockIdx.x;
  if (map == 1) {
    const int64_t G = gridDim.x, m = G / 8, r = G % 8, x = b % 8, k = b / 8;
    return x * m + (x < r ? x : r) + k;
  }
  return b;
}

// Fixed-order sums of the N replicas over a thread's Q quads.
// NR > 0: N known at compile time, all N*Q loads issued before the adds.
// NR == 0: N at run time, in groups of four replicas.
template <int NR, int DT, bool NT, int Q>
__device__ __forceinline__ void sum_quads(const GradPtrs& g, int nr, const int64_t (&qi)[Q],
                                          const bool (&ok)[Q], f32x4 (&acc)[Q]) {
  if constexpr (NR > 0) {
    u32x2 w[NR][Q];
#pragma unroll
    for (int h = 0; h < Q; ++h)
#pragma unroll
      for (int r = 0; r < NR; ++r) w[r][h] = ok[h] ? ldq16<NT>(g.p[r], qi[h]) : (u32x2){0, 0};
#pragma unroll
    for (int h = 0; h < Q; ++h) {
      f32x4 a = widen4<DT>(w[0][h]);
#pragma unroll
      for (int r = 1; r < NR; ++r) a = a + widen4<DT>(w[r][h]);
      acc[h] = a;
    }
  } else {
#pragma unroll
    for (int h = 0; h < Q; ++h)
      acc[h] = widen4<DT>(ok[h] ? ldq16<NT>(g.p[0], qi[h]) : (u32x2){0, 0});
    int r = 1;
    for (; r + 4 <= nr; r += 4) {
      u32x2 w[4][Q];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int h = 0; h < Q; ++h) w[j][h] = ok[h] ? ldq16<NT>(g.p[r + j], qi[h]) : (u32x2){0, 0};
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int h = 0; h < Q; ++h) acc[h] = acc[h] + widen4<DT>(w[j][h]);
    }
    for (; r < nr; ++r)
#pragma unroll
      for (int h = 0; h < Q; ++h)
        acc[h] = acc[h] + widen4<DT>(ok[h] ? ldq16<NT>(g.p[r], qi[h]) : (u32x2){0, 0});
  }
}

// Scalar element p (the ragged tail of < 4 elements).
template <int DT>
__device__ __forceinline__ float sum1(const GradPtrs& g, int nr, int64_t p) {
  float acc = widen1<DT>(g.p[0][p]);
  for (int q = 1; q < nr; ++q) acc = acc + widen1<DT>(g.p[q][p]);
  return acc;
}

// Block-wide reduction of (sum, or): wave64 xor-butterfly (every lane ends
// with the same bits: each level only swaps the operands of an addition),
// then the four waves in order.  The result is valid in thread 0.
__device__ __forceinline__ void block_reduce(double& ss, uint32_t& bad) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    ss = ss + __shfl_xor(ss, off, 64);
    bad = bad | __shfl_xor(bad, off, 64);
  }
  __shared__ double s_ss[kThreads / 64];
  __shared__ uint32_t s_bad[kThreads / 64];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    s_ss[wave] = ss;
    s_bad[wave] = bad;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = s_ss[0];
    uint32_t b = s_bad[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) {
      t = t + s_ss[w];
      b = b | s_bad[w];
    }
    ss = t;
    bad = b;
  }
}

// ---------------------------------------------------------------------------
// Pass 1: reduce-scatter sums, overflow flag and squared-norm partials, one
// tile per block.  The last block also takes the ragged tail (< 4 elements).
struct Pass1Args {
  GradPtrs g;
  int64_t n;          // Psi'
  float* rs;          // fp32 sums (OUT == 1) or unused
  uint16_t* rs16;     // 16-bit sums (OUT == 2) or unused
  Partial* partials;  // one per tile (NORM) or unused
  int32_t nr;
  int32_t tile_map;   // see tile_of_block
};

// OUT: 0 the sums stay in registers; 1 they are stored in fp32; 2 they are
// rounded to the gradient dtype and stored in 16 bits, and the overflow flag
// and the norm are taken on the rounded values (the 16-bit gradients an
// offloaded optimizer receives).
template <int NR, int DT, int OUT, bool NORM, int Q>
__global__ __launch_bounds__(kThreads) void zf_pass1(Pass1Args a) {
  const int nr = NR > 0 ? NR : a.nr;
  const int64_t nq = a.n / kQuad;
  const int64_t tile = tile_of_block(a.tile_map);
  const int64_t q0 = tile * kThreads * Q + threadIdx.x;
  int64_t qi[Q];
  bool ok[Q];
#pragma unroll
  for (int h = 0; h < Q; ++h) {
    qi[h] = q0 + (int64_t)h * kThreads;
    ok[h] = qi[h] < nq;
  }
  f32x4 acc[Q];
  sum_quads<NR, DT, ZF_PASS1_NT_LOADS != 0, Q>(a.g, nr, qi, ok, acc);
  double ss = 0.0;
  uint32_t bad = 0;
#pragma unroll
  for (int h = 0; h < Q; ++h) {
    if (!ok[h]) continue;
    if constexpr (OUT == 1) stq32_nt(a.rs, qi[h], acc[h]);
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
  const int64_t tail0 = nq * kQuad;
  if (tile == gridDim.x - 1 && (int64_t)threadIdx.x < a.n - tail0) {
    const int64_t p = tail0 + threadIdx.x;
    float t = sum1<DT>(a.g, nr, p);
    if constexpr (OUT == 1) a.rs[p] = t;
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
// squared-norm partials, over the same tiles as zf_pass1.
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
    acc[h] = ok[h] ? ldq32(a.rs, q) : (f32x4){0, 0, 0, 0};
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

__global__ __launch_bounds__(kThreads) void zf_finish(FinishArgs a) {
  double ss = 0.0;
  uint32_t bad = 0;
  for (int i = threadIdx.x; i < a.np; i += kThreads) {
    ss = ss + a.partials[i].ss;
    bad = bad | a.partials[i].bad;
  }
  block_reduce(ss, bad);
  if (threadIdx.x != 0) return;
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
__global__ __launch_bounds__(kThreads) void zf_pass2(Pass2Args a) {
  if (a.st->skipped) return;  // the whole grid leaves at once
  Coef c;
  c.gs = a.st->gs;
  c.bc1 = a.st->bc1;
  c.bc2 = a.st->bc2;
  c.dec = a.dec; c.b1 = a.b1; c.c1 = a.c1; c.b2 = a.b2; c.c2 = a.c2;
  c.lrf = a.lrf; c.ef = a.ef;
  const int nr = NR > 0 ? NR : a.nr;
  const int64_t nq = a.n / kQuad;
  const int64_t tile = blockIdx.x;
  const int64_t q0 = tile * kThreads * Q + threadIdx.x;
  int64_t qi[Q];
  bool ok[Q];
#pragma unroll
  for (int h = 0; h < Q; ++h) {
    qi[h] = q0 + (int64_t)h * kThreads;
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
      p[h] = ldq32(a.master, qi[h]);
      m[h] = ldq32(a.m, qi[h]);
      v[h] = ldq32(a.v, qi[h]);
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
// Unit gather: blockIdx.y = rank; unit_buf[r*S + j] = src_r[j].
struct GatherArgs {
  const uint16_t* src[ZF_MAX_RANKS];
  uint16_t* dst;
  int64_t S;
};

__global__ __launch_bounds__(kThreads) void zf_gather_kernel(GatherArgs a) {
  const int r = blockIdx.y;
  const uint16_t* s = a.src[r];
  uint16_t* d = a.dst + (int64_t)r * a.S;
  const int64_t S = a.S;
  const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const uintptr_t ms = reinterpret_cast<uintptr_t>(s) & 15u;
  const uintptr_t md = reinterpret_cast<uintptr_t>(d) & 15u;
  if (ms == md) {
    // same misalignment: a scalar head up to the 16-byte boundary, 16-byte
    // copies, then a scalar tail
    int64_t head = (int64_t)(((16u - ms) & 15u) >> 1);
    if (head > S) head = S;
    const int64_t nvec = (S - head) / 8;
    const uint4* s4 = reinterpret_cast<const uint4*>(s + head);
    uint4* d4 = reinterpret_cast<uint4*>(d + head);
    for (int64_t v = tid; v < nvec; v += stride) d4[v] = s4[v];
    const int64_t tail0 = head + nvec * 8;
    if (tid < head) d[tid] = s[tid];
    if (tid < S - tail0) d[tail0 + tid] = s[tail0 + tid];
  } else {
    for (int64_t j = tid; j < S; j += stride) d[j] = s[j];
  }
}

// ---------------------------------------------------------------------------
// FSDP2 unshard: cast each parameter's fp32 shards (padded-flat [O_u,
// O_u + L_u): the N ranks' chunks side by side, padding rows excluded) to
// 16 bits into the group buffer at the parameter's unpadded offset.
// blockIdx.y = parameter of this launch; blockIdx.x = 2048-element tile.
constexpr int kCastMax = 32;  // parameters per launch
struct CastEntry {
  int64_t src;  // O_u in the fp32 array
  int64_t dst;  // offset in the group buffer
  int64_t len;  // L_u
};
struct CastArgs {
  const float* master;
  uint16_t* out;
  CastEntry e[kCastMax];
};

template <int DT>
__global__ __launch_bounds__(kThreads) void zf_gather_cast_kernel(CastArgs a) {
  const CastEntry e = a.e[blockIdx.y];
  const int64_t t0 = (int64_t)blockIdx.x * kThreads * 8;
  if (t0 >= e.len) return;
  const float* src = a.master + e.src;
  uint16_t* dst = a.out + e.dst;
  const bool vec = (e.src % 4 == 0) && ((reinterpret_cast<uintptr_t>(dst) & 7u) == 0);
  if (vec) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t q = t0 / 4 + h * kThreads + threadIdx.x;
      const int64_t e0 = 4 * q;
      if (e0 + 4 <= e.len) {
        const f32x4 x = reinterpret_cast<const f32x4*>(src)[q];
        reinterpret_cast<u32x2*>(dst)[q] = (u32x2){pack2<DT>(x.x, x.y), pack2<DT>(x.z, x.w)};
      } else {
        for (int64_t k = e0; k < e.len && k < e0 + 4; ++k) dst[k] = narrow1<DT>(src[k]);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t i = t0 + (int64_t)k * kThreads + threadIdx.x;
      if (i < e.len) dst[i] = narrow1<DT>(src[i]);
    }
  }
}

// ---------------------------------------------------------------------------
// Bucket reduce-scatter with accumulation over the element range [e0, e1)
// of the padded flat.  The 16-byte aligned quads [qa, qa + nq) go through
// the tiled vector path; the head [e0, 4*qa) and tail [tail0, e1) (under
// four elements each, or a whole range shorter than two quads) are done by
// block 0's first lanes.  Replicas are 16-bit or fp32 (DT == ZF_F32).

template <int DT, bool NT>
__device__ __forceinline__ f32x4 ldg4(const void* base, int64_t q) {
  if constexpr (DT == ZF_F32) {
    const f32x4* p = reinterpret_cast<const f32x4*>(base) + q;
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
  } else {
    return widen4<DT>(ldq16<NT>(static_cast<const uint16_t*>(base), q));
  }
}
template <int DT>
__device__ __forceinline__ float ldg1(const void* base, int64_t p) {
  if constexpr (DT == ZF_F32) return static_cast<const float*>(base)[p];
  else return widen1<DT>(static_cast<const uint16_t*>(base)[p]);
}

struct BucketArgs {
  const void* g[ZF_MAX_RANKS];
  float* out;
  int64_t qa, nq;        // aligned quads
  int64_t e0, head;      // scalar head [e0, e0 + head)
  int64_t tail0, tail;   // scalar tail [tail0, tail0 + tail)
  int32_t nr;
};

template <int NR, int DT, bool ACC, int Q>
__global__ __launch_bounds__(kThreads) void zf_bucket_rs_kernel(BucketArgs a) {
  const int nr = NR > 0 ? NR : a.nr;
  const int64_t q0 = a.qa + (int64_t)blockIdx.x * kThreads * Q + threadIdx.x;
  const int64_t qend = a.qa + a.nq;
  int64_t qi[Q];
  bool ok[Q];
#pragma unroll
  for (int h = 0; h < Q; ++h) {
    qi[h] = q0 + (int64_t)h * kThreads;
    ok[h] = qi[h] < qend;
  }
  f32x4 acc[Q];
  if constexpr (NR > 0) {
    f32x4 w[NR][Q];
#pragma unroll
    for (int h = 0; h < Q; ++h)
#pragma unroll
      for (int r = 0; r < NR; ++r) w[r][h] = ok[h] ? ldg4<DT, true>(a.g[r], qi[h]) : (f32x4){0, 0, 0, 0};
#pragma unroll
    for (int h = 0; h < Q; ++h) {
      f32x4 t = w[0][h];
#pragma unroll
      for (int r = 1; r < NR; ++r) t = t + w[r][h];
      acc[h] = t;
    }
  } else {
#pragma unroll
    for (int h = 0; h < Q; ++h) acc[h] = ok[h] ? ldg4<DT, true>(a.g[0], qi[h]) : (f32x4){0, 0, 0, 0};
    for (int r = 1; r < nr; ++r)
#pragma unroll
      for (int h = 0; h < Q; ++h)
        acc[h] = acc[h] + (ok[h] ? ldg4<DT, true>(a.g[r], qi[h]) : (f32x4){0, 0, 0, 0});
  }
#pragma unroll
  for (int h = 0; h < Q; ++h) {
    if (!ok[h]) continue;
    f32x4 o = acc[h];
    if constexpr (ACC) o = ldq32(a.out, qi[h]) + o;
    stq32_nt(a.out, qi[h], o);
  }
  if (blockIdx.x == 0) {
    const int64_t t = threadIdx.x;
    int64_t p = -1;
    if (t < a.head) p = a.e0 + t;
    else if (t < a.head + a.tail) p = a.tail0 + (t - a.head);
    if (p >= 0) {
      float sum = ldg1<DT>(a.g[0], p);
      for (int r = 1; r < nr; ++r) sum = sum + ldg1<DT>(a.g[r], p);
      a.out[p] = ACC ? a.out[p] + sum : sum;
    }
  }
}

// Local accumulation acc[i] (+)= f32(grad[i]), i < n.  vec: acc + head is
// 16-byte aligned and grad + head 8-byte aligned, so the nq quads after the
// head are vector accesses; otherwise every element is scalar.
struct AccArgs {
  const uint16_t* g;
  float* acc;
  int64_t n, head, nq;
  int32_t vec;
};

template <int DT, bool ACC>
__global__ __launch_bounds__(kThreads) void zf_accumulate_kernel(AccArgs a) {
  constexpr int Q = 4;
  if (a.vec) {
    const uint16_t* g = a.g + a.head;
    float* o = a.acc + a.head;
    const int64_t q0 = (int64_t)blockIdx.x * kThreads * Q + threadIdx.x;
#pragma unroll
    for (int h = 0; h < Q; ++h) {
      const int64_t q = q0 + (int64_t)h * kThreads;
      if (q < a.nq) {
        f32x4 x = widen4<DT>(ldq16<true>(g, q));
        if constexpr (ACC) x = ldq32(o, q) + x;
        stq32_nt(o, q, x);
      }
    }
    if (blockIdx.x == 0) {
      const int64_t tail0 = a.head + a.nq * kQuad;
      const int64_t t = threadIdx.x;
      int64_t i = -1;
      if (t < a.head) i = t;
      else if (t < a.head + (a.n - tail0)) i = tail0 + (t - a.head);
      if (i >= 0) {
        const float x = widen1<DT>(a.g[i]);
        a.acc[i] = ACC ? a.acc[i] + x : x;
      }
    }
  } else {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < a.n; i += stride) {
      const float x = widen1<DT>(a.g[i]);
      a.acc[i] = ACC ? a.acc[i] + x : x;
    }
  }
}

// ---------------------------------------------------------------------------
// Resharding: copy (or zero) a batch of element runs.  blockIdx.y = run;
// the blocks of grid.x stride over the run's elements.
constexpr int kReshardMax = 64;
struct ReshardRun {
  int64_t src;  // element offset in the source, or -1: write zeros
  int64_t dst;  // element offset in the destination
  int64_t len;
};
struct ReshardArgs {
  const void* src;
  void* dst;
  ReshardRun r[kReshardMax];
};

template <typename T>
__global__ __launch_bounds__(kThreads) void zf_reshard_kernel(ReshardArgs a) {
  const ReshardRun run = a.r[blockIdx.y];
  const T* s = static_cast<const T*>(a.src);
  T* d = static_cast<T*>(a.dst) + run.dst;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < run.len; i += stride)
    d[i] = run.src < 0 ? T(0) : s[run.src + i];
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

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool valid_dtype(int32_t d) { return d == ZF_F16 || d == ZF_BF16; }
bool valid_plan(const zf_plan* p) { return p && p->magic == zf::kPlanMagic; }

int grads_ok(const zf_plan* plan, const void* const* grads, GradPtrs& out) {
  if (!grads) return ZF_EINVAL;
  for (int q = 0; q < plan->summary.n_ranks; ++q) {
    if (!grads[q]) return ZF_EINVAL;
    if (!aligned16(grads[q])) return ZF_EALIGN;
    out.p[q] = static_cast<const uint16_t*>(grads[q]);
  }
  for (int q = plan->summary.n_ranks; q < ZF_MAX_RANKS; ++q) out.p[q] = nullptr;
  return ZF_OK;
}

template <int OUT, bool NORM, int U>
void launch_pass1_u(int nr, int32_t dt, dim3 grid, hipStream_t s, const Pass1Args& a) {
#define ZF_P1(NRV, DTV) \
  hipLaunchKernelGGL((zf_pass1<NRV, DTV, OUT, NORM, zf::kQuadsPerUnr * U>), grid, dim3(kThreads), 0, s, a)
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
  if (plan->unr1 == 2) launch_pass1_u<OUT, NORM, 2>(nr, dt, grid, s, a);
  else launch_pass1_u<OUT, NORM, 1>(nr, dt, grid, s, a);
  return hip_ok(hipGetLastError()) ? ZF_OK : ZF_EHIP;
}

template <int GDT, int PDT, int U, bool OUT16>
void launch_pass2_nr(int nr, bool mat, dim3 grid, hipStream_t s, const Pass2Args& a) {
  constexpr int Q = zf::kQuadsPerUnr * U;
  if (mat) {
    hipLaunchKernelGGL((zf_pass2<0, GDT, PDT, true, Q, OUT16>), grid, dim3(kThreads), 0, s, a);
    return;
  }
#define ZF_P2(NRV) \
  hipLaunchKernelGGL((zf_pass2<NRV, GDT, PDT, false, Q, OUT16>), grid, dim3(kThreads), 0, s, a)
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

template <int U>
void launch_pass2_u(int nr, int32_t gdt, int32_t pdt, bool mat, bool out16, dim3 grid,
                    hipStream_t s, const Pass2Args& a) {
  if (!out16) {  // fp32 parameters: no 16-bit copy, the param dtype is unused
    if (gdt == ZF_BF16) launch_pass2_nr<ZF_BF16, ZF_BF16, U, false>(nr, mat, grid, s, a);
    else launch_pass2_nr<ZF_F16, ZF_BF16, U, false>(nr, mat, grid, s, a);
    return;
  }
  if (gdt == ZF_BF16) {
    if (pdt == ZF_BF16) launch_pass2_nr<ZF_BF16, ZF_BF16, U, true>(nr, mat, grid, s, a);
    else launch_pass2_nr<ZF_BF16, ZF_F16, U, true>(nr, mat, grid, s, a);
  } else {
    if (pdt == ZF_BF16) launch_pass2_nr<ZF_F16, ZF_BF16, U, true>(nr, mat, grid, s, a);
    else launch_pass2_nr<ZF_F16, ZF_F16, U, true>(nr, mat, grid, s, a);
  }
}

int launch_pass2(const zf_plan* plan, int32_t gdt, int32_t pdt, bool mat, bool out16,
                 hipStream_t s, const Pass2Args& a) {
  const dim3 grid((uint32_t)plan->pass2_tiles);
  const int nr = plan->summary.n_ranks;
  if (plan->unr2 == 2) launch_pass2_u<2>(nr, gdt, pdt, mat, out16, grid, s, a);
  else launch_pass2_u<1>(nr, gdt, pdt, mat, out16, grid, s, a);
  return hip_ok(hipGetLastError()) ? ZF_OK : ZF_EHIP;
}

template <bool ACC, int Q>
void launch_bucket_nr(int nr, int32_t dt, dim3 grid, hipStream_t s, const BucketArgs& a) {
#define ZF_BK(NRV, DTV) \
  hipLaunchKernelGGL((zf_bucket_rs_kernel<NRV, DTV, ACC, Q>), grid, dim3(kThreads), 0, s, a)
#define ZF_BK_DT(NRV)                                    \
  do {                                                   \
    if (dt == ZF_BF16) ZF_BK(NRV, ZF_BF16);              \
    else if (dt == ZF_F16) ZF_BK(NRV, ZF_F16);           \
    else ZF_BK(NRV, ZF_F32);                             \
  } while (0)
  switch (nr) {
    case 1: ZF_BK_DT(1); break;
    case 2: ZF_BK_DT(2); break;
    case 3: ZF_BK_DT(3); break;
    case 4: ZF_BK_DT(4); break;
    case 5: ZF_BK_DT(5); break;
    case 6: ZF_BK_DT(6); break;
    case 7: ZF_BK_DT(7); break;
    case 8: ZF_BK_DT(8); break;
    default: ZF_BK_DT(0); break;
  }
#undef ZF_BK_DT
#undef ZF_BK
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
                     void* stream, bool update, bool down16) {
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
  if (sm.workspace_bytes > 0) {
    if (!args->workspace) return ZF_EINVAL;
    if (!aligned16(args->workspace)) return ZF_EALIGN;
    if (args->workspace_size < sm.workspace_bytes) return ZF_ESIZE;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(args->workspace);
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
  if (reduced) {
    const dim3 grid((uint32_t)plan->pass1_tiles);
    if (plan->unr1 == 2)
      hipLaunchKernelGGL(zf_pass1_reduced<zf::kQuadsPerUnr * 2>, grid, dim3(kThreads), 0, s, a1);
    else
      hipLaunchKernelGGL(zf_pass1_reduced<zf::kQuadsPerUnr>, grid, dim3(kThreads), 0, s, a1);
    rc = hip_ok(hipGetLastError()) ? ZF_OK : ZF_EHIP;
  } else {
    if (down16) rc = launch_pass1<2, true>(plan, args->grad_dtype, s, a1);
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
  hipLaunchKernelGGL(zf_level2, dim3((uint32_t)plan->level2_blocks), dim3(kThreads), 0, s, a2l);
  if (!hip_ok(hipGetLastError())) return ZF_EHIP;

  FinishArgs af;
  af.partials = partials2;
  af.st = static_cast<DevState*>(args->state);
  af.beta1 = hp->beta1;
  af.beta2 = hp->beta2;
  af.max_norm = hp->max_norm;
  af.np = plan->level2_blocks;
  af.n_ranks = nr;
  hipLaunchKernelGGL(zf_finish, dim3(1), dim3(kThreads), 0, s, af);
  if (!hip_ok(hipGetLastError())) return ZF_EHIP;
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
  a1.nr = plan->summary.n_ranks;
  a1.tile_map = plan->pass1_map;
  (void)hipGetLastError();
  a1.rs16 = nullptr;
  return launch_pass1<1, false>(plan, grad_dtype, static_cast<hipStream_t>(stream), a1);
}

extern "C" int zf_bucket_reduce_scatter(const zf_plan* plan, int64_t group, int32_t grad_dtype,
                                        const void* const* grads, float* grad_shards,
                                        int64_t numel, int32_t accumulate, void* stream) {
  if (!valid_plan(plan) || !grads || !grad_shards) return ZF_EINVAL;
  if (!valid_dtype(grad_dtype) && grad_dtype != ZF_F32) return ZF_EDTYPE;
  if (accumulate != 0 && accumulate != 1) return ZF_EINVAL;
  if (group < 0 || group >= (int64_t)plan->groups.size()) return ZF_EINVAL;
  if (!aligned16(grad_shards)) return ZF_EALIGN;
  if (numel < plan->summary.psi_pad) return ZF_ESIZE;
  const int nr = plan->summary.n_ranks;
  BucketArgs a;
  for (int q = 0; q < ZF_MAX_RANKS; ++q) a.g[q] = nullptr;
  for (int q = 0; q < nr; ++q) {
    if (!grads[q]) return ZF_EINVAL;
    if (!aligned16(grads[q])) return ZF_EALIGN;
    a.g[q] = grads[q];
  }
  const zf_group_info& g = plan->groups[group];
  const int64_t e0 = plan->units[g.first_unit].O;
  const int64_t e1 = e0 + g.padded;
  const int64_t qa = (e0 + kQuad - 1) / kQuad, qb = e1 / kQuad;
  a.out = grad_shards;
  a.e0 = e0;
  a.nr = nr;
  if (qb > qa) {
    a.qa = qa;
    a.nq = qb - qa;
    a.head = qa * kQuad - e0;
    a.tail0 = qb * kQuad;
    a.tail = e1 - a.tail0;
  } else {  // shorter than two quads: all scalar
    a.qa = 0;
    a.nq = 0;
    a.head = e1 - e0;
    a.tail0 = e1;
    a.tail = 0;
  }
  constexpr int Q = 2;
  int64_t bx = (a.nq + (int64_t)kThreads * Q - 1) / ((int64_t)kThreads * Q);
  if (bx < 1) bx = 1;
  if (bx > 0x7FFFFFFF) return ZF_ESIZE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (accumulate) launch_bucket_nr<true, Q>(nr, grad_dtype, dim3((uint32_t)bx), s, a);
  else launch_bucket_nr<false, Q>(nr, grad_dtype, dim3((uint32_t)bx), s, a);
  return hip_ok(hipGetLastError()) ? ZF_OK : ZF_EHIP;
}

extern "C" int zf_accumulate(int32_t grad_dtype, const void* grad, float* acc, int64_t n,
                             int32_t accumulate, void* stream) {
  if (!grad || !acc || n < 0) return ZF_EINVAL;
  if (!valid_dtype(grad_dtype)) return ZF_EDTYPE;
  if (accumulate != 0 && accumulate != 1) return ZF_EINVAL;
  const uintptr_t ga = reinterpret_cast<uintptr_t>(grad), aa = reinterpret_cast<uintptr_t>(acc);
  if ((ga & 1u) != 0 || (aa & 3u) != 0) return ZF_EALIGN;
  if (n == 0) return ZF_OK;
  AccArgs a;
  a.g = static_cast<const uint16_t*>(grad);
  a.acc = acc;
  a.n = n;
  int64_t head = (int64_t)(((16u - (aa & 15u)) & 15u) / 4u);
  if (head > n) head = n;
  a.head = head;
  a.vec = ((ga + 2u * (uintptr_t)head) & 7u) == 0 ? 1 : 0;
  a.nq = a.vec ? (n - head) / kQuad : 0;
  int64_t bx;
  if (a.vec) {
    bx = (a.nq + (int64_t)kThreads * 4 - 1) / ((int64_t)kThreads * 4);
  } else {
    bx = (n + (int64_t)kThreads * 8 - 1) / ((int64_t)kThreads * 8);
    if (bx > 65536) bx = 65536;
  }
  if (bx < 1) bx = 1;
  if (bx > 0x7FFFFFFF) return ZF_ESIZE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const dim3 grid((uint32_t)bx);
  if (grad_dtype == ZF_BF16) {
    if (accumulate) hipLaunchKernelGGL((zf_accumulate_kernel<ZF_BF16, true>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((zf_accumulate_kernel<ZF_BF16, false>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (accumulate) hipLaunchKernelGGL((zf_accumulate_kernel<ZF_F16, true>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((zf_accumulate_kernel<ZF_F16, false>), grid, dim3(kThreads), 0, s, a);
  }
  return hip_ok(hipGetLastError()) ? ZF_OK : ZF_EHIP;
}

namespace {

// Real runs of a plan in logical order: (logical start, padded offset, len),
// plus the padding runs (offset, len).
struct Run {
  int64_t lam, off, len;
};
void plan_runs(const zf_plan* p, std::vector<Run>& real, std::vector<Run>& pad) {
  const int nr = p->summary.n_ranks;
  for (const zf_unit_info& u : p->units)
    for (int r = 0; r < nr; ++r) {
      int64_t len = u.L - (int64_t)r * u.S;
      if (len < 0) len = 0;
      if (len > u.S) len = u.S;
      const int64_t off = u.O + (int64_t)r * u.S;
      if (len > 0) real.push_back(Run{u.lam + (int64_t)r * u.S, off, len});
      if (len < u.S) pad.push_back(Run{-1, off + len, u.S - len});
    }
}

}  // namespace

extern "C" int zf_reshard(const zf_plan* from, const zf_plan* to, const void* src,
                          int64_t src_numel, void* dst, int64_t dst_numel, int32_t elem_bytes,
                          void* stream) {
  if (!valid_plan(from) || !valid_plan(to) || !src || !dst) return ZF_EINVAL;
  if (elem_bytes != 2 && elem_bytes != 4) return ZF_EINVAL;
  if (from->summary.psi != to->summary.psi) return ZF_EINVAL;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) &
      (uintptr_t)(elem_bytes - 1))
    return ZF_EALIGN;
  if (src_numel < from->summary.psi_pad || dst_numel < to->summary.psi_pad) return ZF_ESIZE;
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  const uintptr_t s1 = s0 + (uintptr_t)from->summary.psi_pad * elem_bytes;
  const uintptr_t d1 = d0 + (uintptr_t)to->summary.psi_pad * elem_bytes;
  if (s0 < d1 && d0 < s1) return ZF_EINVAL;  // overlapping arrays
  std::vector<ReshardRun> runs;
  try {
    std::vector<Run> ra, rb, pa, pb;
    plan_runs(from, ra, pa);
    plan_runs(to, rb, pb);
    // merge the two logical orders: each overlap of a source run and a
    // destination run is one copy
    size_t i = 0, j = 0;
    while (i < ra.size() && j < rb.size()) {
      const int64_t lo = std::max(ra[i].lam, rb[j].lam);
      const int64_t hi = std::min(ra[i].lam + ra[i].len, rb[j].lam + rb[j].len);
      if (lo < hi)
        runs.push_back(ReshardRun{ra[i].off + (lo - ra[i].lam), rb[j].off + (lo - rb[j].lam),
                                  hi - lo});
      if (ra[i].lam + ra[i].len < rb[j].lam + rb[j].len) ++i;
      else ++j;
    }
    for (const Run& p : pb) runs.push_back(ReshardRun{-1, p.off, p.len});
  } catch (const std::bad_alloc&) {
    return ZF_ENOMEM;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  for (size_t first = 0; first < runs.size(); first += kReshardMax) {
    ReshardArgs a;
    a.src = src;
    a.dst = dst;
    const size_t count = std::min<size_t>(kReshardMax, runs.size() - first);
    int64_t longest = 0;
    for (size_t k = 0; k < count; ++k) {
      a.r[k] = runs[first + k];
      longest = std::max(longest, a.r[k].len);
    }
    int64_t bx = (longest + (int64_t)kThreads * 8 - 1) / ((int64_t)kThreads * 8);
    bx = std::min<int64_t>(std::max<int64_t>(bx, 1), 4096);
    const dim3 grid((uint32_t)bx, (uint32_t)count);
    if (elem_bytes == 4)
      hipLaunchKernelGGL(zf_reshard_kernel<uint32_t>, grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL(zf_reshard_kernel<uint16_t>, grid, dim3(kThreads), 0, s, a);
    if (!hip_ok(hipGetLastError())) return ZF_EHIP;
  }
  return ZF_OK;
}

extern "C" int zf_gather(const zf_plan* plan, int64_t unit, int32_t dtype,
                         const void* const* shards, void* unit_buf, int64_t unit_buf_numel,
                         void* stream) {
  if (!valid_plan(plan) || !shards || !unit_buf) return ZF_EINVAL;
  if (!valid_dtype(dtype)) return ZF_EDTYPE;
  if (unit < 0 || unit >= plan->summary.n_units) return ZF_EINVAL;
  if (unit_buf_numel < plan->units[unit].P) return ZF_ESIZE;
  if ((reinterpret_cast<uintptr_t>(unit_buf) & 1u) != 0) return ZF_EALIGN;
  const int nr = plan->summary.n_ranks;
  GatherArgs a;
  for (int r = 0; r < ZF_MAX_RANKS; ++r) a.src[r] = nullptr;
  for (int r = 0; r < nr; ++r) {
    if (!shards[r]) return ZF_EINVAL;
    if ((reinterpret_cast<uintptr_t>(shards[r]) & 1u) != 0) return ZF_EALIGN;
    a.src[r] = static_cast<const uint16_t*>(shards[r]);
  }
  a.dst = static_cast<uint16_t*>(unit_buf);
  a.S = plan->units[unit].S;
  int64_t bx = (a.S / 8 + kThreads - 1) / kThreads;
  if (bx < 1) bx = 1;
  if (bx > 4096) bx = 4096;
  (void)hipGetLastError();
  hipLaunchKernelGGL(zf_gather_kernel, dim3((uint32_t)bx, (uint32_t)nr), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), a);
  return hip_ok(hipGetLastError()) ? ZF_OK : ZF_EHIP;
}

extern "C" int zf_gather_cast(const zf_plan* plan, int64_t group, int32_t dtype,
                              const float* master, int64_t master_numel, void* out,
                              int64_t out_numel, void* stream) {
  if (!valid_plan(plan) || !master || !out) return ZF_EINVAL;
  if (!valid_dtype(dtype)) return ZF_EDTYPE;
  if (group < 0 || group >= (int64_t)plan->groups.size()) return ZF_EINVAL;
  if (!aligned16(master) || (reinterpret_cast<uintptr_t>(out) & 1u) != 0) return ZF_EALIGN;
  const zf_group_info& g = plan->groups[group];
  if (master_numel < plan->summary.psi_pad || out_numel < g.numel) return ZF_ESIZE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  int64_t dst = 0;
  for (int64_t first = 0; first < g.n_units; first += kCastMax) {
    CastArgs a;
    a.master = master;
    a.out = static_cast<uint16_t*>(out);
    int64_t count = g.n_units - first, max_len = 0;
    if (count > kCastMax) count = kCastMax;
    for (int64_t k = 0; k < count; ++k) {
      const zf_unit_info& u = plan->units[g.first_unit + first + k];
      a.e[k].src = u.O;
      a.e[k].dst = dst;
      a.e[k].len = u.L;
      dst += u.L;
      if (u.L > max_len) max_len = u.L;
    }
    const int64_t bx = (max_len + kThreads * 8 - 1) / (kThreads * 8);
    const dim3 grid((uint32_t)(bx < 1 ? 1 : bx), (uint32_t)count);
    if (dtype == ZF_BF16)
      hipLaunchKernelGGL(zf_gather_cast_kernel<ZF_BF16>, grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL(zf_gather_cast_kernel<ZF_F16>, grid, dim3(kThreads), 0, s, a);
    if (!hip_ok(hipGetLastError())) return ZF_EHIP;
  }
  return ZF_OK;
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
