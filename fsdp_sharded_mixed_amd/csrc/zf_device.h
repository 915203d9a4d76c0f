// zf_device.h -- pieces shared by the library's kernel files: the quad
// layout of a lane's elements, 128-bit loads and non-temporal stores, the
// exact 16-bit <-> binary32 conversions, the fixed-order replica sums, the
// deterministic block reduction, and argument checks used by every entry
// point.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "zf_internal.h"

namespace zf {
namespace dev {

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
typedef float f32x2 __attribute__((ext_vector_type(2)));
constexpr int kQuad = 4;

template <bool NT>
__device__ __forceinline__ u32x2 ldq16(const uint16_t* base, int64_t q) {
  const u32x2* p = reinterpret_cast<const u32x2*>(base) + q;
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT = false>
__device__ __forceinline__ f32x4 ldq32(const float* base, int64_t q) {
  const f32x4* p = reinterpret_cast<const f32x4*>(base) + q;
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
__device__ __forceinline__ void stq32_nt(float* base, int64_t q, f32x4 x) {
  __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(base) + q);
}
// A plain fp32 quad store, written as two 8-byte halves: a store that does
// not look like stq32_nt of the same value, so that the compiler never merges
// the two into one and drops the non-temporal hint (the backend joins the
// halves into one 16-byte store again).
__device__ __forceinline__ void stq32_halves(float* base, int64_t q, f32x4 x) {
  f32x2* p = reinterpret_cast<f32x2*>(base) + 2 * q;
  p[0] = (f32x2){x.x, x.y};
  p[1] = (f32x2){x.z, x.w};
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
// Argument checks shared by the entry points.

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool valid_dtype(int32_t d) { return d == ZF_F16 || d == ZF_BF16; }
inline bool valid_plan(const zf_plan* p) { return p && p->magic == zf::kPlanMagic; }

inline int grads_ok(const zf_plan* plan, const void* const* grads, GradPtrs& out) {
  if (!grads) return ZF_EINVAL;
  for (int q = 0; q < plan->summary.n_ranks; ++q) {
    if (!grads[q]) return ZF_EINVAL;
    if (!aligned16(grads[q])) return ZF_EALIGN;
    out.p[q] = static_cast<const uint16_t*>(grads[q]);
  }
  for (int q = plan->summary.n_ranks; q < ZF_MAX_RANKS; ++q) out.p[q] = nullptr;
  return ZF_OK;
}

}  // namespace dev
}  // namespace zf
