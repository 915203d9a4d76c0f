// zf_backward.hip -- the backward-side reduction: one bucket's (or FSDP
// unit's) reduce-scatter of 16-bit or fp32 replicas into the fp32 gradient
// shards, storing or accumulating over micro-batches, and the no_sync local
// fp32 accumulation of one replica.
//
// Pages followed (by title and section): CMU 15-779 Lecture 13 notes, "Zero
// Redundancy and PyTorch FSDP", 3.2 (a reduce-scatter per bucket during
// backward) and 5.6 (accumulation: reduce every micro-batch, or accumulate
// locally and reduce once); Megatron / DeepSpeed / torchtitan architecture
// and source guide, 三.3 (gradient buckets, fp32 main_grad accumulation,
// no_sync), 四.3 (IPG buckets) and 五.7 (accumulation on the shard).
//
// Arithmetic: sum = f32(g_0) + ... + f32(g_{N-1}) in rank order; the shard
// becomes sum, or shard + sum; the local accumulation is acc + f32(g) --
// each + one binary32 addition.
//
// Every stream is read once and written once per launch: the replicas and
// the fp32 accumulator are read with the non-temporal hint (accumulator
// reads: -7% for the bucketed 654M step's launches, -2% for the no_sync
// accumulation), the results stored with it.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "zf_device.h"
#include "zf_hip_status.h"
#include "zf_internal.h"

namespace {

using namespace zf::dev;
using zf::hip_ok;
using zf::kThreads;

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
    if constexpr (ACC) o = ldq32<true>(a.out, qi[h]) + o;
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
// head are vector accesses; otherwise every element is scalar.  One quad per
// thread per block, uncapped: against four quads, the no_sync backward phase
// -9.9% (654M, four micro-batches); two quads -3.3%; caps of 3-4 blocks per
// CU lose.  The bucket reduce-scatter keeps two quads uncapped (one quad
// +5%, caps of 3-4 blocks +18% to +55%).
constexpr int kAccQuads = 1;
struct AccArgs {
  const uint16_t* g;
  float* acc;
  int64_t n, head, nq;
  int32_t vec;
};

template <int DT, bool ACC>
__global__ __launch_bounds__(kThreads) void zf_accumulate_kernel(AccArgs a) {
  constexpr int Q = kAccQuads;
  if (a.vec) {
    const uint16_t* g = a.g + a.head;
    float* o = a.acc + a.head;
    const int64_t q0 = (int64_t)blockIdx.x * kThreads * Q + threadIdx.x;
#pragma unroll
    for (int h = 0; h < Q; ++h) {
      const int64_t q = q0 + (int64_t)h * kThreads;
      if (q < a.nq) {
        f32x4 x = widen4<DT>(ldq16<true>(g, q));
        if constexpr (ACC) x = ldq32<true>(o, q) + x;
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
// Host side.

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

}  // namespace

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
    bx = (a.nq + (int64_t)kThreads * kAccQuads - 1) / ((int64_t)kThreads * kAccQuads);
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
