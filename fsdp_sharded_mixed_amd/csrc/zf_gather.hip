// zf_gather.hip -- layout kernels: the ZeRO-3 / FSDP unit gather of 16-bit
// shards, FSDP2's cast-at-gather of fp32 shards, and resharding of a
// per-element array between two plans.
//
// Pages followed (by title and section): CMU 15-779 Lecture 13 notes, "Zero
// Redundancy and PyTorch FSDP", 3.3 and 5.1 (all-gather of a unit before
// use); Femtotron dev log #9 (unshard into a padded buffer) and #5
// (resharding when the DP size changes); Megatron / DeepSpeed / torchtitan
// architecture and source guide, 五.4 (FSDP2 casts to the parameter dtype at
// all-gather time) and 六.4 (checkpoint resharding).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <new>
#include <vector>

#include "zf_device.h"
#include "zf_hip_status.h"
#include "zf_internal.h"

namespace {

using namespace zf::dev;
using zf::hip_ok;
using zf::kThreads;

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
// One block per 2048-element tile; the launch's parameters own consecutive
// runs of tiles (parameter k: tiles [first_tile[k], first_tile[k+1])), so
// a short parameter costs no idle blocks beside a long one.  The fp32 reads
// carry the non-temporal hint (-12% for the 2.1B FSDP2 gathers); the 16-bit
// stores do not (the next forward reads them; no measurable gain either).
constexpr int kCastMax = 32;  // parameters per launch
constexpr int64_t kCastTile = (int64_t)kThreads * 8;
struct CastEntry {
  int64_t src;  // O_u in the fp32 array
  int64_t dst;  // offset in the group buffer
  int64_t len;  // L_u
};
struct CastArgs {
  const float* master;
  uint16_t* out;
  CastEntry e[kCastMax];
  int64_t first_tile[kCastMax];  // nondecreasing; INT64_MAX past the last parameter
};

template <int DT>
__global__ __launch_bounds__(kThreads) void zf_gather_cast_kernel(CastArgs a) {
  const int64_t b = blockIdx.x;
  int k = 0;  // the block's parameter: how many later parameters start at or before b
#pragma unroll
  for (int j = 1; j < kCastMax; ++j) k += a.first_tile[j] <= b ? 1 : 0;
  const CastEntry e = a.e[k];
  const int64_t t0 = (b - a.first_tile[k]) * kCastTile;
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
        const f32x4 x = ldq32<true>(src, q);
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

}  // namespace

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
  // every launch's tiles fit one grid dimension (checked before any launch)
  for (int64_t first = 0; first < g.n_units; first += kCastMax) {
    int64_t tiles = 0;
    for (int64_t k = first; k < g.n_units && k < first + kCastMax; ++k)
      tiles += (plan->units[g.first_unit + k].L + kCastTile - 1) / kCastTile;
    if (tiles > 0x7FFFFFFF) return ZF_ESIZE;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  int64_t dst = 0;
  for (int64_t first = 0; first < g.n_units; first += kCastMax) {
    CastArgs a;
    a.master = master;
    a.out = static_cast<uint16_t*>(out);
    int64_t count = g.n_units - first, tiles = 0;
    if (count > kCastMax) count = kCastMax;
    for (int64_t k = 0; k < kCastMax; ++k) {
      if (k >= count) {
        a.e[k] = CastEntry{0, 0, 0};
        a.first_tile[k] = INT64_MAX;
        continue;
      }
      const zf_unit_info& u = plan->units[g.first_unit + first + k];
      a.e[k].src = u.O;
      a.e[k].dst = dst;
      a.e[k].len = u.L;
      a.first_tile[k] = tiles;
      dst += u.L;
      tiles += (u.L + kCastTile - 1) / kCastTile;
    }
    if (tiles < 1) tiles = 1;  // only empty parameters: one block that finds nothing to do
    const dim3 grid((uint32_t)tiles);
    if (dtype == ZF_BF16)
      hipLaunchKernelGGL(zf_gather_cast_kernel<ZF_BF16>, grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL(zf_gather_cast_kernel<ZF_F16>, grid, dim3(kThreads), 0, s, a);
    if (!hip_ok(hipGetLastError())) return ZF_EHIP;
  }
  return ZF_OK;
}
