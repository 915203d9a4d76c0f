// zf_internal.h -- the plan record and step internals shared by the planner,
// the step code and the offload step.
#pragma once
#include <cstdint>
#include <vector>

#include "zf.h"

namespace zf {

constexpr uint64_t kPlanMagic = 0x7a665f706c616e31ull;  // "zf_plan1"

// Grids: one tile per block (the hardware dispatcher balances the tiles).
// Pass 1 writes one squared-norm partial per tile; a second level of
// kLevel2Blocks blocks reduces fixed, contiguous ranges of them; a single
// block finishes.  The tiling depends only on the plan, so the norm's
// rounding does not depend on the device or the run.
// Tiling (measured on MI355X, in-process A/B over builds on one GPU):
//  - pass 1 streams the N replicas with the non-temporal load hint, one
//    8-byte quad per lane per replica (16-byte loads of quad pairs cost
//    +50% at N = 8, where the sums' stores become strided, and +8% at N = 2).  With
//    N <= 4 it walks the tiles XCD-contiguously (N = 2: -6%, 3: -5%,
//    4: -5%); at N = 8 that walk costs +4%, so many replicas keep one
//    shared window.  One 2-quad step per thread for N <= 2 (-6% at 4.06B)
//    and for N >= 6 (step time at 73M: N = 6 -1.2%, 8 -1.5%, 12 -2.8%, 16
//    -1.6%, 32 -1.9%, with the caps below), two steps for N = 3-5 (one step
//    at N = 5: +0.7%);
//  - the update pass reads master, m and v with the non-temporal hint (under
//    the occupancy cap: 73M -4%, 654M -7%, 4.06B -2%, FSDP2 2.1B -2%; before
//    the cap the same hint had cost +15%) and the materialised sums with
//    plain loads (the hint there: neutral at 73M, +6% for FSDP2); its tiles
//    walk in block order (the XCD-contiguous walk costs +3% there), or
//    backward behind a cached-sums window (cached_sums_quads);
//  - the update pass takes one quad per thread per tile; recomputing the
//    sums it runs 128-thread blocks, at most 5 per CU (10 waves), reading
//    materialised sums 256-thread blocks, at most 3 per CU (12 waves), 4
//    behind a cached-sums window: the bytes in flight per CU decide it.
//    128-thread blocks at 4, 5, 6 per CU against 256-thread blocks at 3,
//    recomputing: 4.06B +5.9%, -2.5%, -1.2%; 2.1B ZeRO-3 +3.4%, -4.7%,
//    -4.2%; 654M +6.4%, -2.0%, -2.0%; 73M at N = 2-4 +0.7% to +6.4%, -2.0%
//    to -3.8%, -2.7% to -4.4%; reading FSDP2's fp32 gradient shards they
//    lose (+2.3% at 5 per CU).  Before that, one quad per thread in
//    256-thread blocks at 3 per CU (4 behind a window) against the earlier
//    two quads at 2 per CU, the step: 4.06B -3.9%, 2.1B ZeRO-3 -3.3%, FSDP2
//    2.1B -3.8%, 654M -2.3%, 73M at N = 2 -4.8%, 73M at N = 8 (window)
//    -2.2%; one quad at 2, 4, 5, 6 blocks or uncapped gave 4.06B +3.1%, -1.8%, +0.5%, +2.1%, +5.3% and 73M at N = 8
//    +3.3%, -2.2%, -2.2%, -1.9%, -2.1%; two quads at 3 blocks +1.1% and
//    -1.0%.  (Two quads at 2 blocks had beaten the register-limited 8 blocks
//    by 3-10% and 1 block by 10%.)  Pass 1 runs at most 3 blocks per CU
//    when it streams 6 to 8 replicas and writes the sums, 4 with more (one
//    step at 73M, N = 8: cap 3 -2.0%, no cap +0.6%, 4 -0.2%, 6 +1.0%; N =
//    16: cap 4 -2.3%, 3 +0.1%; the earlier two-step tiles had taken cap 3 at
//    N = 6-8 for -2% to -3%); with 2 replicas, read-only or writing, it needs
//    every block it can get (a cap of 4 costs +13% to +90%).
//  - pass 1 splits full tiles from the last one: a full tile's loads carry
//    no range check and issue back to back (-2% at N = 8; the update pass
//    measured within 1% either way and keeps one code path).
//    The cap is dynamic LDS that the kernel never touches, sized so that no
//    more blocks fit in a CU's 160 KiB.

constexpr int kThreads = 256;        // 4 wave64 per block
constexpr int kQuadsPerUnr = 2;      // pass 1: quads (4 elements) per thread per tile step
constexpr int kQuadsPass2 = 1;       // the update pass: quads per thread per tile step
// the update pass's block size: 128 threads when it recomputes the sums from
// the replicas, 256 when it reads materialised sums
constexpr int kThreadsPass2Recompute = 128;
constexpr int kThreadsPass2Mat = 256;
constexpr int threads_pass2(bool mat) { return mat ? kThreadsPass2Mat : kThreadsPass2Recompute; }
inline int unr_pass1(int n_ranks) { return (n_ranks <= 2 || n_ranks >= 6) ? 1 : 2; }
inline int map_pass1(int n_ranks) { return n_ranks <= 4 ? 1 : 0; }
constexpr int kMaxLevel2Blocks = 1024;

// Materialised sums and the memory-side cache.  Pass 1 stores the fp32 sums
// (N > 4) and the update pass reads them back.  When they are small next to
// the chip's 256 MB Infinity Cache, pass 1 stores the sums of its last
// kCachedSumsBytes with plain, cache-allocating stores (the rest, and every
// larger plan's sums, non-temporal) and the update pass walks its tiles from
// the last to the first, so it starts on sums the cache still holds instead
// of reading them from HBM.  In-process A/B runs, one shared workspace, step
// time against the all-non-temporal forward walk: 73M at N = 5, 6, 8, 16:
// -5.5%, -4.1%, -3.2%, -0.3%; 40M at N = 8 -5.3%; 100M (381 MiB of sums)
// -0.8%; forced on at 572 MiB +1.4% and at 2.4 GiB +0.4%.  Windows of 192
// MiB and of the whole sums did worse at most sizes.
constexpr int64_t kCachedSumsBytes = 256ll << 20;
constexpr int64_t kCachedSumsLimit = 448ll << 20;
// quads of the window for a plan of psi_pad elements (0: no window).  A
// test build (ZF_TEST_CACHED_SUMS_MB) gives every plan a window of that many
// MiB, so that small plans split their sums between non-temporal and
// cache-allocating stores the way the 73M-parameter plan at N = 8 does.
inline int64_t cached_sums_quads(int64_t psi_pad) {
#ifdef ZF_TEST_CACHED_SUMS_MB
  (void)psi_pad;
  return (int64_t)ZF_TEST_CACHED_SUMS_MB * (1 << 16);
#else
  if (psi_pad * 4 > kCachedSumsLimit) return 0;
  return kCachedSumsBytes / 16;
#endif
}

// Resident-block caps (blocks per CU, 0: none) and the dynamic LDS per block
// that enforces one: k blocks fit in the CU's LDS, k + 1 do not (the margin
// covers the kernels' own few hundred bytes of static LDS).
constexpr int64_t kLdsPerCU = 160 * 1024;
inline int occ_pass1(int n_ranks, bool writes_sums) {
  if (!writes_sums || n_ranks < 6) return 0;
  return n_ranks > 8 ? 4 : 3;
}
inline int occ_pass2(bool mat, bool cached_sums) {
  if (!mat) return 5;  // 128-thread blocks: 10 waves per CU
  return cached_sums ? 4 : 3;
}
inline uint32_t occupancy_lds(int blocks_per_cu) {
  if (blocks_per_cu <= 0) return 0;
  return (uint32_t)(kLdsPerCU / (blocks_per_cu + 1) + 1024);
}
static_assert(kLdsPerCU / (kLdsPerCU / 3 + 1024) == 2, "two blocks per CU");
static_assert(kLdsPerCU / (kLdsPerCU / 4 + 1024) == 3, "three blocks per CU");
static_assert(kLdsPerCU / (kLdsPerCU / 5 + 1024) == 4, "four blocks per CU");
static_assert(kLdsPerCU / (kLdsPerCU / 6 + 1024) == 5, "five blocks per CU");

// The device state block (the caller's zf_state_bytes() buffer), also read
// on the host by the offload step.
struct alignas(16) DevState {
  double loss_scale;     // S for the next step
  double beta1_pow;      // beta1^t after t applied steps (1 at t = 0)
  double beta2_pow;
  int64_t t;
  int32_t growth_ctr, growth_interval, dynamic, pad0;
  // result of the last step
  int32_t overflow, skipped;
  double sumsq, norm, coef, scale_used;
  float gs, bc1, bc2, pad1;
};
static_assert(sizeof(DevState) <= 256, "state block");
constexpr int64_t kStateBytes = 256;

// Validates `args` and enqueues the step on `stream`: pass 1, the norm
// reduction and the finish kernel, then (update == true) the update pass.
// With update == false the fp32 state and params are neither needed nor
// touched and grad_shards must be given (pass 1 leaves the sums there, in
// fp32, or with down16 rounded to the gradient dtype in its first Psi'*2
// bytes, the norm and overflow then taken on the rounded values).
// noalloc: the workspace is the library's static device scratch array
// (zf_shard_step_noalloc) instead of args->workspace, which must then be
// NULL with workspace_size 0.
int step_enqueue(const zf_plan* plan, const zf_hparams* hp, const zf_step_args* args,
                 void* stream, bool update, bool down16, bool noalloc = false);

// Binary32 hyperparameters of the update, each rounded once from its double.
struct UpdateConsts {
  float dec, b1, c1, b2, c2, lrf, ef;
};
inline UpdateConsts update_consts(const zf_hparams* hp) {
  UpdateConsts c;
  c.dec = (float)(1.0 - hp->lr * hp->weight_decay);
  c.b1 = (float)hp->beta1;
  c.c1 = (float)(1.0 - hp->beta1);
  c.b2 = (float)hp->beta2;
  c.c2 = (float)(1.0 - hp->beta2);
  c.lrf = (float)hp->lr;
  c.ef = (float)hp->eps;
  return c;
}

// The HIP error code behind the calling thread's last ZF_EHIP (0: none).
extern thread_local int last_hip_error;

// CPU-Adam (host, AVX2): the update pass's element arithmetic over [0, n)
// with the given step scalars, split over n_threads threads (<= 0: all).
bool host_simd_ok();
// grad_dtype: ZF_F32 (grad points to binary32) or ZF_F16 / ZF_BF16 (16-bit
// gradients, widened exactly).
void cpu_adam_run(const zf_hparams* hp, float gs, float bc1, float bc2, int64_t n,
                  const void* grad, int32_t grad_dtype, float* master, float* exp_avg,
                  float* exp_avg_sq, uint16_t* params, int32_t param_dtype, int32_t n_threads);

}  // namespace zf

struct zf_plan {
  uint64_t magic;
  zf_plan_summary summary;
  std::vector<zf_unit_info> units;
  std::vector<zf_group_info> groups;
  int32_t unr1;                 // tile steps of pass 1 per thread
  int32_t pass1_map;            // pass-1 tile walk (0 shared window, 1 XCD-contiguous)
  int64_t pass1_tiles;          // pass-1 blocks = squared-norm partials
  int32_t level2_blocks;        // blocks reducing the partials
  int64_t ws_partials_offset;   // bytes
  int64_t ws_partials2_offset;  // bytes
  int64_t ws_rs_offset;         // bytes, -1 if the sums are recomputed
  int64_t ws_partials_bytes;    // bytes of the two partials regions (the
                                // workspace without the fp32 sums)
  int64_t cached_sums_quads;    // fp32 sums stored cache-allocating (see cached_sums_quads)
};

namespace zf {
// The update pass's blocks for a plan: one tile of threads_pass2(mat) x
// kQuadsPass2 quads each (at least one block; the last one also
// takes the ragged tail).
inline int64_t pass2_tiles(const zf_plan* p, bool mat) {
  const int64_t q = (int64_t)threads_pass2(mat) * kQuadsPass2;
  const int64_t t = (p->summary.psi_pad / 4 + q - 1) / q;
  return t < 1 ? 1 : t;
}
}  // namespace zf
