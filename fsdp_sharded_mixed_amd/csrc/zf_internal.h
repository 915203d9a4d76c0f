// zf_internal.h -- the plan record shared by the planner and the step code.
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
// Tiling (measured on MI355X, in-process A/B over builds on one box):
//  - pass 1 streams the N replicas with the non-temporal load hint.  With
//    N <= 4 it walks the tiles XCD-contiguously (N = 2: -6%, 3: -5%,
//    4: -5%); at N = 8 that walk costs +4%, so many replicas keep one
//    shared window.  One 2-quad step per thread for N <= 2 (-6% at 4.06B),
//    two steps otherwise;
//  - the update pass uses plain loads; two 2-quad steps per thread on large
//    recomputing plans, one otherwise (within 1% either way).
// Builds may pin a choice for measurement: ZF_FORCE_UNR1, ZF_FORCE_UNR2 (1|2),
// ZF_FORCE_MAP1 (0|1), ZF_PASS1_NT_LOADS (0|1).
#ifndef ZF_PASS1_NT_LOADS
#define ZF_PASS1_NT_LOADS 1
#endif
constexpr int kThreads = 256;        // 4 wave64 per block
constexpr int kQuadsPerUnr = 2;      // quads (4 elements) per thread per tile step
constexpr int64_t kBigPlan = int64_t(1) << 27;  // padded elements
inline int unr_pass1(int n_ranks) {
#ifdef ZF_FORCE_UNR1
  (void)n_ranks;
  return ZF_FORCE_UNR1;
#else
  return n_ranks <= 2 ? 1 : 2;
#endif
}
inline int map_pass1(int n_ranks) {
#ifdef ZF_FORCE_MAP1
  (void)n_ranks;
  return ZF_FORCE_MAP1;
#else
  return n_ranks <= 4 ? 1 : 0;
#endif
}
inline int unr_pass2(int n_ranks, int64_t psi_pad, bool materialize) {
  (void)n_ranks;
#ifdef ZF_FORCE_UNR2
  (void)psi_pad;
  (void)materialize;
  return ZF_FORCE_UNR2;
#else
  return (!materialize && psi_pad >= kBigPlan) ? 2 : 1;
#endif
}
constexpr int kMaxLevel2Blocks = 1024;

}  // namespace zf

struct zf_plan {
  uint64_t magic;
  zf_plan_summary summary;
  std::vector<zf_unit_info> units;
  std::vector<zf_group_info> groups;
  int32_t unr1, unr2;           // tile depth of pass 1 / pass 2 (x2 quads per thread)
  int32_t pass1_map;            // pass-1 tile walk (0 shared window, 1 XCD-contiguous)
  int64_t pass1_tiles;          // pass-1 blocks = squared-norm partials
  int32_t level2_blocks;        // blocks reducing the partials
  int64_t pass2_tiles;          // update-pass blocks
  int64_t ws_partials_offset;   // bytes
  int64_t ws_partials2_offset;  // bytes
  int64_t ws_rs_offset;         // bytes, -1 if the sums are recomputed
};
