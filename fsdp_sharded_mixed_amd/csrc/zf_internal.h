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
// Tiling (measured on MI355X): pass 1 streams the N replicas with the
// non-temporal load hint; two vectors per thread pay off once N >= 4.  The
// update pass uses plain loads; two vectors per thread pay off on large
// recomputing plans, one on materialising ones (more, smaller tiles).
constexpr int kThreads = 256;        // 4 wave64 per block
constexpr int kVec = 8;              // elements per thread per vector
constexpr int64_t kBigPlan = int64_t(1) << 27;  // padded elements
inline int unr_pass1(int n_ranks) { return n_ranks >= 4 ? 2 : 1; }
inline int unr_pass2(int n_ranks, int64_t psi_pad, bool materialize) {
  (void)n_ranks;
  return (!materialize && psi_pad >= kBigPlan) ? 2 : 1;
}
constexpr int kMaxLevel2Blocks = 1024;

}  // namespace zf

struct zf_plan {
  uint64_t magic;
  zf_plan_summary summary;
  std::vector<zf_unit_info> units;
  int32_t unr1, unr2;           // vectors per thread in pass 1 / pass 2
  int64_t pass1_tiles;          // pass-1 blocks = squared-norm partials
  int32_t level2_blocks;        // blocks reducing the partials
  int64_t pass2_tiles;          // update-pass blocks
  int64_t ws_partials_offset;   // bytes
  int64_t ws_partials2_offset;  // bytes
  int64_t ws_rs_offset;         // bytes, -1 if the sums are recomputed
};
