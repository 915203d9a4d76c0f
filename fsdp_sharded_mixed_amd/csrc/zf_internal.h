// zf_internal.h -- the plan record shared by the planner and the step code.
#pragma once
#include <cstdint>
#include <vector>

#include "zf.h"

namespace zf {

constexpr uint64_t kPlanMagic = 0x7a665f706c616e31ull;  // "zf_plan1"

// Pass-1 grid: a fixed number of blocks per plan, so the squared-norm
// partials (and hence the norm's rounding) do not depend on the device.
constexpr int kThreads = 256;       // 4 wave64 per block
constexpr int kVec = 8;             // elements per thread per iteration
constexpr int kMaxPass1Blocks = 2048;

}  // namespace zf

struct zf_plan {
  uint64_t magic;
  zf_plan_summary summary;
  std::vector<zf_unit_info> units;
  int32_t pass1_blocks;
  int64_t ws_partials_offset;   // bytes
  int64_t ws_rs_offset;         // bytes, -1 if the sums are recomputed
};
