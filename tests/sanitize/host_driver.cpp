// Drives the library's host-only code -- the planner (every layout, random
// segment lists, error paths), the bucket planner and CPU-Adam (lengths,
// threads, offsets, both 16-bit outputs) -- so that a build with
// AddressSanitizer and UndefinedBehaviorSanitizer can report any
// out-of-bounds access, leak or undefined operation.  Test infrastructure.
#include <cassert>
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "zf.h"

int main() {
  std::mt19937_64 rng(5);
  for (int trial = 0; trial < 400; ++trial) {
    const int nseg = 1 + (int)(rng() % 12);
    const int n = 1 + (int)(rng() % 64);
    const int layout = (int)(rng() % 3);
    std::vector<zf_segment> segs(nseg);
    std::vector<int64_t> numel(nseg);
    int32_t unit = 0;
    for (int i = 0; i < nseg; ++i) {
      const int64_t rows = 1 + (int64_t)(rng() % 9), cols = 1 + (int64_t)(rng() % 7);
      if (i > 0 && rng() % 3 == 0) ++unit;
      segs[i] = zf_segment{rows * cols, unit, 0, (rng() % 2) ? rows : 0};
      numel[i] = rows * cols;
    }
    zf_plan* p = nullptr;
    const int stage = (int)(rng() % 4);
    assert(zf_plan_flat(segs.data(), nseg, n, layout, stage, &p) == ZF_OK && p);
    zf_plan_summary s;
    assert(zf_plan_info(p, &s) == ZF_OK);
    for (int64_t u = 0; u < s.n_units; ++u) {
      zf_unit_info ui;
      assert(zf_plan_unit(p, u, &ui) == ZF_OK && ui.P % n == 0 && ui.L <= ui.P);
    }
    for (int64_t g = 0; g < s.n_groups; ++g) {
      zf_group_info gi;
      assert(zf_plan_group(p, g, &gi) == ZF_OK);
    }
    assert(zf_plan_unit(p, s.n_units, nullptr) == ZF_EINVAL);
    assert(zf_workspace_bytes(p) == s.workspace_bytes);
    zf_plan_free(p);
    std::vector<int32_t> ids(nseg);
    int64_t nb = 0;
    assert(zf_plan_buckets(numel.data(), nseg, n, (int64_t)(rng() % 40) - 1, ids.data(), &nb) ==
           ZF_OK);
    assert(nb >= 1 && nb <= nseg);
  }
  // error paths
  zf_plan* p = nullptr;
  zf_segment bad[2] = {{10, 0, 0, 0}, {5, 2, 0, 0}};
  assert(zf_plan_flat(bad, 2, 2, ZF_PER_UNIT, 2, &p) == ZF_EINVAL && !p);
  assert(zf_plan_flat(bad, 1, 0, ZF_PER_UNIT, 2, &p) == ZF_ESIZE);
  zf_segment rowbad[1] = {{10, 0, 0, 3}};
  assert(zf_plan_flat(rowbad, 1, 2, ZF_PER_PARAM_DIM0, 3, &p) == ZF_EINVAL);
  zf_plan_free(nullptr);
  for (int st = 0; st >= -8; --st) (void)zf_strerror(st);

  // CPU-Adam
  zf_hparams hp{1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0};
  std::normal_distribution<float> nd(0.0f, 1.0f);
  for (int64_t n : {0, 1, 15, 16, 17, 1000, 70001}) {
    for (int off = 0; off < 3; ++off) {
      for (int threads : {1, 3, 0}) {
        std::vector<float> g(n + off + 1), pm(n + off + 1), m(n + off + 1), v(n + off + 1);
        std::vector<uint16_t> out(n + off + 1);
        for (size_t i = 0; i < g.size(); ++i) {
          g[i] = nd(rng);
          pm[i] = 0.02f * nd(rng);
        }
        zf_cpu_adam_args a{n, g.data() + off, pm.data() + off, m.data() + off, v.data() + off,
                           out.data() + off, (threads % 2) ? ZF_BF16 : ZF_F16, threads,
                           1e-3f, 0.1f, 0.001f, 0};
        const int rc = zf_cpu_adam(&hp, &a);
        assert(rc == ZF_OK || rc == ZF_EUNSUP);
      }
    }
  }
  std::puts("host driver: ok");
  return 0;
}
