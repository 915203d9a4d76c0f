// Concurrency driver for ThreadSanitizer: CPU-Adam's persistent worker pool
// under several calling threads at once.
//
// Four threads each run a sequence of multithreaded zf_cpu_adam calls (with
// different thread counts, so the pool grows while others wait their turn)
// on their own arrays, while the main thread keeps calling too.  Every
// thread then repeats its sequence single-threaded on a copy of its inputs:
// the results must agree bit for bit (the update is element-wise, so the
// split over threads cannot change a bit), and TSan must report nothing.
#include <cassert>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <thread>
#include <vector>

#include "zf.h"

namespace {

struct Arrays {
  std::vector<float> g, p, m, v;
  std::vector<uint16_t> out;
};

Arrays make(int64_t n, uint32_t seed) {
  std::mt19937 rng(seed);
  std::normal_distribution<float> nd(0.0f, 1.0f);
  Arrays a;
  a.g.resize(n);
  a.p.resize(n);
  a.m.assign(n, 0.0f);
  a.v.assign(n, 0.0f);
  a.out.assign(n, 0);
  for (int64_t i = 0; i < n; ++i) {
    a.g[i] = nd(rng);
    a.p[i] = 0.02f * nd(rng);
  }
  return a;
}

int run_sequence(Arrays& a, const int* threads, int calls) {
  zf_hparams hp{1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0};
  const int64_t n = (int64_t)a.g.size();
  for (int k = 0; k < calls; ++k) {
    zf_cpu_adam_args args{n, a.g.data(), a.p.data(), a.m.data(), a.v.data(), a.out.data(),
                          ZF_BF16, threads[k % 4], 1e-3f, 0.1f, 0.001f, 0};
    const int rc = zf_cpu_adam(&hp, &args);
    if (rc != ZF_OK) return rc;
  }
  return ZF_OK;
}

bool same(const Arrays& x, const Arrays& y) {
  const size_t f = x.p.size() * sizeof(float);
  return std::memcmp(x.p.data(), y.p.data(), f) == 0 && std::memcmp(x.m.data(), y.m.data(), f) == 0 &&
         std::memcmp(x.v.data(), y.v.data(), f) == 0 &&
         std::memcmp(x.out.data(), y.out.data(), x.out.size() * 2) == 0;
}

}  // namespace

int main() {
  const int64_t n = 300001;  // 4 parts of >= 64 Ki elements, ragged end
  const int calls = 6;
  const int mixed[4] = {4, 2, 0, 3};
  const int single[4] = {1, 1, 1, 1};
  std::vector<Arrays> multi, ref;
  for (int t = 0; t < 5; ++t) {
    multi.push_back(make(n, 100 + t));
    ref.push_back(make(n, 100 + t));
  }
  {
    Arrays probe = make(16, 1);
    if (run_sequence(probe, single, 1) == ZF_EUNSUP) {
      std::puts("threads driver: no AVX2 on this host, nothing to check");
      return 0;
    }
  }
  std::vector<int> rc(5, -99);
  std::vector<std::thread> th;
  for (int t = 0; t < 4; ++t)
    th.emplace_back([&, t] { rc[t] = run_sequence(multi[t], mixed, calls); });
  rc[4] = run_sequence(multi[4], mixed, calls);  // the main thread calls meanwhile
  for (std::thread& x : th) x.join();
  for (int t = 0; t < 5; ++t) {
    assert(rc[t] == ZF_OK);
    assert(run_sequence(ref[t], single, calls) == ZF_OK);
    if (!same(multi[t], ref[t])) {
      std::printf("thread %d: multithreaded result differs\n", t);
      return 1;
    }
  }
  std::puts("threads driver: ok");
  return 0;
}
