// zf_cpu_adam.cpp -- CPU-Adam, the host side of ZeRO-Offload (host C++ only).
//
// CMU 15-779 Lecture 13 notes, "Zero Redundancy and PyTorch FSDP", 7.1: with
// the optimizer offloaded, the fp32 master, both Adam moments and the update
// live on the CPU; 7.2: the update there is a SIMD, multithreaded Adam.
//
// The element update is the step's (one binary32 operation per operator, in
// the update pass's order): g = acc*gs; p = p*dec; m = b1*m + c1*g;
// v = b2*v + c2*(g*g); p = p - lr*((m/bc1) / (sqrt(v/bc2) + eps)).  AVX2 has
// correctly rounded division and square root and this file is built without
// FMA contraction, so the host produces the device's bits.  Every worker
// runs with the default MXCSR (round to nearest even, no flush-to-zero, no
// denormals-are-zero) and restores the caller's afterwards.
#include <immintrin.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "zf_internal.h"

namespace {

constexpr int64_t kVec = 16;  // elements per inner step (two 8-lane vectors)
constexpr int kMaxThreads = 256;
constexpr unsigned kDefaultCsr = 0x1F80;  // all exceptions masked, RNE, no FTZ / DAZ

struct Consts {
  float gs, dec, b1, c1, b2, c2, bc1, bc2, lrf, ef;
};

bool host_has_simd() {
  static const bool ok = [] {
    __builtin_cpu_init();
    return __builtin_cpu_supports("avx2") && __builtin_cpu_supports("f16c");
  }();
  return ok;
}

struct Lanes {
  __m256 gs, dec, b1, c1, b2, c2, bc1, bc2, lrf, ef;
};

__attribute__((target("avx2,f16c"))) inline Lanes broadcast(const Consts& c) {
  Lanes l;
  l.gs = _mm256_set1_ps(c.gs);
  l.dec = _mm256_set1_ps(c.dec);
  l.b1 = _mm256_set1_ps(c.b1);
  l.c1 = _mm256_set1_ps(c.c1);
  l.b2 = _mm256_set1_ps(c.b2);
  l.c2 = _mm256_set1_ps(c.c2);
  l.bc1 = _mm256_set1_ps(c.bc1);
  l.bc2 = _mm256_set1_ps(c.bc2);
  l.lrf = _mm256_set1_ps(c.lrf);
  l.ef = _mm256_set1_ps(c.ef);
  return l;
}

// Eight elements in place; returns the new master values.
__attribute__((target("avx2,f16c"))) inline __m256 adam8(const Lanes& c, const float* a,
                                                          float* p, float* m, float* v) {
  const __m256 g = _mm256_mul_ps(_mm256_loadu_ps(a), c.gs);
  __m256 pp = _mm256_mul_ps(_mm256_loadu_ps(p), c.dec);
  const __m256 mm = _mm256_add_ps(_mm256_mul_ps(c.b1, _mm256_loadu_ps(m)), _mm256_mul_ps(c.c1, g));
  const __m256 vv = _mm256_add_ps(_mm256_mul_ps(c.b2, _mm256_loadu_ps(v)),
                                  _mm256_mul_ps(c.c2, _mm256_mul_ps(g, g)));
  const __m256 d = _mm256_add_ps(_mm256_sqrt_ps(_mm256_div_ps(vv, c.bc2)), c.ef);
  const __m256 mh = _mm256_div_ps(mm, c.bc1);
  pp = _mm256_sub_ps(pp, _mm256_mul_ps(c.lrf, _mm256_div_ps(mh, d)));
  _mm256_storeu_ps(p, pp);
  _mm256_storeu_ps(m, mm);
  _mm256_storeu_ps(v, vv);
  return pp;
}

// bf16 round-to-nearest-even of eight binary32 values, one per 32-bit lane
// (a NaN stays a quiet NaN with its sign and top payload bits).
__attribute__((target("avx2,f16c"))) inline __m256i bf16_lanes(__m256 x) {
  const __m256i u = _mm256_castps_si256(x);
  const __m256i odd = _mm256_and_si256(_mm256_srli_epi32(u, 16), _mm256_set1_epi32(1));
  const __m256i r =
      _mm256_srli_epi32(_mm256_add_epi32(_mm256_add_epi32(u, _mm256_set1_epi32(0x7FFF)), odd), 16);
  const __m256i mag = _mm256_and_si256(u, _mm256_set1_epi32(0x7FFFFFFF));
  const __m256i nan = _mm256_cmpgt_epi32(mag, _mm256_set1_epi32(0x7F800000));
  const __m256i q = _mm256_or_si256(_mm256_srli_epi32(u, 16), _mm256_set1_epi32(0x0040));
  return _mm256_blendv_epi8(r, q, nan);
}

// Sixteen elements [i, i + 16) of the arrays.
__attribute__((target("avx2,f16c"))) inline void step16(const Lanes& c, const float* a, float* p,
                                                         float* m, float* v, uint16_t* out,
                                                         int32_t dt) {
  const __m256 lo = adam8(c, a, p, m, v);
  const __m256 hi = adam8(c, a + 8, p + 8, m + 8, v + 8);
  if (!out) return;
  if (dt == ZF_BF16) {
    // packus keeps 0..0xFFFF exactly; it interleaves 128-bit halves, which
    // the 64-bit permute puts back in order
    const __m256i packed = _mm256_packus_epi32(bf16_lanes(lo), bf16_lanes(hi));
    _mm256_storeu_si256(reinterpret_cast<__m256i*>(out),
                        _mm256_permute4x64_epi64(packed, 0xD8));
  } else {
    const int kRne = _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC;
    _mm_storeu_si128(reinterpret_cast<__m128i*>(out), _mm256_cvtps_ph(lo, kRne));
    _mm_storeu_si128(reinterpret_cast<__m128i*>(out + 8), _mm256_cvtps_ph(hi, kRne));
  }
}

// Elements [b, e) on this thread.  The ragged end (< 16) is staged through
// zero-padded local arrays so every element takes the same vector path.
__attribute__((target("avx2,f16c"))) void adam_range(const Consts& k, const float* a, float* p,
                                                     float* m, float* v, uint16_t* out,
                                                     int32_t dt, int64_t b, int64_t e) {
  const unsigned saved = _mm_getcsr();
  _mm_setcsr(kDefaultCsr);
  const Lanes c = broadcast(k);
  int64_t i = b;
  for (; i + kVec <= e; i += kVec) step16(c, a + i, p + i, m + i, v + i, out ? out + i : nullptr, dt);
  if (i < e) {
    const int64_t r = e - i;
    alignas(32) float ta[kVec] = {}, tp[kVec] = {}, tm[kVec] = {}, tv[kVec] = {};
    alignas(32) uint16_t to[kVec] = {};
    std::memcpy(ta, a + i, r * sizeof(float));
    std::memcpy(tp, p + i, r * sizeof(float));
    std::memcpy(tm, m + i, r * sizeof(float));
    std::memcpy(tv, v + i, r * sizeof(float));
    step16(c, ta, tp, tm, tv, out ? to : nullptr, dt);
    std::memcpy(p + i, tp, r * sizeof(float));
    std::memcpy(m + i, tm, r * sizeof(float));
    std::memcpy(v + i, tv, r * sizeof(float));
    if (out) std::memcpy(out + i, to, r * sizeof(uint16_t));
  }
  _mm_setcsr(saved);
}

int resolve_threads(int32_t n_threads, int64_t n) {
  int t = n_threads > 0 ? n_threads : (int)std::thread::hardware_concurrency();
  if (t < 1) t = 1;
  if (t > kMaxThreads) t = kMaxThreads;
  // at least 64 Ki elements per thread
  const int64_t most = std::max<int64_t>(1, n / 65536);
  if (t > most) t = (int)most;
  return t;
}

// [0, n) over t threads in contiguous ranges whose starts are multiples of
// kVec; the calling thread takes the first range.
void run_adam(const Consts& k, const float* a, float* p, float* m, float* v, uint16_t* out,
              int32_t dt, int64_t n, int t) {
  if (n <= 0) return;
  const int64_t blocks = (n + kVec - 1) / kVec;
  std::vector<std::thread> pool;
  pool.reserve(t > 0 ? t - 1 : 0);
  auto range = [&](int j, int64_t& b, int64_t& e) {
    b = std::min(n, blocks * j / t * kVec);
    e = std::min(n, blocks * (j + 1) / t * kVec);
  };
  for (int j = 1; j < t; ++j) {
    int64_t b, e;
    range(j, b, e);
    if (b >= e) continue;
    try {
      pool.emplace_back(adam_range, std::cref(k), a, p, m, v, out, dt, b, e);
    } catch (...) {  // no thread available: this range runs here
      adam_range(k, a, p, m, v, out, dt, b, e);
    }
  }
  int64_t b0, e0;
  range(0, b0, e0);
  if (b0 < e0) adam_range(k, a, p, m, v, out, dt, b0, e0);
  for (auto& th : pool) th.join();
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }


}  // namespace

extern "C" int zf_cpu_adam(const zf_hparams* hp, const zf_cpu_adam_args* a) {
  if (!hp || !a || a->n < 0 || a->reserved != 0) return ZF_EINVAL;
  if (a->params && a->param_dtype != ZF_F16 && a->param_dtype != ZF_BF16) return ZF_EDTYPE;
  if (a->n == 0) return ZF_OK;
  if (!a->grad || !a->master || !a->exp_avg || !a->exp_avg_sq) return ZF_EINVAL;
  const void* f32s[] = {a->grad, a->master, a->exp_avg, a->exp_avg_sq};
  for (const void* q : f32s)
    if (!aligned(q, 4)) return ZF_EALIGN;
  if (a->params && !aligned(a->params, 2)) return ZF_EALIGN;
  if (!host_has_simd()) return ZF_EUNSUP;
  zf::cpu_adam_run(hp, a->gs, a->bc1, a->bc2, a->n, a->grad, a->master, a->exp_avg,
                   a->exp_avg_sq, static_cast<uint16_t*>(a->params), a->param_dtype,
                   a->n_threads);
  return ZF_OK;
}


bool zf::host_simd_ok() { return host_has_simd(); }

void zf::cpu_adam_run(const zf_hparams* hp, float gs, float bc1, float bc2, int64_t n,
                      const float* grad, float* master, float* exp_avg, float* exp_avg_sq,
                      uint16_t* params, int32_t param_dtype, int32_t n_threads) {
  const zf::UpdateConsts u = zf::update_consts(hp);
  const Consts k{gs, u.dec, u.b1, u.c1, u.b2, u.c2, bc1, bc2, u.lrf, u.ef};
  run_adam(k, grad, master, exp_avg, exp_avg_sq, params, param_dtype, n,
           resolve_threads(n_threads, n));
}
