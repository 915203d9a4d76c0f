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
#include <condition_variable>
#include <cstdint>
#include <cstring>
#include <functional>
#include <mutex>
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

// Eight gradients as binary32: fp32 as is, fp16 and bf16 widened exactly.
template <int GT>
__attribute__((target("avx2,f16c"))) inline __m256 load_grad8(const void* a, int64_t i) {
  if constexpr (GT == ZF_F16) {
    return _mm256_cvtph_ps(
        _mm_loadu_si128(reinterpret_cast<const __m128i*>(static_cast<const uint16_t*>(a) + i)));
  } else if constexpr (GT == ZF_BF16) {
    const __m128i h =
        _mm_loadu_si128(reinterpret_cast<const __m128i*>(static_cast<const uint16_t*>(a) + i));
    return _mm256_castsi256_ps(_mm256_slli_epi32(_mm256_cvtepu16_epi32(h), 16));
  } else {
    return _mm256_loadu_ps(static_cast<const float*>(a) + i);
  }
}

// Eight elements in place; returns the new master values.
__attribute__((target("avx2,f16c"))) inline __m256 adam8(const Lanes& c, __m256 acc, float* p,
                                                          float* m, float* v) {
  const __m256 g = _mm256_mul_ps(acc, c.gs);
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

// Sixteen elements: gradients a[i, i + 16), state and outputs from p, m, v,
// out.
template <int GT>
__attribute__((target("avx2,f16c"))) inline void step16(const Lanes& c, const void* a, int64_t i,
                                                         float* p, float* m, float* v,
                                                         uint16_t* out, int32_t dt) {
  const __m256 lo = adam8(c, load_grad8<GT>(a, i), p, m, v);
  const __m256 hi = adam8(c, load_grad8<GT>(a, i + 8), p + 8, m + 8, v + 8);
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
template <int GT>
__attribute__((target("avx2,f16c"))) void adam_range(const Consts& k, const void* a, float* p,
                                                     float* m, float* v, uint16_t* out,
                                                     int32_t dt, int64_t b, int64_t e) {
  constexpr size_t gb = GT == ZF_F32 ? sizeof(float) : sizeof(uint16_t);
  const unsigned saved = _mm_getcsr();
  _mm_setcsr(kDefaultCsr);
  const Lanes c = broadcast(k);
  int64_t i = b;
  for (; i + kVec <= e; i += kVec)
    step16<GT>(c, a, i, p + i, m + i, v + i, out ? out + i : nullptr, dt);
  if (i < e) {
    const int64_t r = e - i;
    alignas(32) float ta[kVec] = {}, tp[kVec] = {}, tm[kVec] = {}, tv[kVec] = {};
    alignas(32) uint16_t to[kVec] = {};
    std::memcpy(ta, static_cast<const char*>(a) + i * gb, r * gb);
    std::memcpy(tp, p + i, r * sizeof(float));
    std::memcpy(tm, m + i, r * sizeof(float));
    std::memcpy(tv, v + i, r * sizeof(float));
    step16<GT>(c, ta, 0, tp, tm, tv, out ? to : nullptr, dt);
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

// Persistent workers: made on first use (and added when a call asks for
// more), parked on a condition variable between calls, joined at exit.  A
// call runs part 0 on the calling thread and parts 1..t-1 on workers 1..t-1;
// calls from several threads take turns.
class Workers {
 public:
  static Workers& get() {
    static Workers w;
    return w;
  }
  // fn(j) for every j in [0, t); returns when all have finished.  Falls back
  // to running a part on the caller when no worker can be started.
  void run(int t, const std::function<void(int)>& fn) {
    std::lock_guard<std::mutex> turn(turn_);
    int have = 0;
    {
      std::unique_lock<std::mutex> lk(mu_);
      while ((int)threads_.size() < t - 1) {
        try {
          const int id = (int)threads_.size() + 1;
          threads_.emplace_back([this, id] { loop(id); });
        } catch (...) {
          break;
        }
      }
      have = std::min(t - 1, (int)threads_.size());
      job_ = &fn;
      job_n_ = have + 1;
      pending_ = have;
      ++gen_;
    }
    work_.notify_all();
    fn(0);
    for (int j = have + 1; j < t; ++j) fn(j);  // parts no worker could take
    std::unique_lock<std::mutex> lk(mu_);
    done_.wait(lk, [this] { return pending_ == 0; });
    job_ = nullptr;
  }

 private:
  Workers() = default;
  ~Workers() {
    {
      std::lock_guard<std::mutex> lk(mu_);
      stop_ = true;
    }
    work_.notify_all();
    for (std::thread& th : threads_) th.join();
  }
  void loop(int id) {
    uint64_t seen = 0;
    std::unique_lock<std::mutex> lk(mu_);
    for (;;) {
      work_.wait(lk, [&] { return stop_ || gen_ != seen; });
      if (stop_) return;
      seen = gen_;
      if (id >= job_n_) continue;
      const std::function<void(int)>* fn = job_;
      lk.unlock();
      (*fn)(id);
      lk.lock();
      if (--pending_ == 0) done_.notify_all();
    }
  }
  std::mutex turn_, mu_;
  std::condition_variable work_, done_;
  std::vector<std::thread> threads_;
  const std::function<void(int)>* job_ = nullptr;
  int job_n_ = 0, pending_ = 0;
  uint64_t gen_ = 0;
  bool stop_ = false;
};

// [0, n) over t parts in contiguous ranges whose starts are multiples of
// kVec; the calling thread takes the first range.
template <int GT>
void run_adam(const Consts& k, const void* a, float* p, float* m, float* v, uint16_t* out,
              int32_t dt, int64_t n, int t) {
  if (n <= 0) return;
  const int64_t blocks = (n + kVec - 1) / kVec;
  auto part = [&](int j) {
    const int64_t b = std::min(n, blocks * j / t * kVec);
    const int64_t e = std::min(n, blocks * (j + 1) / t * kVec);
    if (b < e) adam_range<GT>(k, a, p, m, v, out, dt, b, e);
  };
  if (t <= 1) {
    part(0);
    return;
  }
  Workers::get().run(t, part);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }


}  // namespace

extern "C" int zf_cpu_adam(const zf_hparams* hp, const zf_cpu_adam_args* a) {
  if (!hp || !a || a->n < 0) return ZF_EINVAL;
  const int32_t gdt = a->grad_dtype == 0 ? ZF_F32 : a->grad_dtype;
  if (gdt != ZF_F32 && gdt != ZF_F16 && gdt != ZF_BF16) return ZF_EDTYPE;
  if (a->params && a->param_dtype != ZF_F16 && a->param_dtype != ZF_BF16) return ZF_EDTYPE;
  if (a->n == 0) return ZF_OK;
  if (!a->grad || !a->master || !a->exp_avg || !a->exp_avg_sq) return ZF_EINVAL;
  const void* f32s[] = {a->master, a->exp_avg, a->exp_avg_sq};
  for (const void* q : f32s)
    if (!aligned(q, 4)) return ZF_EALIGN;
  if (!aligned(a->grad, gdt == ZF_F32 ? 4 : 2)) return ZF_EALIGN;
  if (a->params && !aligned(a->params, 2)) return ZF_EALIGN;
  if (!host_has_simd()) return ZF_EUNSUP;
  zf::cpu_adam_run(hp, a->gs, a->bc1, a->bc2, a->n, a->grad, gdt, a->master, a->exp_avg,
                   a->exp_avg_sq, static_cast<uint16_t*>(a->params), a->param_dtype,
                   a->n_threads);
  return ZF_OK;
}


bool zf::host_simd_ok() { return host_has_simd(); }

void zf::cpu_adam_run(const zf_hparams* hp, float gs, float bc1, float bc2, int64_t n,
                      const void* grad, int32_t grad_dtype, float* master, float* exp_avg,
                      float* exp_avg_sq, uint16_t* params, int32_t param_dtype,
                      int32_t n_threads) {
  const zf::UpdateConsts u = zf::update_consts(hp);
  const Consts k{gs, u.dec, u.b1, u.c1, u.b2, u.c2, bc1, bc2, u.lrf, u.ef};
  const int t = resolve_threads(n_threads, n);
  if (grad_dtype == ZF_F16)
    run_adam<ZF_F16>(k, grad, master, exp_avg, exp_avg_sq, params, param_dtype, n, t);
  else if (grad_dtype == ZF_BF16)
    run_adam<ZF_BF16>(k, grad, master, exp_avg, exp_avg_sq, params, param_dtype, n, t);
  else
    run_adam<ZF_F32>(k, grad, master, exp_avg, exp_avg_sq, params, param_dtype, n, t);
}
