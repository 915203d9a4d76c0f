// zf_inputs.hip -- seeded synthetic inputs (splitmix64 + Irwin-Hall(12)).
// The definition is stated in zf_inputs.h.  Input generation only: nothing
// here belongs to the step.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "zf_inputs.h"

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__host__ __device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__host__ __device__ __forceinline__ uint64_t stream_state(uint64_t seed, uint64_t stream) {
  return mix64(seed + (stream + 1ull) * kGamma);
}

__device__ __forceinline__ float irwin_hall(uint64_t st, int64_t i) {
  const uint64_t base = st + (uint64_t)i * 3ull * kGamma;
  uint32_t sum = 0;
#pragma unroll
  for (int c = 1; c <= 3; ++c) {
    const uint64_t w = mix64(base + (uint64_t)c * kGamma);
    sum += (uint32_t)(w & 0xFFFFu) + (uint32_t)((w >> 16) & 0xFFFFu) +
           (uint32_t)((w >> 32) & 0xFFFFu) + (uint32_t)(w >> 48);
  }
  // |sum - 393210| < 2^24: the conversion and the power-of-two scaling are exact
  return (float)((int32_t)sum - 393210) * (1.0f / 65536.0f);
}

template <int DT>
__global__ void fill16(uint16_t* dst, int64_t n, uint64_t st, int64_t base, float sf, float kf) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += stride) {
    float x = irwin_hall(st, base + k) * sf;
    x = x * kf;
    if constexpr (DT == 2) dst[k] = __builtin_bit_cast(uint16_t, (__bf16)x);
    else dst[k] = __builtin_bit_cast(uint16_t, (_Float16)x);
  }
}

__global__ void fill32(float* dst, int64_t n, uint64_t st, int64_t base, float sf) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n; k += stride)
    dst[k] = irwin_hall(st, base + k) * sf;
}

dim3 grid_for(int64_t n) {
  int64_t b = (n + 255) / 256;
  if (b < 1) b = 1;
  if (b > 16384) b = 16384;
  return dim3((uint32_t)b);
}

}  // namespace

extern "C" int zfi_fill_normal16(void* dst, int64_t n, int32_t dtype, uint64_t seed,
                                 uint64_t stream, int64_t logical_base, double sigma,
                                 double scale, void* stream_handle) {
  if (!dst || n < 0 || logical_base < 0 || (dtype != 1 && dtype != 2)) return -1;
  if ((reinterpret_cast<uintptr_t>(dst) & 1u) != 0) return -1;
  if (n == 0) return 0;
  const uint64_t st = stream_state(seed, stream);
  hipStream_t s = static_cast<hipStream_t>(stream_handle);
  (void)hipGetLastError();
  if (dtype == 2)
    hipLaunchKernelGGL(fill16<2>, grid_for(n), dim3(256), 0, s, static_cast<uint16_t*>(dst), n,
                       st, logical_base, (float)sigma, (float)scale);
  else
    hipLaunchKernelGGL(fill16<1>, grid_for(n), dim3(256), 0, s, static_cast<uint16_t*>(dst), n,
                       st, logical_base, (float)sigma, (float)scale);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int zfi_fill_normal32(float* dst, int64_t n, uint64_t seed, uint64_t stream,
                                 int64_t logical_base, double sigma, void* stream_handle) {
  if (!dst || n < 0 || logical_base < 0) return -1;
  if ((reinterpret_cast<uintptr_t>(dst) & 3u) != 0) return -1;
  if (n == 0) return 0;
  const uint64_t st = stream_state(seed, stream);
  (void)hipGetLastError();
  hipLaunchKernelGGL(fill32, grid_for(n), dim3(256), 0, static_cast<hipStream_t>(stream_handle),
                     dst, n, st, logical_base, (float)sigma);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" uint64_t zfi_stream_output(uint64_t seed, uint64_t stream, uint64_t j) {
  return mix64(stream_state(seed, stream) + (j + 1ull) * kGamma);
}

// ---------------------------------------------------------------------------
// Bandwidth probe.
namespace {

typedef float f32x4p __attribute__((ext_vector_type(4)));

struct ProbeArgs {
  const float* src[8];
  float* dst[8];
  int64_t nq;
};

template <int R, int W>
__global__ __launch_bounds__(256) void stream_probe(ProbeArgs a) {
  constexpr int Q = 2;
  const int64_t q0 = (int64_t)blockIdx.x * 256 * Q + threadIdx.x;
  f32x4p x[Q];
#pragma unroll
  for (int h = 0; h < Q; ++h) {
    const int64_t q = q0 + (int64_t)h * 256;
    f32x4p t = {0, 0, 0, 0};
    if (q < a.nq) {
#pragma unroll
      for (int r = 0; r < R; ++r) t = t + reinterpret_cast<const f32x4p*>(a.src[r])[q];
    }
    x[h] = t;
  }
#pragma unroll
  for (int h = 0; h < Q; ++h) {
    const int64_t q = q0 + (int64_t)h * 256;
    if (q >= a.nq) continue;
#pragma unroll
    for (int k = 0; k < W; ++k)
      __builtin_nontemporal_store(x[h], reinterpret_cast<f32x4p*>(a.dst[k]) + q);
  }
}

// The same sums in a chosen shape: Q quads per lane per tile, non-temporal
// loads as well as stores, and at most `cap` resident blocks per CU (dynamic
// LDS that no lane touches; n is never negative).
template <int R, int W, int Q>
__global__ __launch_bounds__(256) void stream_probe_shaped(ProbeArgs a) {
  extern __shared__ uint32_t probe_cap_lds[];
  if (a.nq < 0) probe_cap_lds[threadIdx.x] = 0u;
  const int64_t q0 = (int64_t)blockIdx.x * 256 * Q + threadIdx.x;
  f32x4p x[Q];
#pragma unroll
  for (int h = 0; h < Q; ++h) {
    const int64_t q = q0 + (int64_t)h * 256;
    f32x4p t = {0, 0, 0, 0};
    if (q < a.nq) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        t = t + __builtin_nontemporal_load(reinterpret_cast<const f32x4p*>(a.src[r]) + q);
    }
    x[h] = t;
  }
#pragma unroll
  for (int h = 0; h < Q; ++h) {
    const int64_t q = q0 + (int64_t)h * 256;
    if (q >= a.nq) continue;
#pragma unroll
    for (int k = 0; k < W; ++k)
      __builtin_nontemporal_store(x[h], reinterpret_cast<f32x4p*>(a.dst[k]) + q);
  }
}

template <int R, int W>
void launch_shaped_q(int q, dim3 g, uint32_t lds, hipStream_t s, const ProbeArgs& a) {
  if (q == 1) hipLaunchKernelGGL((stream_probe_shaped<R, W, 1>), g, dim3(256), lds, s, a);
  else if (q == 2) hipLaunchKernelGGL((stream_probe_shaped<R, W, 2>), g, dim3(256), lds, s, a);
  else hipLaunchKernelGGL((stream_probe_shaped<R, W, 4>), g, dim3(256), lds, s, a);
}

template <int R>
void launch_shaped_w(int w, int q, dim3 g, uint32_t lds, hipStream_t s, const ProbeArgs& a) {
  switch (w) {
    case 1: launch_shaped_q<R, 1>(q, g, lds, s, a); break;
    case 2: launch_shaped_q<R, 2>(q, g, lds, s, a); break;
    case 4: launch_shaped_q<R, 4>(q, g, lds, s, a); break;
    default: launch_shaped_q<R, 8>(q, g, lds, s, a); break;
  }
}

template <int R>
void launch_probe_w(int w, dim3 g, hipStream_t s, const ProbeArgs& a) {
  switch (w) {
    case 1: hipLaunchKernelGGL((stream_probe<R, 1>), g, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((stream_probe<R, 2>), g, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((stream_probe<R, 4>), g, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((stream_probe<R, 8>), g, dim3(256), 0, s, a); break;
  }
}

}  // namespace

extern "C" int zfi_stream_probe_shaped(const float* const* src, int32_t n_src,
                                       float* const* dst, int32_t n_dst, int64_t n,
                                       int32_t quads, int32_t blocks_per_cu,
                                       void* stream_handle) {
  if (!src || !dst || n <= 0 || n % 4 != 0) return -1;
  if (!(n_src == 1 || n_src == 2 || n_src == 4 || n_src == 8)) return -1;
  if (!(n_dst == 1 || n_dst == 2 || n_dst == 4 || n_dst == 8)) return -1;
  if (!(quads == 1 || quads == 2 || quads == 4)) return -1;
  if (blocks_per_cu < 0 || blocks_per_cu > 8) return -1;
  ProbeArgs a;
  for (int k = 0; k < 8; ++k) {
    a.src[k] = nullptr;
    a.dst[k] = nullptr;
  }
  for (int k = 0; k < n_src; ++k) {
    if (!src[k] || (reinterpret_cast<uintptr_t>(src[k]) & 15u)) return -1;
    a.src[k] = src[k];
  }
  for (int k = 0; k < n_dst; ++k) {
    if (!dst[k] || (reinterpret_cast<uintptr_t>(dst[k]) & 15u)) return -1;
    a.dst[k] = dst[k];
  }
  a.nq = n / 4;
  const int64_t per = 256 * (int64_t)quads;
  const int64_t blocks = (a.nq + per - 1) / per;
  if (blocks > 0x7FFFFFFF) return -1;
  const dim3 g((uint32_t)blocks);
  // a CU holds 160 KiB of LDS: k blocks fit, k + 1 do not
  const uint32_t lds = blocks_per_cu ? (uint32_t)(160 * 1024 / (blocks_per_cu + 1) + 1024) : 0u;
  hipStream_t s = static_cast<hipStream_t>(stream_handle);
  (void)hipGetLastError();
  switch (n_src) {
    case 1: launch_shaped_w<1>(n_dst, quads, g, lds, s, a); break;
    case 2: launch_shaped_w<2>(n_dst, quads, g, lds, s, a); break;
    case 4: launch_shaped_w<4>(n_dst, quads, g, lds, s, a); break;
    default: launch_shaped_w<8>(n_dst, quads, g, lds, s, a); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int zfi_stream_probe(const float* const* src, int32_t n_src, float* const* dst,
                                int32_t n_dst, int64_t n, void* stream_handle) {
  if (!src || !dst || n <= 0 || n % 4 != 0) return -1;
  if (!(n_src == 1 || n_src == 2 || n_src == 4 || n_src == 8)) return -1;
  if (!(n_dst == 1 || n_dst == 2 || n_dst == 4 || n_dst == 8)) return -1;
  ProbeArgs a;
  for (int k = 0; k < 8; ++k) {
    a.src[k] = nullptr;
    a.dst[k] = nullptr;
  }
  for (int k = 0; k < n_src; ++k) {
    if (!src[k] || (reinterpret_cast<uintptr_t>(src[k]) & 15u)) return -1;
    a.src[k] = src[k];
  }
  for (int k = 0; k < n_dst; ++k) {
    if (!dst[k] || (reinterpret_cast<uintptr_t>(dst[k]) & 15u)) return -1;
    a.dst[k] = dst[k];
  }
  a.nq = n / 4;
  const int64_t blocks = (a.nq + 511) / 512;
  if (blocks > 0x7FFFFFFF) return -1;
  const dim3 g((uint32_t)blocks);
  hipStream_t s = static_cast<hipStream_t>(stream_handle);
  (void)hipGetLastError();
  switch (n_src) {
    case 1: launch_probe_w<1>(n_dst, g, s, a); break;
    case 2: launch_probe_w<2>(n_dst, g, s, a); break;
    case 4: launch_probe_w<4>(n_dst, g, s, a); break;
    default: launch_probe_w<8>(n_dst, g, s, a); break;
  }
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// ---------------------------------------------------------------------------
// Update-mix probe: the update pass's bytes per element with none of its
// arithmetic.  One quad per lane, T-thread blocks, at most `cap` resident
// blocks per CU (dynamic LDS that no lane touches; nq is never negative).
// MODE 2 reads two 16-bit arrays (the replicas an N = 2 update pass
// re-reads, plain loads); MODE 0 one fp32 array (materialised sums, plain
// loads).  Both then read three fp32 arrays with the non-temporal hint and
// write them back, and write one 16-bit array, all stores non-temporal.
namespace {

typedef uint32_t u32x2p __attribute__((ext_vector_type(2)));

struct MixArgs {
  const uint16_t* g0;
  const uint16_t* g1;
  const float* sums;
  float* p;
  float* m;
  float* v;
  uint16_t* out;
  int64_t nq;
};

template <int MODE, int T>
__global__ __launch_bounds__(256) void update_mix_probe(MixArgs a) {
  extern __shared__ uint32_t probe_cap_lds[];
  if (a.nq < 0) probe_cap_lds[threadIdx.x] = 0u;
  const int64_t q = (int64_t)blockIdx.x * T + threadIdx.x;
  if (q >= a.nq) return;
  f32x4p g;
  if constexpr (MODE == 2) {
    // element i of each replica widened from bfloat16, the two added
    const u32x2p x0 = reinterpret_cast<const u32x2p*>(a.g0)[q];
    const u32x2p x1 = reinterpret_cast<const u32x2p*>(a.g1)[q];
    const f32x4p w0 = {__uint_as_float(x0.x << 16), __uint_as_float(x0.x & 0xFFFF0000u),
                       __uint_as_float(x0.y << 16), __uint_as_float(x0.y & 0xFFFF0000u)};
    const f32x4p w1 = {__uint_as_float(x1.x << 16), __uint_as_float(x1.x & 0xFFFF0000u),
                       __uint_as_float(x1.y << 16), __uint_as_float(x1.y & 0xFFFF0000u)};
    g = w0 + w1;
  } else {
    g = reinterpret_cast<const f32x4p*>(a.sums)[q];
  }
  f32x4p p = __builtin_nontemporal_load(reinterpret_cast<const f32x4p*>(a.p) + q);
  f32x4p m = __builtin_nontemporal_load(reinterpret_cast<const f32x4p*>(a.m) + q);
  f32x4p v = __builtin_nontemporal_load(reinterpret_cast<const f32x4p*>(a.v) + q);
  p = p + g;
  m = m + g;
  v = v + g;
  __builtin_nontemporal_store(p, reinterpret_cast<f32x4p*>(a.p) + q);
  __builtin_nontemporal_store(m, reinterpret_cast<f32x4p*>(a.m) + q);
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4p*>(a.v) + q);
  const u32x2p o = {(__float_as_uint(p.x) >> 16) | (__float_as_uint(p.y) & 0xFFFF0000u),
                    (__float_as_uint(p.z) >> 16) | (__float_as_uint(p.w) & 0xFFFF0000u)};
  __builtin_nontemporal_store(o, reinterpret_cast<u32x2p*>(a.out) + q);
}

template <int MODE>
void launch_mix(int threads, dim3 g, uint32_t lds, hipStream_t s, const MixArgs& a) {
  if (threads == 128) hipLaunchKernelGGL((update_mix_probe<MODE, 128>), g, dim3(128), lds, s, a);
  else hipLaunchKernelGGL((update_mix_probe<MODE, 256>), g, dim3(256), lds, s, a);
}

bool aligned16p(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int zfi_update_mix_probe(const void* g0, const void* g1, const float* sums, float* p,
                                    float* m, float* v, void* out16, int64_t n,
                                    int32_t block_threads, int32_t blocks_per_cu,
                                    void* stream_handle) {
  const bool replicas = g0 != nullptr || g1 != nullptr;
  if (replicas ? (!g0 || !g1 || sums) : !sums) return -1;
  if (!p || !m || !v || !out16 || n <= 0 || n % 4 != 0) return -1;
  const void* all[] = {replicas ? g0 : sums, replicas ? g1 : sums, p, m, v, out16};
  for (const void* q : all)
    if (!aligned16p(q)) return -1;
  if (block_threads != 128 && block_threads != 256) return -1;
  if (blocks_per_cu < 0 || blocks_per_cu > 8) return -1;
  MixArgs a;
  a.g0 = static_cast<const uint16_t*>(g0);
  a.g1 = static_cast<const uint16_t*>(g1);
  a.sums = sums;
  a.p = p;
  a.m = m;
  a.v = v;
  a.out = static_cast<uint16_t*>(out16);
  a.nq = n / 4;
  const int64_t blocks = (a.nq + block_threads - 1) / block_threads;
  if (blocks > 0x7FFFFFFF) return -1;
  const dim3 g((uint32_t)blocks);
  // a CU holds 160 KiB of LDS: k blocks fit, k + 1 do not
  const uint32_t lds = blocks_per_cu ? (uint32_t)(160 * 1024 / (blocks_per_cu + 1) + 1024) : 0u;
  hipStream_t s = static_cast<hipStream_t>(stream_handle);
  (void)hipGetLastError();
  if (replicas) launch_mix<2>(block_threads, g, lds, s, a);
  else launch_mix<0>(block_threads, g, lds, s, a);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// ---------------------------------------------------------------------------
// Lowering probes: binary32 square root and division as this compiler emits
// them under the step library's flags (correctly rounded divide and sqrt,
// no contraction), for tests that compare them with IEEE results.
namespace {

__global__ __launch_bounds__(256) void sqrt_probe(float* out, int64_t n, uint32_t first) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x; k < n; k += stride)
    out[k] = sqrtf(__uint_as_float(first + (uint32_t)k));
}

__global__ __launch_bounds__(256) void div_probe(const float* a, const float* b, float* out,
                                                 int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x; k < n; k += stride)
    out[k] = a[k] / b[k];
}

uint32_t probe_blocks(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return (uint32_t)(b < 8192 ? (b < 1 ? 1 : b) : 8192);
}

}  // namespace

extern "C" int zfi_sqrt_probe(float* out, int64_t n, uint32_t first_bits, void* stream_handle) {
  if (!out || n < 0 || n > (int64_t)0x100000000LL - (int64_t)first_bits) return -1;
  if (reinterpret_cast<uintptr_t>(out) & 3u) return -1;
  if (n == 0) return 0;
  (void)hipGetLastError();
  hipLaunchKernelGGL(sqrt_probe, dim3(probe_blocks(n)), dim3(256), 0,
                     static_cast<hipStream_t>(stream_handle), out, n, first_bits);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int zfi_div_probe(const float* a, const float* b, float* out, int64_t n,
                             void* stream_handle) {
  if (!a || !b || !out || n < 0) return -1;
  const uintptr_t mis = reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b) |
                        reinterpret_cast<uintptr_t>(out);
  if (mis & 3u) return -1;
  if (n == 0) return 0;
  (void)hipGetLastError();
  hipLaunchKernelGGL(div_probe, dim3(probe_blocks(n)), dim3(256), 0,
                     static_cast<hipStream_t>(stream_handle), a, b, out, n);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}
