/*
 * zf_inputs.h -- seeded synthetic inputs on the GPU (a library of its own).
 *
 * Not part of the step: it only fills device buffers with reproducible
 * pseudo-random values, so that the step can be driven at full model size
 * without host traffic.  It holds no arithmetic of the step.
 *
 * Definition (implemented here and, independently, by the CPU oracle):
 *   splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
 *   generators", OOPSLA 2014) is used as a counter-based generator: output j
 *   of a generator whose state starts at s is mix64(s + (j+1)*0x9E3779B97F4A7C15).
 *   A stream's starting state is output number `stream` of the generator
 *   seeded with `seed`.  Element i of a stream takes outputs 3i, 3i+1, 3i+2,
 *   splits them into twelve 16-bit words k_0..k_11, and
 *       z = (k_0 + ... + k_11 - 393210) / 65536      (Irwin-Hall(12), exact)
 *   is a standard-normal stand-in bounded by +-6.  A 16-bit draw is
 *   RNE16((z * f32(sigma)) * f32(scale)), each product one binary32
 *   rounding; an fp32 draw is z * f32(sigma).
 * Element k of a fill has logical index logical_base + k, so a value depends
 * only on (seed, stream, logical index), never on where the buffer sits.
 */
#ifndef ZF_INPUTS_H
#define ZF_INPUTS_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Fill dst[0..n) (device, 16-bit, 2-byte aligned) with draws of `stream`.
 * dtype: 1 = fp16, 2 = bf16.  Enqueued on the hipStream_t `stream_handle`.
 * Returns 0, or -1 (bad argument) / -5 (HIP error). */
int zfi_fill_normal16(void* dst, int64_t n, int32_t dtype, uint64_t seed, uint64_t stream,
                      int64_t logical_base, double sigma, double scale, void* stream_handle);

/* Fill dst[0..n) (device fp32, 4-byte aligned) with z * f32(sigma). */
int zfi_fill_normal32(float* dst, int64_t n, uint64_t seed, uint64_t stream,
                      int64_t logical_base, double sigma, void* stream_handle);

/* Output j of `stream`'s splitmix64 generator (host computation). */
uint64_t zfi_stream_output(uint64_t seed, uint64_t stream, uint64_t j);

/* Bandwidth probe for the bench (no arithmetic of the step): dst[k][i] =
 * src[0][i] + ... + src[n_src-1][i] for every destination k < n_dst and
 * i < n, in the access pattern of the step's kernels (16-byte loads and
 * non-temporal 16-byte stores per lane, 4-element quads 256 apart per lane,
 * one tile of 512 quads per block), so that a plain copy (1 source, 1
 * destination) and the update pass's mix (4 and 4) can be timed on the
 * GPU that runs the step.  n_src and n_dst in 1..8; every pointer 16-byte
 * aligned; n a multiple of 4.  Returns 0, -1 (bad argument) or -5. */
int zfi_stream_probe(const float* const* src, int32_t n_src, float* const* dst, int32_t n_dst,
                     int64_t n, void* stream_handle);

/* The same probe in a chosen shape, to find the GPU's best figure for an
 * access mix: `quads` (1, 2 or 4) quads per lane per 256-thread block,
 * non-temporal loads as well as stores, and at most `blocks_per_cu` (1..8;
 * 0: no limit) resident blocks per compute unit.  Arguments otherwise as
 * zfi_stream_probe.  Returns 0, -1 (bad argument) or -5. */
int zfi_stream_probe_shaped(const float* const* src, int32_t n_src, float* const* dst,
                            int32_t n_dst, int64_t n, int32_t quads, int32_t blocks_per_cu,
                            void* stream_handle);

/* Probe of the update pass's bytes with none of its arithmetic, so that the
 * update pass can be compared with a kernel that only moves what it moves:
 * per element, either two 16-bit arrays g0, g1 (the replicas an N = 2
 * update pass re-reads; sums NULL) or one fp32 array `sums` (materialised
 * sums; g0 = g1 = NULL) is read with plain loads, and p, m, v (fp32) are
 * read non-temporal and written back non-temporal: p[i] += x, m[i] += x,
 * v[i] += x in binary32, where x = bf16(g0[i]) + bf16(g1[i]) (the 16-bit
 * arrays read as bfloat16) or x = sums[i], and out16[i] = the top 16 bits
 * of the new p[i].  One 4-element quad per lane in blocks of
 * block_threads (128 or 256), at most blocks_per_cu (0: no limit, 1..8)
 * resident blocks per compute unit.  Device pointers, 16-byte aligned; n a
 * multiple of 4.  Returns 0, -1 (bad argument) or -5. */
int zfi_update_mix_probe(const void* g0, const void* g1, const float* sums, float* p, float* m,
                         float* v, void* out16, int64_t n, int32_t block_threads,
                         int32_t blocks_per_cu, void* stream_handle);

/* Lowering probes for tests (no arithmetic of the step): binary32 sqrt and
 * division exactly as this compiler emits them under the step library's
 * flags (-fhip-fp32-correctly-rounded-divide-sqrt, -ffp-contract=off).
 * zfi_sqrt_probe: out[i] = sqrtf(x) for the binary32 x whose bits are
 * first_bits + i, i < n, n <= 2^32 - first_bits.  zfi_div_probe: out[i] =
 * a[i] / b[i], i < n.  Device pointers, 4-byte aligned.  Returns 0, -1
 * (bad argument) or -5. */
int zfi_sqrt_probe(float* out, int64_t n, uint32_t first_bits, void* stream_handle);
int zfi_div_probe(const float* a, const float* b, float* out, int64_t n, void* stream_handle);

#ifdef __cplusplus
}
#endif
#endif
