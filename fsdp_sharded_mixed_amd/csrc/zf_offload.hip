// zf_offload.hip -- the ZeRO-Offload step: GPU reduction, PCIe both ways,
// CPU-Adam in between (host code; the kernels are the step's).
//
// CMU 15-779 Lecture 13 notes, "Zero Redundancy and PyTorch FSDP", 7.1-7.2:
// only the 16-bit parameters stay on the GPU; gradients go down, the CPU
// updates the fp32 state, and the new 16-bit parameters go up in chunks
// that overlap the CPU update of the next chunk.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "zf_hip_status.h"
#include "zf_internal.h"

namespace {

using zf::hip_ok;

constexpr int64_t kChunkAlign = 16;  // chunk starts: whole CPU-Adam vectors

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

void fill_result(const zf::DevState& h, zf_step_result* out) {
  if (!out) return;
  out->overflow = h.overflow;
  out->skipped = h.skipped;
  out->t = h.t;
  out->sumsq = h.sumsq;
  out->norm = h.norm;
  out->coef = h.coef;
  out->scale_used = h.scale_used;
  out->scale_next = h.loss_scale;
  out->gs = h.gs;
  out->growth_ctr = h.growth_ctr;
  out->bc1 = h.bc1;
  out->bc2 = h.bc2;
}

// The uploads run on a stream of their own, so that PCIe carries the
// parameters up while the sums still come down on the caller's stream.  One
// stream per device, made on first use (default priority, not blocking the
// legacy stream) and kept until the process ends.
hipStream_t upload_stream() {
  static std::mutex mu;
  static std::vector<hipStream_t> streams;
  int dev = 0;
  if (!hip_ok(hipGetDevice(&dev)) || dev < 0) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if ((size_t)dev >= streams.size()) streams.resize(dev + 1, nullptr);
  if (!streams[dev] && !hip_ok(hipStreamCreateWithFlags(&streams[dev], hipStreamNonBlocking)))
    streams[dev] = nullptr;
  return streams[dev];
}

}  // namespace

extern "C" int zf_offload_step(const zf_plan* plan, const zf_hparams* hp,
                               const zf_offload_args* a, void* stream, zf_step_result* result) {
  if (!plan || plan->magic != zf::kPlanMagic || !hp || !a) return ZF_EINVAL;
  if ((a->down16 != 0 && a->down16 != 1) || a->n_chunks < 1 || a->n_chunks > 4096)
    return ZF_EINVAL;
  const bool down16 = a->down16 == 1;
  // bytes per downloaded element: the fp32 sums, or the sums rounded to the
  // gradient dtype
  const int64_t eb = down16 ? 2 : 4;
  if (a->param_dtype != ZF_F16 && a->param_dtype != ZF_BF16) return ZF_EDTYPE;
  if (!a->params || !a->grad_shards || !a->h_state || !a->h_grad || !a->h_master ||
      !a->h_exp_avg || !a->h_exp_avg_sq || !a->h_params)
    return ZF_EINVAL;
  if (!aligned(a->params, 16) || !aligned(a->h_state, 16)) return ZF_EALIGN;
  const void* hf[] = {a->h_grad, a->h_master, a->h_exp_avg, a->h_exp_avg_sq};
  for (const void* q : hf)
    if (!aligned(q, 16)) return ZF_EALIGN;
  if (!aligned(a->h_params, 16)) return ZF_EALIGN;
  if (!zf::host_simd_ok()) return ZF_EUNSUP;
  const int64_t n = plan->summary.psi_pad;
  if (a->numel < n) return ZF_ESIZE;

  // the GPU side: pass 1, norm reduction, finish (validates the rest)
  zf_step_args s{};
  s.grad_dtype = a->grad_dtype;
  s.param_dtype = a->param_dtype;
  s.grads = a->grads;
  s.params = a->params;
  s.grad_shards = a->grad_shards;
  s.grads_reduced = a->grads_reduced;
  s.numel = a->numel;
  s.workspace = a->workspace;
  s.workspace_size = a->workspace_size;
  s.state = a->state;
  // the step records "before pass 1" and "after the finish" into ours
  void* step_events[4] = {nullptr, nullptr, nullptr, nullptr};
  if (a->phase_events) {
    step_events[0] = a->phase_events[0];
    step_events[2] = a->phase_events[1];
    s.phase_events = step_events;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  auto record = [&](int i) {
    if (!a->phase_events || !a->phase_events[i]) return true;
    return hip_ok(hipEventRecord(static_cast<hipEvent_t>(a->phase_events[i]), st));
  };
  int rc = zf::step_enqueue(plan, hp, &s, stream, false, down16);
  if (rc != ZF_OK) return rc;
  const int64_t C = std::min<int64_t>(a->n_chunks, (n + kChunkAlign - 1) / kChunkAlign);
  auto chunk = [&](int64_t c, int64_t& b, int64_t& e) {
    const int64_t blocks = (n + kChunkAlign - 1) / kChunkAlign;
    b = std::min(n, blocks * c / C * kChunkAlign);
    e = std::min(n, blocks * (c + 1) / C * kChunkAlign);
  };
  // down: the state block, then the sums chunk by chunk, each with an event
  std::vector<hipEvent_t> down(C, nullptr);
  // (`st` may be the legacy stream, whose handle is null)
  hipStream_t up = st;
  auto cleanup = [&]() {
    for (hipEvent_t& ev : down)
      if (ev) (void)hipEventDestroy(ev);
  };
  // an error after copies were enqueued: wait until none is still moving
  // data into the caller's buffers, then report it
  auto fail = [&]() {
    (void)hipStreamSynchronize(st);
    if (up != st) (void)hipStreamSynchronize(up);
    cleanup();
    return ZF_EHIP;
  };
  if (!hip_ok(hipMemcpyAsync(a->h_state, a->state, sizeof(zf::DevState), hipMemcpyDeviceToHost, st)))
    return fail();
  for (int64_t c = 0; c < C; ++c) {
    int64_t b, e;
    chunk(c, b, e);
    if (!hip_ok(hipEventCreateWithFlags(&down[c], hipEventDisableTiming)) ||
        !hip_ok(hipMemcpyAsync(reinterpret_cast<char*>(a->h_grad) + b * eb,
                               reinterpret_cast<const char*>(a->grad_shards) + b * eb,
                               (e - b) * eb, hipMemcpyDeviceToHost, st)) ||
        !hip_ok(hipEventRecord(down[c], st)))
      return fail();
  }
  if (!record(2)) return fail();
  // the state block arrived with the first chunk (same stream, earlier)
  if (!hip_ok(hipEventSynchronize(down[0]))) return fail();
  zf::DevState h;
  std::memcpy(&h, a->h_state, sizeof(h));
  if (!h.skipped && !(up = upload_stream())) {
    up = st;
    return fail();
  }
  if (!h.skipped) {
    uint16_t* hp16 = static_cast<uint16_t*>(a->h_params);
    char* dp16 = static_cast<char*>(a->params);
    for (int64_t c = 0; c < C; ++c) {
      int64_t b, e;
      chunk(c, b, e);
      if (!hip_ok(hipEventSynchronize(down[c]))) return fail();
      zf::cpu_adam_run(hp, h.gs, h.bc1, h.bc2, e - b,
                       reinterpret_cast<const char*>(a->h_grad) + b * eb,
                       down16 ? a->grad_dtype : ZF_F32, a->h_master + b, a->h_exp_avg + b,
                       a->h_exp_avg_sq + b, hp16 + b, a->param_dtype, a->n_threads);
      // up: this chunk's 16-bit parameters while the CPU takes the next one
      if (!hip_ok(hipMemcpyAsync(dp16 + 2 * b, hp16 + b, (e - b) * sizeof(uint16_t),
                                 hipMemcpyHostToDevice, up)))
        return fail();
    }
  }
  // every upload has landed before the caller's stream goes on
  const bool ok = hip_ok(hipStreamSynchronize(up)) && record(3) &&
                  hip_ok(hipStreamSynchronize(st));
  if (!ok) return fail();
  cleanup();
  fill_result(h, result);
  return ZF_OK;
}
