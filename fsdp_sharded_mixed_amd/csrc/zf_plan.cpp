// zf_plan.cpp -- FlatParameter layout planner and model-state ledger (host).
//
// Layout (CMU 15-779 Lecture 13 notes, "Zero Redundancy and PyTorch FSDP",
// 5.2): the tensors of a unit are concatenated into one 1-D FlatParameter,
// right-padded with zeros to a multiple of the shard count N and split into
// N equal shards, shard r for rank r.  Femtotron dev log #6 shards the
// whole master as one giant 1-D vector (the global-flat layout); the notes'
// simulator (0.4) and FSDP use one unit per layer.  FSDP2 (Megatron /
// DeepSpeed / torchtitan source guide, 五.4) instead shards every parameter
// along dim 0 like torch.chunk, padding each rank's chunk to ceil(R/N) rows:
// one shard unit per parameter, padded at row granularity.
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <new>

#include "zf_internal.h"

namespace {

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Per-rank bytes of model state once backward has finished (notes 2.3, 3.5
// and the summary): 16-bit params (2 B), 16-bit grads (2 B) and fp32 master,
// exp_avg, exp_avg_sq (12 B) per element, full or 1/N depending on the
// stage; sharded stages count padded elements (notes 3.6).
void fill_ledger(zf_plan* p) {
  zf_plan_summary& s = p->summary;
  const int64_t full = s.psi_pad, shard = s.psi_pad / s.n_ranks;
  s.state_bytes[0] = (2 + 2 + 12) * s.psi;
  s.state_bytes[1] = 2 * full + 2 * full + 12 * shard;
  s.state_bytes[2] = 2 * full + 2 * shard + 12 * shard;
  s.state_bytes[3] = (2 + 2 + 12) * shard;
  // FSDP2 with fp32 parameters (source guide 五.6): the fp32 shard is the
  // parameter and the master; fp32 grad shard; m and v.
  s.state_bytes[4] = (4 + 4 + 8) * shard;
  // Stage-3 peak (notes, exercise 5): backward runs units last to first;
  // while it is in unit b a rank holds its resident shards (16-bit params
  // and fp32 states), the grad shards already reduce-scattered for the
  // units after b, and unit b's gathered params plus its full grads.
  int64_t peak = 0, reduced_after = 0;
  for (int64_t b = s.n_units - 1; b >= 0; --b) {
    const zf_unit_info& u = p->units[b];
    const int64_t here = (2 + 12) * shard + 2 * reduced_after + (2 + 2) * u.P;
    if (here > peak) peak = here;
    reduced_after += u.S;
  }
  s.stage3_peak_bytes = peak;
  // Ring traffic per rank (notes 4.1-4.2): each reduce-scatter or
  // all-gather pass over 2*Psi' bytes sends (N-1)/N of them.
  const double pass = 2.0 * (double)s.psi_pad * (double)(s.n_ranks - 1) / (double)s.n_ranks;
  s.comm_bytes[0] = 2 * pass;  // DP all-reduce = RS + AG
  s.comm_bytes[1] = 2 * pass;  // stage 1: RS grads + AG params
  s.comm_bytes[2] = 2 * pass;  // stage 2: same volume
  s.comm_bytes[3] = 3 * pass;  // stage 3: AG fwd + AG bwd + RS
  s.comm_bytes[4] = 3 * pass;  // slides' stage 1: AR grads + AG params
}

}  // namespace

extern "C" int zf_plan_flat(const zf_segment* segs, int64_t nseg, int32_t n_ranks,
                            int32_t layout, int32_t stage, zf_plan** out) {
  if (!out) return ZF_EINVAL;
  *out = nullptr;
  if (!segs || nseg < 1) return ZF_EINVAL;
  if (layout != ZF_GLOBAL_FLAT && layout != ZF_PER_UNIT && layout != ZF_PER_PARAM_DIM0)
    return ZF_EINVAL;
  if (stage < 0 || stage > 3) return ZF_EINVAL;
  if (n_ranks < 1 || n_ranks > ZF_MAX_RANKS) return ZF_ESIZE;

  zf_plan* p = new (std::nothrow) zf_plan();
  if (!p) return ZF_ENOMEM;
  p->magic = zf::kPlanMagic;
  std::memset(&p->summary, 0, sizeof(p->summary));
  const int64_t kLimit = int64_t(1) << 62;
  int64_t lam = 0;
  int32_t cur = -1;
  try {
    for (int64_t i = 0; i < nseg; ++i) {
      const int32_t uid = (layout == ZF_GLOBAL_FLAT) ? 0 : segs[i].unit;
      if (segs[i].numel < 1) { delete p; return ZF_EINVAL; }
      if (segs[i].numel > kLimit - lam) { delete p; return ZF_ESIZE; }
      if (uid != cur) {
        if (uid != cur + 1) { delete p; return ZF_EINVAL; }
        zf_group_info g{};
        g.first_unit = (int64_t)p->units.size();
        p->groups.push_back(g);
        if (layout != ZF_PER_PARAM_DIM0) {
          zf_unit_info u{};
          u.lam = lam;
          p->units.push_back(u);
        }
        cur = uid;
      }
      if (layout == ZF_PER_PARAM_DIM0) {
        // one unit per parameter; its rows carry the padding granularity
        const int64_t rows = segs[i].dim0 > 0 ? segs[i].dim0 : segs[i].numel;
        if (segs[i].numel % rows != 0) { delete p; return ZF_EINVAL; }
        zf_unit_info u{};
        u.lam = lam;
        u.L = segs[i].numel;
        const int64_t cols = segs[i].numel / rows;
        const int64_t chunk = (rows + n_ranks - 1) / n_ranks;
        u.S = chunk * cols;
        u.P = u.S * n_ranks;
        p->units.push_back(u);
      } else {
        p->units.back().L += segs[i].numel;
      }
      p->groups.back().n_units = (int64_t)p->units.size() - p->groups.back().first_unit;
      p->groups.back().numel += segs[i].numel;
      lam += segs[i].numel;
    }
  } catch (const std::bad_alloc&) {
    delete p;
    return ZF_ENOMEM;
  }
  int64_t off = 0, max_pad = 0;
  for (zf_unit_info& u : p->units) {
    if (layout != ZF_PER_PARAM_DIM0) {
      u.P = round_up(u.L, n_ranks);
      u.S = u.P / n_ranks;
    }
    if (u.P < u.L || u.P >= kLimit) { delete p; return ZF_ESIZE; }
    u.O = off;
    off += u.P;
    if (u.P > max_pad) max_pad = u.P;
    if (off >= kLimit) { delete p; return ZF_ESIZE; }
  }
  int64_t max_group = 0;
  for (zf_group_info& g : p->groups) {
    for (int64_t k = 0; k < g.n_units; ++k) g.padded += p->units[g.first_unit + k].P;
    if (g.numel > max_group) max_group = g.numel;
  }
  zf_plan_summary& s = p->summary;
  s.psi = lam;
  s.psi_pad = off;
  s.n_units = (int64_t)p->units.size();
  s.max_unit_pad = max_pad;
  s.n_groups = (int64_t)p->groups.size();
  s.max_group_numel = max_group;
  s.n_ranks = n_ranks;
  s.layout = layout;
  s.stage = stage;
  // Recompute the sums in the update pass (re-read 2N bytes per element)
  // unless writing and re-reading an fp32 copy (8 bytes) is cheaper.
  // ZF_PER_PARAM_DIM0 (FSDP2) keeps a resident fp32 gradient shard, which
  // holds the sums; otherwise they are recomputed from the replicas in the
  // update pass unless writing and re-reading an fp32 copy (8 bytes) is
  // cheaper than re-reading N replicas (2N bytes).
  s.policy = layout == ZF_PER_PARAM_DIM0 ? 2 : ((2 * n_ranks > 8) ? 1 : 0);

  const int64_t nq = s.psi_pad / 4;  // quads; the ragged tail rides on the last tile
  p->unr1 = zf::unr_pass1(n_ranks);
  p->pass1_map = zf::map_pass1(n_ranks);
  p->cached_sums_quads = zf::cached_sums_quads(s.psi_pad);
  s.cached_sums_bytes =
      s.policy != 0 ? std::min(s.psi_pad * 4, p->cached_sums_quads * 16) : 0;
  const int64_t q1 = (int64_t)zf::kThreads * zf::kQuadsPerUnr * p->unr1;
  const int64_t t1 = (nq + q1 - 1) / q1;
  p->pass1_tiles = t1 < 1 ? 1 : t1;
  // every launch grid must fit grid.x: pass 1's tiles and the update pass's
  // smallest tiles (zf::pass2_tiles with 128-thread blocks)
  if (p->pass1_tiles > 0x7FFFFFFF || zf::pass2_tiles(p, false) > 0x7FFFFFFF) {
    delete p;
    return ZF_ESIZE;
  }
  int64_t l2 = (p->pass1_tiles + zf::kThreads - 1) / zf::kThreads;
  if (l2 > zf::kMaxLevel2Blocks) l2 = zf::kMaxLevel2Blocks;
  p->level2_blocks = (int32_t)l2;
  p->ws_partials_offset = 0;
  int64_t ws = round_up(p->pass1_tiles * 16, 256);
  p->ws_partials2_offset = ws;
  ws += round_up(l2 * 16, 256);
  p->ws_partials_bytes = ws;
  p->ws_rs_offset = -1;
  if (s.policy == 1) {
    p->ws_rs_offset = ws;
    ws += round_up(s.psi_pad * 4, 256);
  }
  s.workspace_bytes = ws;
  fill_ledger(p);
  *out = p;
  return ZF_OK;
}

// Megatron gradient buckets (source guide 三.3): consecutive parameters of
// the buffer fill a bucket until it holds bucket_numel elements (default
// max(40M, 1M * dp_size)); parameters are not split.
extern "C" int zf_plan_buckets(const int64_t* numel, int64_t nseg, int32_t n_ranks,
                               int64_t bucket_numel, int32_t* unit_out, int64_t* n_buckets) {
  if (!numel || !unit_out || !n_buckets || nseg < 1) return ZF_EINVAL;
  if (n_ranks < 1 || n_ranks > ZF_MAX_RANKS) return ZF_ESIZE;
  int64_t cap = bucket_numel;
  if (cap <= 0) {
    cap = int64_t(1000000) * n_ranks;
    if (cap < 40000000) cap = 40000000;
  }
  int64_t fill = 0;
  int32_t id = 0;
  for (int64_t i = 0; i < nseg; ++i) {
    if (numel[i] < 1) return ZF_EINVAL;
    if (numel[i] > std::numeric_limits<int64_t>::max() - fill) return ZF_ESIZE;
    unit_out[i] = id;
    fill += numel[i];
    if (fill >= cap && i + 1 < nseg) {
      if (id == std::numeric_limits<int32_t>::max()) return ZF_ESIZE;
      ++id;
      fill = 0;
    }
  }
  *n_buckets = (int64_t)id + 1;
  return ZF_OK;
}

extern "C" int zf_plan_info(const zf_plan* plan, zf_plan_summary* out) {
  if (!plan || plan->magic != zf::kPlanMagic || !out) return ZF_EINVAL;
  *out = plan->summary;
  return ZF_OK;
}

extern "C" int zf_plan_unit(const zf_plan* plan, int64_t u, zf_unit_info* out) {
  if (!plan || plan->magic != zf::kPlanMagic || !out) return ZF_EINVAL;
  if (u < 0 || u >= (int64_t)plan->units.size()) return ZF_EINVAL;
  *out = plan->units[u];
  return ZF_OK;
}

extern "C" int zf_plan_group(const zf_plan* plan, int64_t g, zf_group_info* out) {
  if (!plan || plan->magic != zf::kPlanMagic || !out) return ZF_EINVAL;
  if (g < 0 || g >= (int64_t)plan->groups.size()) return ZF_EINVAL;
  *out = plan->groups[g];
  return ZF_OK;
}

extern "C" void zf_plan_free(zf_plan* plan) {
  if (!plan || plan->magic != zf::kPlanMagic) return;
  plan->magic = 0;
  delete plan;
}

extern "C" int64_t zf_workspace_bytes(const zf_plan* plan) {
  if (!plan || plan->magic != zf::kPlanMagic) return ZF_EINVAL;
  return plan->summary.workspace_bytes;
}

extern "C" const char* zf_strerror(int status) {
  switch (status) {
    case ZF_OK: return "ok";
    case ZF_EINVAL: return "invalid argument";
    case ZF_EALIGN: return "pointer not 16-byte aligned";
    case ZF_EDTYPE: return "unknown dtype";
    case ZF_ESIZE: return "size out of range";
    case ZF_EHIP: return "HIP runtime error";
    case ZF_ENOMEM: return "host allocation failed";
    case ZF_EUNSUP: return "the host CPU lacks AVX2 or F16C (CPU-Adam)";
    default: return "unknown status";
  }
}
