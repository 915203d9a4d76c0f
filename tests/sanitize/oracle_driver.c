/* Drives every oracle function on small inputs (padding, N = 1, injected
 * overflow, empty ranges, every layout) so that a build with AddressSanitizer
 * and UndefinedBehaviorSanitizer can report any out-of-bounds access or
 * undefined operation.  Values are checked by the pin suite, not here; the
 * few asserts only keep the calls meaningful.  Test infrastructure. */
#include <assert.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "zf_oracle.h"

#define MAXU 16

static void* xcalloc(size_t n, size_t s) {
  void* p = calloc(n ? n : 1, s);
  assert(p);
  return p;
}

static void run_layout(int32_t n, int32_t layout, const int64_t* numel, const int32_t* unit,
                       int64_t nseg, int32_t gdt) {
  or_unit units[MAXU];
  int64_t nu, psi, psi_pad, s_tot = 0, i, u;
  int32_t r, k;
  uint16_t** grads = xcalloc((size_t)n, sizeof(uint16_t*));
  float **master = xcalloc((size_t)n, sizeof(float*)), **m = xcalloc((size_t)n, sizeof(float*));
  float **v = xcalloc((size_t)n, sizeof(float*)), **gs = xcalloc((size_t)n, sizeof(float*));
  uint16_t** shards = xcalloc((size_t)n, sizeof(uint16_t*));
  or_hparams hp = {1e-3, 0.9, 0.999, 1e-8, 0.01, 0.5};
  or_scale_state st = {1024.0, 0, 0, 2000, 1, 0};
  or_result res;
  int64_t ab, peak;
  if (layout == 2) {
    int64_t rows[8];
    for (i = 0; i < nseg; ++i) rows[i] = (i % 2) ? 0 : (numel[i] % 3 == 0 ? numel[i] / 3 : 1);
    assert(or_layout_dim0(numel, rows, nseg, n, units, MAXU, &nu, &psi, &psi_pad) == 0);
  } else {
    assert(or_layout(numel, unit, nseg, n, layout, units, MAXU, &nu, &psi, &psi_pad) == 0);
  }
  for (u = 0; u < nu; ++u) s_tot += units[u].S;
  for (k = 0; k <= 4; ++k) assert(or_ledger(units, nu, n, k, &ab, &peak) == 0);
  for (k = 0; k < 5; ++k) (void)or_comm_bytes(psi_pad, n, k);
  for (r = 0; r < n; ++r) {
    grads[r] = xcalloc((size_t)psi_pad, 2);
    for (u = 0; u < nu; ++u)
      or_gen16(grads[r] + units[u].O, units[u].L, gdt, 7, (1u << 20) | (unsigned)r,
               units[u].lam, 1e-2, 1024.0);
    master[r] = xcalloc((size_t)s_tot, 4);
    m[r] = xcalloc((size_t)s_tot, 4);
    v[r] = xcalloc((size_t)s_tot, 4);
    gs[r] = xcalloc((size_t)s_tot, 4);
    shards[r] = xcalloc((size_t)s_tot, 2);
    or_gen32(master[r], s_tot, 7, 1ull << 40, 0, 0.02);
  }
  {
    uint16_t* full = xcalloc((size_t)psi_pad, 2);
    uint16_t* unit_buf = xcalloc((size_t)psi_pad, 2);
    float* acc = xcalloc((size_t)psi_pad, 4);
    for (k = 0; k < 3; ++k) {
      if (layout == 2) {
        assert(or_fsdp2_step(gdt, n, units, nu, (const uint16_t* const*)grads, master, m, v, gs,
                             &hp, &st, &res) == 0);
        assert(or_fsdp2_gather(units, nu, n, 0, nu, gdt, (const float* const*)master,
                               unit_buf) == 0);
      } else {
        assert(or_zero_step(gdt, gdt, n, units, nu, k == 2 ? 3 : 2,
                            (const uint16_t* const*)grads, master, m, v, full, shards, &hp, &st,
                            &res) == 0);
        for (u = 0; u < nu; ++u)
          assert(or_gather_unit(units, nu, n, u, (const uint16_t* const*)shards, unit_buf) == 0);
      }
      /* buckets and accumulation over the same units */
      for (u = 0; u < nu; ++u)
        assert(or_rs_accumulate(gdt, n, units, nu, u, (const void* const*)grads, gs, k > 0) == 0);
      for (r = 0; r < n; ++r) {
        or_widen_array(gdt, psi_pad, grads[r], acc);
        assert(or_local_accumulate(gdt, psi_pad, grads[r], acc, 1) == 0);
      }
      assert(or_step_reduced(gdt, n, units, nu, 3, gs, master, m, v, NULL, NULL, &hp, &st,
                             &res) == 0);
    }
    /* an injected overflow */
    grads[n - 1][units[0].O] = 0x7C00;
    assert(or_zero_step(gdt, gdt, n, units, nu, 2, (const uint16_t* const*)grads, master, m, v,
                        full, shards, &hp, &st, &res) == 0);
    free(full);
    free(unit_buf);
    free(acc);
  }
  for (r = 0; r < n; ++r) {
    free(grads[r]);
    free(master[r]);
    free(m[r]);
    free(v[r]);
    free(gs[r]);
    free(shards[r]);
  }
  free(grads);
  free(master);
  free(m);
  free(v);
  free(gs);
  free(shards);
}

int main(void) {
  int64_t numel[] = {37, 5, 101, 64, 3, 9};
  int32_t unit[] = {0, 1, 1, 2, 3, 4};
  int32_t ids[6];
  int64_t nb, i, idx[5] = {0, 1, 17, 100, 212};
  int32_t ns[] = {1, 2, 3, 5, 8};
  uint64_t s = 42;
  float f[300], acc5[5];
  uint16_t h[300];
  double ss;
  int32_t nf;
  or_scalars sc;
  or_result res;
  or_hparams hp = {1e-3, 0.9, 0.999, 1e-8, 0.01, 1.0};
  or_scale_state st = {1.0, 0, 0, 2000, 0, 0};
  or_inject inj = {2, 1, 17, 0x7F80, {0, 0, 0}};
  size_t j;
  for (j = 0; j < sizeof ns / sizeof ns[0]; ++j) {
    run_layout(ns[j], 0, numel, unit, 6, 1);
    run_layout(ns[j], 1, numel, unit, 6, 2);
    run_layout(ns[j], 2, numel, unit, 6, 2);
  }
  assert(or_bucket_assign(numel, 6, 2, 40, ids, &nb) == 0);
  assert(or_bucket_assign(numel, 6, 64, 0, ids, &nb) == 0);
  (void)or_splitmix64_next(&s);
  or_gen32(f, 300, 1, 5, 0, 1.0);
  or_cast_array(1, 300, f, h);
  or_cast_array(2, 300, f, h);
  for (i = 0; i < 300; ++i) (void)or_f16_to_f32(h[i]);
  assert(or_regen_accum_sumsq(1, 3, 4, 1, 9, 2, 1e-2, 1024.0, 0, 300, &inj, &ss, &nf) == 0);
  assert(or_regen_accum_acc(2, 2, 3, 0, 9, 2, 1e-2, 1.0, 5, idx, &inj, acc5) == 0);
  assert(or_regen_sumsq(1, 2, 9, 1, 1e-2, 1.0, 10, 10, NULL, &ss, &nf) == 0);
  assert(or_finish(1.0, 0, 2, &hp, &st, &sc, &res) == 0);
  assert(or_finish(INFINITY, 1, 2, &hp, &st, &sc, &res) == 0);
  puts("oracle driver: ok");
  return 0;
}
