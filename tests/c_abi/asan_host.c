/* Host-side checks of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.
 *
 * Built by tests/test_asan_host.py with the sanitizers on the host code only; every call
 * below returns from its host-side argument checks before any HIP call, so no GPU is
 * needed and no device pointer is ever dereferenced (the "pointers" are small integers).
 * Covers: moonep_query over a sweep of sizes, including limits and int32 overflow,
 * checked against the rules moonep.h states and against the layout's own invariants;
 * every entry point's argument-error paths; moonep_strerror for every code; the stream
 * library's argument checks. */
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moonep.h"
#include "moonep_streams.h"

static int g_checks = 0, g_fails = 0;
#define EXPECT(cond)                                                          \
  do {                                                                        \
    ++g_checks;                                                               \
    if (!(cond)) {                                                            \
      ++g_fails;                                                              \
      if (g_fails < 20) printf("FAIL line %d: %s\n", __LINE__, #cond);        \
    }                                                                         \
  } while (0)

/* the rules of moonep_query as moonep.h states them */
static int expected_rc(long R, long E, long K, long S, long slots) {
  if (R < 1 || E < 1 || K < 1 || S < 1 || slots < 0 || E % R != 0 || K > E) return MOONEP_EINVAL;
  if (R > MOONEP_MAX_R || E > MOONEP_MAX_E || K > MOONEP_MAX_K || slots > MOONEP_MAX_SLOTS)
    return MOONEP_ELIMIT;
  const long long C = (long long)S * K;
  const long long G = E / R + slots;
  const long long NvS = (C + G * (MOONEP_ROW_ALIGN - 1) + MOONEP_ROW_ALIGN - 1) /
                        MOONEP_ROW_ALIGN * MOONEP_ROW_ALIGN;
  const long long A = (long long)R * S * K;
  if (C > INT_MAX || NvS * R > INT_MAX || A > INT_MAX) return MOONEP_ELIMIT;
  return MOONEP_OK;
}

static void check_layout(const moonep_sizes* s) {
  EXPECT(s->E_loc * s->R == s->E);
  EXPECT(s->C == s->S * s->K);
  EXPECT(s->NvS % MOONEP_ROW_ALIGN == 0 && s->NvS >= s->C);
  EXPECT(s->T == (int64_t)s->R * s->S && s->A == s->T * s->K);
  EXPECT(s->recv_rows == (int64_t)s->R * s->NvS);
  EXPECT(s->P_max == s->E + s->R);
  EXPECT(s->nblk >= 1 && (int64_t)s->nblk * s->blk >= s->A && (int64_t)(s->nblk - 1) * s->blk < s->A);
  const int64_t offs[] = {s->o_hdr, s->o_load, s->o_shed, s->o_keep, s->o_home_row, s->o_pfirst,
                          s->o_pnum, s->o_pieces, s->o_slot_expert, s->o_off, s->o_red, s->o_xtab,
                          s->o_ptab, s->o_dst_row, s->o_w};
  const int n = (int)(sizeof(offs) / sizeof(offs[0]));
  for (int i = 0; i < n; ++i) {
    EXPECT(offs[i] % 64 == 0);                        /* 256-byte aligned arrays */
    if (i > 0) EXPECT(offs[i] > offs[i - 1]);
  }
  EXPECT(s->o_w + s->A <= s->plan_bytes / 4);
  EXPECT(s->workspace_bytes > 0 && s->workspace_bytes % 4 == 0);
}

int main(void) {
  /* 1. sizes */
  const long vals[] = {-1, 0, 1, 2, 3, 4, 7, 8, 16, 24, 63, 64, 65, 128, 255, 256, 257, 384,
                       1023, 1024, 1025, 4096, 1L << 16, 1L << 20, 1L << 26, INT_MAX};
  const int nv = (int)(sizeof(vals) / sizeof(vals[0]));
  for (int a = 0; a < nv; ++a)
    for (int b = 0; b < nv; ++b)
      for (int c = 0; c < nv; c += 2)
        for (int d = 0; d < nv; d += 3)
          for (int e = 0; e < nv; e += 5) {
            const long R = vals[a], E = vals[b], K = vals[c], S = vals[d], slots = vals[e];
            if (R > INT_MAX || E > INT_MAX) continue;
            moonep_sizes s;
            memset(&s, 0xA5, sizeof(s));
            const int rc = moonep_query((int)R, (int)E, (int)K, (int)S, (int)slots, &s);
            EXPECT(rc == expected_rc(R, E, K, S, slots));
            if (rc == MOONEP_OK) check_layout(&s);
          }
  EXPECT(moonep_query(4, 16, 2, 4, 4, NULL) == MOONEP_EINVAL);

  /* 2. argument errors: host checks only, nothing reaches HIP */
  void* fake = (void*)(uintptr_t)256;                 /* never dereferenced */
  void* odd = (void*)(uintptr_t)260;
  moonep_plan_desc d;
  memset(&d, 0, sizeof(d));
  EXPECT(moonep_plan(NULL, fake, 4, 16, 2, 4, 4, fake, fake, &d, 0) == MOONEP_EINVAL);
  EXPECT(moonep_plan(fake, fake, 4, 16, 2, 4, 4, fake, fake, NULL, 0) == MOONEP_EINVAL);
  EXPECT(moonep_plan(fake, fake, 3, 16, 2, 4, 4, fake, fake, &d, 0) == MOONEP_EINVAL);
  EXPECT(moonep_plan(fake, fake, 65, 65, 2, 4, 4, fake, fake, &d, 0) == MOONEP_ELIMIT);
  EXPECT(moonep_plan(fake, fake, 4, 16, 2, 4, 4, odd, fake, &d, 0) == MOONEP_EALIGN);
  EXPECT(moonep_plan(fake, fake, 4, 16, 2, 4, 4, fake, odd, &d, 0) == MOONEP_EALIGN);
  EXPECT(moonep_plan(fake, (void*)(uintptr_t)258, 4, 16, 2, 4, 4, fake, fake, &d, 0) == MOONEP_EALIGN);
  EXPECT(moonep_plan_noalloc(NULL, fake, 4, 16, 2, 4, 4, fake, &d, 0) == MOONEP_EINVAL);
  EXPECT(moonep_plan_noalloc(fake, fake, 64, 1024, 32, 1 << 13, 8, fake, &d, 0) == MOONEP_ELIMIT);
  EXPECT(moonep_plan_noalloc(fake, fake, 4, 16, 2, 4, 4, odd, &d, 0) == MOONEP_EALIGN);

  /* an uninitialised descriptor is refused by every call that takes one */
  moonep_plan_stats st;
  EXPECT(moonep_dispatch(&d, fake, 16, fake, 0) == MOONEP_EPLAN);
  EXPECT(moonep_dispatch(NULL, fake, 16, fake, 0) == MOONEP_EPLAN);
  EXPECT(moonep_combine(&d, fake, 16, fake, 0) == MOONEP_EPLAN);
  EXPECT(moonep_dispatch_staged(&d, fake, 16, fake, fake, 0) == MOONEP_EPLAN);
  EXPECT(moonep_combine_staged(&d, fake, 16, fake, fake, 0) == MOONEP_EPLAN);
  EXPECT(moonep_dispatch_bwd(&d, fake, 16, fake, 0) == MOONEP_EPLAN);
  EXPECT(moonep_combine_bwd(&d, fake, fake, 16, fake, fake, 0) == MOONEP_EPLAN);
  EXPECT(moonep_reduce_grad(&d, fake, fake, 16, 0) == MOONEP_EPLAN);
  EXPECT(moonep_prefetch_weight(&d, fake, 16, fake, 0) == MOONEP_EPLAN);
  EXPECT(moonep_expert_stub(&d, fake, fake, fake, fake, 16, 16, fake, 0) == MOONEP_EPLAN);
  EXPECT(moonep_plan_status(&d, &st, 0) == MOONEP_EPLAN);

  /* a well-formed descriptor (sizes from moonep_query), then per-call argument errors */
  d.magic = 0x4D4F4E45u;
  d.dev = fake;
  EXPECT(moonep_query(4, 16, 2, 4, 4, &d.sz) == MOONEP_OK);
  EXPECT(moonep_dispatch(&d, NULL, 16, fake, 0) == MOONEP_EINVAL);
  EXPECT(moonep_dispatch(&d, fake, 12, fake, 0) == MOONEP_EINVAL);      /* H % 8 */
  EXPECT(moonep_dispatch(&d, fake, 0, fake, 0) == MOONEP_EINVAL);
  EXPECT(moonep_dispatch(&d, odd, 16, fake, 0) == MOONEP_EALIGN);
  EXPECT(moonep_combine(&d, fake, 16, NULL, 0) == MOONEP_EINVAL);
  EXPECT(moonep_combine(&d, fake, 16, odd, 0) == MOONEP_EALIGN);
  EXPECT(moonep_dispatch_staged(&d, fake, 16, NULL, fake, 0) == MOONEP_EINVAL);
  EXPECT(moonep_dispatch_staged(&d, fake, 16, odd, fake, 0) == MOONEP_EALIGN);
  EXPECT(moonep_combine_staged(&d, fake, 16, fake, NULL, 0) == MOONEP_EINVAL);
  EXPECT(moonep_dispatch_bwd(&d, fake, 20, fake, 0) == MOONEP_EINVAL);
  EXPECT(moonep_combine_bwd(&d, fake, fake, 16, fake, NULL, 0) == MOONEP_EINVAL);
  EXPECT(moonep_combine_bwd(&d, fake, fake, 16, fake, (void*)(uintptr_t)257, 0) == MOONEP_EALIGN);
  EXPECT(moonep_reduce_grad(&d, NULL, fake, 16, 0) == MOONEP_EINVAL);
  EXPECT(moonep_reduce_grad(&d, fake, fake, 6, 0) == MOONEP_EINVAL);     /* G_el % 4 */
  EXPECT(moonep_reduce_grad(&d, fake, NULL, 16, 0) == MOONEP_EINVAL);    /* slots > 0 */
  EXPECT(moonep_reduce_grad(&d, odd, fake, 16, 0) == MOONEP_EALIGN);
  EXPECT(moonep_prefetch_weight(&d, fake, 12, fake, 0) == MOONEP_EINVAL);
  EXPECT(moonep_prefetch_weight(&d, fake, 16, NULL, 0) == MOONEP_EINVAL);
  EXPECT(moonep_expert_stub(&d, fake, fake, fake, fake, 8, 16, fake, 0) == MOONEP_EINVAL); /* W_el < H */
  EXPECT(moonep_plan_status(&d, NULL, 0) == MOONEP_EINVAL);
  /* tampered sizes */
  d.sz.NvS += 16;
  EXPECT(moonep_dispatch(&d, fake, 16, fake, 0) == MOONEP_EPLAN);
  d.sz.NvS -= 16;
  d.sz.o_w += 64;
  EXPECT(moonep_combine(&d, fake, 16, fake, 0) == MOONEP_EPLAN);

  /* 3. error strings */
  const int codes[] = {MOONEP_OK, MOONEP_EINVAL, MOONEP_ELIMIT, MOONEP_EPLAN, MOONEP_EHIP,
                       MOONEP_EALIGN, -99, 1, INT_MIN};
  for (unsigned i = 0; i < sizeof(codes) / sizeof(codes[0]); ++i) {
    const char* m = moonep_strerror(codes[i]);
    EXPECT(m != NULL && strlen(m) > 0);
  }

  /* 4. the stream library's argument checks */
  EXPECT(moonep_stream_read(NULL, 4096, 1, 1, fake, 0) == -1);
  EXPECT(moonep_stream_read(fake, 4095, 1, 1, fake, 0) == -1);
  EXPECT(moonep_stream_read(fake, 4096, 2, 1, fake, 0) == -1);
  EXPECT(moonep_stream_write(fake, 4096, 1, 3, 0) == -1);
  EXPECT(moonep_stream_write(odd, 4096, 1, 1, 0) == -1);
  EXPECT(moonep_stream_copy(fake, fake, 0, 0, 0, 0) == -1);
  EXPECT(moonep_rows_fanout(fake, 4, 0, fake, fake, 8, 64, 1, 0) == -1);
  EXPECT(moonep_rows_fanout(fake, 4, 2, NULL, fake, 8, 64, 1, 0) == -1);
  EXPECT(moonep_rows_gather(fake, 4, 2, fake, 8, fake, 24, 1, 0) == -1);
  EXPECT(moonep_rows_gather(fake, 0, 2, fake, 8, fake, 64, 1, 0) == -1);
  EXPECT(moonep_rows_update(fake, 4, 2, fake, fake, fake, 8, 24, 0) == -1);   /* not 16 B */
  EXPECT(moonep_rows_update(fake, 4, 0, fake, fake, fake, 8, 64, 0) == -1);   /* K < 1 */
  EXPECT(moonep_rows_update(fake, 4, 2, fake, NULL, fake, 8, 64, 0) == -1);
  EXPECT(moonep_rows_update(fake, 4, 2, fake, fake, fake, 0, 64, 0) == -1);   /* no rows */

  printf("asan host %s: %d checks, %d failed\n", g_fails ? "FAILED" : "ok", g_checks, g_fails);
  return g_fails ? 1 : 0;
}
