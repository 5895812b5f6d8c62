// Drives the host-side paths of the C ABI (include/la.h) that run before anything reaches
// the device: argument validation of every entry point with fake device addresses (never
// dereferenced: every such call is rejected), and the host-only queries (workspace size,
// segment plan) over a sweep of shapes up to 2^40 tokens.  Built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_sanitizers.py); exit status 0 when
// every call returned what it should.  Test infrastructure.
#include <stdint.h>
#include <stdio.h>

#include "la.h"

static int fails = 0;
#define EXPECT(cond)                                                       \
  do {                                                                     \
    if (!(cond)) {                                                         \
      fprintf(stderr, "failed: %s (line %d)\n", #cond, __LINE__);          \
      ++fails;                                                             \
    }                                                                      \
  } while (0)

static void *F(uintptr_t a) { return (void *)(a << 20); }  // fake, 16-byte aligned

int main() {
  const int variants[] = {LA_ADDITIVE, LA_BASED, LA_GATED, LA_GATED_DELTA, LA_BASED_COMPACT};
  const int64_t Ts[] = {0, 1, 63, 64, 65, 4096, 65536, 1 << 20, (int64_t)1 << 30, (int64_t)1 << 40};
  const int widths[][2] = {{16, 64}, {64, 64}, {128, 128}, {256, 256}, {64, 17}, {128, 40}};
  // host-only queries over shapes: no launch, no device memory
  for (int var : variants)
    for (int dt = 0; dt < 2; ++dt)
      for (int64_t T : Ts)
        for (auto &w : widths)
          for (int BH : {1, 2, 16, 300, 4096}) {
            size_t bytes = 0;
            const int st = la_prefill_workspace_size(var, dt, 1, BH, T, w[0], w[1], &bytes);
            EXPECT(st == LA_OK || st == LA_ERR_UNSUPPORTED);
            int ns = -1, cps = -1;
            const int st2 = la_prefill_segments(var, dt, 1, BH, T, w[0], w[1], &ns, &cps);
            EXPECT(st2 == st);
            if (st2 == LA_OK) EXPECT(ns >= 1 && cps >= 0 && (int64_t)ns * cps * 64 >= (ns > 1 ? T : 0));
          }
  size_t b = 0;
  EXPECT(la_prefill_workspace_size(LA_GATED_DELTA, LA_BF16, 1, 1, 10, 128, 128, nullptr) == LA_ERR_NULL);
  EXPECT(la_prefill_workspace_size(LA_GATED_DELTA, LA_BF16, 0, 1, 10, 128, 128, &b) == LA_ERR_INVALID);
  EXPECT(la_prefill_workspace_size(LA_GATED_DELTA, LA_BF16, 1, 1, -1, 128, 128, &b) == LA_ERR_INVALID);
  EXPECT(la_prefill_workspace_size(LA_GATED_DELTA, LA_BF16, 1 << 16, 1 << 16, 10, 128, 128, &b) ==
         LA_ERR_UNSUPPORTED);
  EXPECT(la_prefill_workspace_size(9, LA_BF16, 1, 1, 10, 128, 128, &b) == LA_ERR_INVALID);

  // prefill: every rejection before a launch
  void *q = F(1), *k = F(2), *v = F(3), *al = F(4), *be = F(5), *o = F(6), *ws = F(64);
  float *S = (float *)F(8), *S0 = (float *)F(10);
  size_t need = 0;
  la_prefill_workspace_size(LA_GATED_DELTA, LA_BF16, 1, 2, 1000, 128, 128, &need);
  EXPECT(need > 0);
  // missing workspace, too small, misaligned, aliasing, forbidden / missing gate pointers
  EXPECT(la_prefill(LA_GATED_DELTA, LA_BF16, 1, 2, 1000, 128, 128, 0, q, k, v, al, be, S0, nullptr, o, S, nullptr,
                    nullptr, 0, nullptr) == LA_ERR_WORKSPACE);
  EXPECT(la_prefill(LA_GATED_DELTA, LA_BF16, 1, 2, 1000, 128, 128, 0, q, k, v, al, be, S0, nullptr, o, S, nullptr, ws,
                    need - 1, nullptr) == LA_ERR_WORKSPACE);
  EXPECT(la_prefill(LA_GATED_DELTA, LA_BF16, 1, 2, 1000, 128, 128, 0, (char *)q + 2, k, v, al, be, S0, nullptr, o, S,
                    nullptr, ws, need, nullptr) == LA_ERR_ALIGN);
  EXPECT(la_prefill(LA_GATED_DELTA, LA_BF16, 1, 2, 1000, 128, 128, 0, q, k, v, al, be, S0, nullptr, q, S, nullptr, ws,
                    need, nullptr) == LA_ERR_ALIAS);
  EXPECT(la_prefill(LA_GATED_DELTA, LA_BF16, 1, 2, 1000, 128, 128, 0, q, k, v, al, be, S0, nullptr, o, S, nullptr,
                    (char *)o + 64, need, nullptr) == LA_ERR_ALIAS);
  EXPECT(la_prefill(LA_GATED_DELTA, LA_BF16, 1, 2, 1000, 128, 128, 0, q, k, v, al, nullptr, S0, nullptr, o, S, nullptr,
                    ws, need, nullptr) == LA_ERR_NULL);
  EXPECT(la_prefill(LA_ADDITIVE, LA_BF16, 1, 2, 1000, 128, 128, 0, q, k, v, al, nullptr, S0, nullptr, o, S, nullptr,
                    ws, need, nullptr) == LA_ERR_INVALID);
  EXPECT(la_prefill(LA_BASED, LA_BF16, 1, 2, 1000, 16, 64, 0, q, k, v, nullptr, nullptr, S0, nullptr, o, S, nullptr,
                    ws, need, nullptr) == LA_ERR_INVALID);  // s0 without z0
  EXPECT(la_prefill(LA_GATED_DELTA, LA_BF16, 1, 2, 1000, 96, 96, 0, q, k, v, al, be, S0, nullptr, o, S, nullptr, ws,
                    need, nullptr) == LA_ERR_UNSUPPORTED);
  EXPECT(la_prefill_pass(7, LA_GATED_DELTA, LA_BF16, 1, 2, 1000, 128, 128, 0, q, k, v, al, be, S0, nullptr, o, S,
                         nullptr, ws, need, nullptr) == LA_ERR_INVALID);
  EXPECT(la_prefill_noalloc(LA_GATED_DELTA, LA_BF16, 1, 8, (int64_t)1 << 20, 256, 256, 0, q, k, v, al, be, S0,
                            nullptr, o, S, nullptr, nullptr) == LA_ERR_WORKSPACE);

  // decode
  EXPECT(la_decode_step(LA_GATED_DELTA, LA_BF16, 0, 128, 128, 0, S0, nullptr, S, nullptr, q, k, v, al, be, o,
                        nullptr) == LA_ERR_INVALID);
  EXPECT(la_decode_step(LA_GATED_DELTA, LA_BF16, 8, 128, 128, 0, S0, nullptr, S, nullptr, q, k, v, nullptr, be, o,
                        nullptr) == LA_ERR_NULL);
  EXPECT(la_decode_step(LA_GATED_DELTA, LA_BF16, 8, 128, 128, 0, S0, nullptr, S, nullptr, q, k, v, al, be,
                        (char *)S + 8, nullptr) == LA_ERR_ALIAS);
  EXPECT(la_decode_step(LA_BASED, LA_BF16, 8, 16, 64, 0, S0, nullptr, S, nullptr, q, k, v, nullptr, nullptr, o,
                        nullptr) == LA_ERR_NULL);
  EXPECT(la_decode_step(LA_GATED_DELTA, LA_BF16, 8, 100, 128, 0, S0, nullptr, S, nullptr, q, k, v, al, be, o,
                        nullptr) == LA_ERR_UNSUPPORTED);

  // NoteBank steps and state scaling
  float *dh = (float *)F(20), *dm = (float *)F(21);
  EXPECT(la_write_scores(LA_BF16, 1, 2, 100, 128, 0, k, dh, dm, nullptr) == LA_ERR_INVALID);
  EXPECT(la_write_scores(LA_BF16, 1, 2, 100, 100, 32, k, dh, dm, nullptr) == LA_ERR_UNSUPPORTED);
  EXPECT(la_write_scores(LA_BF16, 1, 2, 100, 128, 32, k, (float *)k, dm, nullptr) == LA_ERR_ALIAS);
  EXPECT(la_write_windows(1, 100, 32, 8, 40, dm, (int64_t *)F(22), (float *)F(23), nullptr) == LA_ERR_INVALID);
  EXPECT(la_note_addresses(LA_BF16, 1, 17, 100, 128, 4, 16, dh, q, (const int64_t *)F(24), (const int32_t *)F(25),
                           (int64_t *)F(26), F(27), nullptr) == LA_ERR_UNSUPPORTED);
  EXPECT(la_address_votes(LA_BF16, 4, 3, 5, 12, F(30), F(31), 2, (const int64_t *)F(32), (float *)F(33),
                          (int32_t *)F(34), (int32_t *)F(35), (int32_t *)F(36), nullptr) == LA_ERR_UNSUPPORTED);
  EXPECT(la_state_scale(16, 1.5f, S0, S, nullptr) == LA_ERR_INVALID);
  EXPECT(la_state_scale(16, 0.5f, S0, (float *)((char *)S0 + 16), nullptr) == LA_ERR_ALIAS);
  EXPECT(la_state_scale(16, 0.5f, nullptr, S, nullptr) == LA_ERR_NULL);
  for (int st = -8; st <= 1; ++st) EXPECT(la_status_string(st) != nullptr);
  if (fails) fprintf(stderr, "%d expectation(s) failed\n", fails);
  else printf("abi driver: all calls as expected\n");
  return fails ? 1 : 0;
}
