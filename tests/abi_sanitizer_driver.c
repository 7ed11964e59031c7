/* Host-side checks of the C ABI under AddressSanitizer and
 * UndefinedBehaviorSanitizer: every entry point is called with arguments that
 * fail validation (so nothing reaches the GPU), the pure queries with shapes
 * up to the int32 limits, and every returned status is compared with the
 * expected one.  Built and run by tests/test_host_sanitizers.py against a
 * host-only, sanitized build of the library sources.  Exit status 0 = all
 * checks passed. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mq.h"

static int failures = 0;

#define EXPECT(expr, want)                                                            \
  do {                                                                                \
    long long got_ = (long long)(expr);                                               \
    if (got_ != (long long)(want)) {                                                  \
      fprintf(stderr, "%s:%d: %s = %lld, want %lld\n", __FILE__, __LINE__, #expr, got_, \
              (long long)(want));                                                     \
      ++failures;                                                                     \
    }                                                                                 \
  } while (0)

/* fake, aligned device addresses: validation never dereferences them */
#define P(a) ((void*)(uintptr_t)(a))

static mq_packed packed(int32_t n, int32_t k) {
  mq_packed w;
  w.n = n;
  w.k = k;
  for (int p = 0; p < MQ_NPLANES; ++p) w.plane[p] = P(0x10000 + 0x1000 * p);
  return w;
}

static void status_strings(void) {
  for (int s = -3; s < 16; ++s) {
    const char* t = mq_status_str(s);
    EXPECT(t != NULL, 1);
    EXPECT(strlen(t) > 0, 1);
  }
}

static void pure_queries(void) {
  const int32_t big[] = {1, 64, 4096, 14336, 1 << 20, 2147483647, -1, 0};
  for (unsigned i = 0; i < sizeof(big) / sizeof(big[0]); ++i)
    for (unsigned j = 0; j < sizeof(big) / sizeof(big[0]); ++j)
      for (int p = -1; p <= MQ_NPLANES; ++p) (void)mq_plane_bytes(big[i], big[j], p);
  EXPECT(mq_plane_bytes(14336, 4096, 0), 14336LL * 4096 / 4);
  EXPECT(mq_plane_bytes(14336, 4096, 1), 14336LL * 4096 / 8);
  EXPECT(mq_plane_bytes(1 << 20, 1 << 20, 0), (long long)((1ULL << 40) / 4));  /* at the size limit */
  EXPECT(mq_plane_bytes(2147483647, 2147483584, 0), 0);                        /* beyond it */
  for (int r = -1; r < 10; ++r)
    for (int rule = -1; rule < 4; ++rule) (void)mq_planes_needed(r, rule);
  EXPECT(mq_planes_needed(2, MQ_PREFIX), 1);
  EXPECT(mq_planes_needed(6, MQ_ROUND_EXTRA), 5);
  for (unsigned i = 0; i < sizeof(big) / sizeof(big[0]); ++i)
    for (unsigned j = 0; j < sizeof(big) / sizeof(big[0]); ++j)
      for (int m = -1; m < 300; m += 37) (void)mq_linear_workspace_bytes(m, big[i], big[j]);
}

static void linear_rejections(void) {
  mq_packed w = packed(64, 256);
  mq_packed bad_k = packed(64, 100);
  mq_packed huge = packed(2147483647, 2147483584);
  EXPECT(mq_linear(P(0x1000), MQ_F16, 1, &w, 5, MQ_PREFIX, 64, P(0x2000), P(0x3000), P(0x4000), NULL, 0, NULL),
         MQ_EWIDTH);
  EXPECT(mq_linear(P(0x1000), MQ_F16, 1, &w, 4, 7, 64, P(0x2000), P(0x3000), P(0x4000), NULL, 0, NULL), MQ_ERULE);
  EXPECT(mq_linear(P(0x1000), MQ_F16, 1, &w, 4, MQ_PREFIX, 96, P(0x2000), P(0x3000), P(0x4000), NULL, 0, NULL),
         MQ_ESHAPE);
  EXPECT(mq_linear(P(0x1000), MQ_F16, 1, &bad_k, 4, MQ_PREFIX, 64, P(0x2000), P(0x3000), P(0x4000), NULL, 0, NULL),
         MQ_ESHAPE);
  EXPECT(mq_linear(P(0x1000), MQ_F16, 1, NULL, 4, MQ_PREFIX, 64, P(0x2000), P(0x3000), P(0x4000), NULL, 0, NULL),
         MQ_EINVAL);
  EXPECT(mq_linear(P(0x1001), MQ_F16, 1, &w, 4, MQ_PREFIX, 64, P(0x2000), P(0x3000), P(0x4000), NULL, 0, NULL),
         MQ_EALIGN);
  EXPECT(mq_linear(P(0x1000), MQ_F32, 1, &w, 4, MQ_PREFIX, 64, P(0x2000), P(0x3000), P(0x4000), NULL, 0, NULL),
         MQ_EDTYPE);
  EXPECT(mq_linear(P(0x1000), MQ_F16, -1, &w, 4, MQ_PREFIX, 64, P(0x2000), P(0x3000), P(0x4000), NULL, 0, NULL),
         MQ_EINVAL);
  /* sizes at the int32 limits must be rejected without overflow */
  EXPECT(mq_linear(P(0x1000), MQ_F16, 2147483647, &huge, 4, MQ_PREFIX, 64, P(0x2000), P(0x3000), P(0x4000), NULL, 0,
                   NULL) != MQ_OK,
         1);
  mq_packed missing = packed(64, 256);
  missing.plane[1] = NULL;
  EXPECT(mq_linear(P(0x1000), MQ_F16, 1, &missing, 3, MQ_PREFIX, 64, P(0x2000), P(0x3000), P(0x4000), NULL, 0, NULL),
         MQ_ENOPLANE);
  EXPECT(mq_linear_noalloc(P(0x1000), MQ_F16, 1, &w, 5, MQ_PREFIX, 64, P(0x2000), P(0x3000), P(0x4000), NULL),
         MQ_EWIDTH);
  EXPECT(mq_linear_noalloc(P(0x1000), MQ_F16, 2048, &huge, 4, MQ_PREFIX, 64, P(0x2000), P(0x3000), P(0x4000), NULL) !=
             MQ_OK,
         1);
}

static void mixed_rejections(void) {
  mq_packed w = packed(64, 256);
  mq_call calls[3];
  for (int i = 0; i < 3; ++i) {
    calls[i].x = P(0x1000);
    calls[i].x_dtype = MQ_F16;
    calls[i].m = 1;
    calls[i].w = &w;
    calls[i].r = 4;
    calls[i].rule = MQ_PREFIX;
    calls[i].group = 64;
    calls[i].scales = P(0x2000);
    calls[i].zeros = P(0x3000);
    calls[i].y = P(0x4000 + 0x1000 * i);
  }
  calls[2].r = 9;
  int32_t failed = 123;
  EXPECT(mq_linear_mixed(calls, 3, NULL, 0, &failed, NULL), MQ_EWIDTH);
  EXPECT(failed, 2);
  EXPECT(mq_linear_mixed(NULL, 3, NULL, 0, &failed, NULL), MQ_EINVAL);
  EXPECT(mq_linear_mixed(calls, -1, NULL, 0, NULL, NULL), MQ_EINVAL);
}

static void other_rejections(void) {
  mq_packed w = packed(64, 256);
  EXPECT(mq_pack_parent(NULL, 64, 256, &w, NULL), MQ_EINVAL);
  EXPECT(mq_pack_parent(P(0x1000), 64, 100, &w, NULL), MQ_ESHAPE);
  EXPECT(mq_pack_parent(P(0x1000), 2147483647, 2147483584, &w, NULL) != MQ_OK, 1);
  EXPECT(mq_slice_codes(&w, 5, MQ_PREFIX, P(0x1000), NULL), MQ_EWIDTH);
  EXPECT(mq_slice_codes(&w, 4, MQ_PREFIX, P(0x1008), NULL), MQ_EALIGN);
  EXPECT(mq_dequant(&w, 4, MQ_PREFIX, 64, P(0x2000), P(0x3000), 9, P(0x1000), NULL), MQ_EDTYPE);
  EXPECT(mq_dequant(&w, 4, MQ_PREFIX, 48, P(0x2000), P(0x3000), MQ_F32, P(0x1000), NULL), MQ_ESHAPE);
}

static void produce_rejections(void) {
  int32_t widths[6] = {3, 4, 8, 2, 6, 8};
  float lams[6] = {1.0f, 1.0f, 1.0f, 1.0f, 1.0f, 1.0f};
  float bad_lams[3] = {1.0f, -1.0f, 1.0f};
  float nan_lams[3] = {1.0f, NAN, 1.0f};
  int32_t dup[3] = {3, 3, 8};
  int32_t odd[3] = {3, 5, 8};
#define PRODUCE(n, k, g, wd, lm, nw, rule, ng, gd, w_) \
  mq_produce_parent((const float*)P(w_), n, k, g, wd, lm, nw, rule, ng, gd, P(0x2000), P(0x3000), P(0x4000), NULL)
  EXPECT(PRODUCE(64, 256, 64, widths, lams, 6, MQ_PREFIX, 80, 100, 0x1000), MQ_EINVAL);
  EXPECT(PRODUCE(64, 256, 64, widths, lams, 0, MQ_PREFIX, 80, 100, 0x1000), MQ_EINVAL);
  EXPECT(PRODUCE(64, 256, 64, dup, lams, 3, MQ_PREFIX, 80, 100, 0x1000), MQ_EWIDTH);
  EXPECT(PRODUCE(64, 256, 64, odd, lams, 3, MQ_PREFIX, 80, 100, 0x1000), MQ_EWIDTH);
  EXPECT(PRODUCE(64, 256, 64, widths, bad_lams, 3, MQ_PREFIX, 80, 100, 0x1000), MQ_EINVAL);
  EXPECT(PRODUCE(64, 256, 64, widths, nan_lams, 3, MQ_PREFIX, 80, 100, 0x1000), MQ_EINVAL);
  EXPECT(PRODUCE(64, 256, 64, widths, lams, 3, MQ_PREFIX, 101, 100, 0x1000), MQ_EINVAL);
  EXPECT(PRODUCE(64, 256, 64, widths, lams, 3, 5, 80, 100, 0x1000), MQ_ERULE);
  EXPECT(PRODUCE(64, 4096, 2048, widths, lams, 3, MQ_PREFIX, 80, 100, 0x1000), MQ_ESHAPE);
  EXPECT(PRODUCE(2147483647, 2147483584, 64, widths, lams, 3, MQ_PREFIX, 80, 100, 0x1000), MQ_ESIZE);
  EXPECT(PRODUCE(64, 256, 64, widths, lams, 3, MQ_PREFIX, 80, 100, 0x1004), MQ_EALIGN);
  EXPECT(PRODUCE(64, 256, 64, NULL, lams, 3, MQ_PREFIX, 80, 100, 0x1000), MQ_EINVAL);
#undef PRODUCE
}

int main(void) {
  status_strings();
  pure_queries();
  linear_rejections();
  mixed_rejections();
  other_rejections();
  produce_rejections();
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("abi sanitizer driver: all checks passed\n");
  return 0;
}
