/*
 * Host-side validation of the C ABI, built and run under AddressSanitizer
 * (host code only; no GPU is touched: every call below is refused, or is a
 * pure host function, before any device work).  Exits non-zero on the first
 * unexpected status; ASan aborts on any invalid host memory access.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "woq.h"

static int failures = 0;

#define EXPECT(call, want)                                                        \
  do {                                                                            \
    const int32_t got_ = (call);                                                  \
    if (got_ != (want)) {                                                         \
      fprintf(stderr, "%s:%d: %s returned %d (%s), expected %d\n", __FILE__,      \
              __LINE__, #call, got_, woq_status_str(got_), (int)(want));          \
      ++failures;                                                                 \
    }                                                                             \
  } while (0)

int main(void) {
  void* a16 = (void*)(uintptr_t)(1u << 20);        /* never dereferenced */
  void* odd = (void*)(uintptr_t)((1u << 20) + 8);
  char buf[512];

  /* status strings and version: every code, and codes outside the list */
  for (int c = -3; c < 20; ++c) {
    const char* s = woq_status_str(c);
    if (!s || !s[0]) { fprintf(stderr, "empty status string for %d\n", c); ++failures; }
  }
  if (woq_version() <= 0) ++failures;

  /* plans: every size class, buffers from 1 byte up (truncated, NUL-terminated) */
  const int64_t ms[] = {0, 1, 2, 3, 4, 5, 16, 17, 24, 33, 64, 65, 100, 128, 129, 2048};
  const int64_t ns[] = {1, 64, 300, 1024, 14336};
  const int64_t ks[] = {0, 32, 256, 2080, 4096, 32768, 32800};
  const int32_t gs[] = {32, 64, 128, 256};
  for (size_t mi = 0; mi < sizeof ms / sizeof ms[0]; ++mi)
    for (size_t ni = 0; ni < sizeof ns / sizeof ns[0]; ++ni)
      for (size_t ki = 0; ki < sizeof ks / sizeof ks[0]; ++ki)
        for (size_t gi = 0; gi < sizeof gs / sizeof gs[0]; ++gi) {
          const int64_t m = ms[mi], n = ns[ni], k = ks[ki];
          const int32_t g = gs[gi];
          if (k % g) continue;
          for (int o = 0; o < 2; ++o) {
            for (size_t len = 1; len <= sizeof buf; len = len * 3 + 1) {
              memset(buf, 'x', sizeof buf);
              EXPECT(woq_linear_plan(m, n, k, g, o, buf, len), WOQ_OK);
              if (strlen(buf) >= len) { fprintf(stderr, "plan not terminated\n"); ++failures; }
            }
            (void)woq_linear_workspace_bytes(m, n, k, g, o);
            (void)woq_linear_int4_groups_zp4_workspace_bytes(m, n, k, g, o);
            (void)woq_linear_int4_rows_workspace_bytes(m, n, k, o);
          }
        }
  EXPECT(woq_linear_plan(1, 64, 256, 32, 0, NULL, 16), WOQ_EINVAL);
  EXPECT(woq_linear_plan(1, 64, 256, 32, 0, buf, 0), WOQ_EINVAL);
  EXPECT(woq_linear_plan(1, 64, 256, 48, 0, buf, sizeof buf), WOQ_EGROUP);
  if (woq_prepared_bytes(-1, 64) != 0 || woq_prepared_bytes(3, 48) != 0) ++failures;
  if (woq_linear_noalloc_max_workspace_bytes() == 0) ++failures;

  /* the linear layer: shapes, pointers, dtype, alignment, workspace */
  EXPECT(woq_linear_int4_groups(NULL, -1, NULL, NULL, NULL, NULL, NULL, 64, 256, 32, 1, NULL, NULL, 0, NULL),
         WOQ_EINVAL);
  EXPECT(woq_linear_int4_groups(NULL, 1, NULL, NULL, NULL, NULL, NULL, 64, 256, 48, 1, NULL, NULL, 0, NULL),
         WOQ_EGROUP);
  EXPECT(woq_linear_int4_groups(NULL, 1, NULL, NULL, NULL, NULL, NULL, 64, 240, 48, 1, NULL, NULL, 0, NULL),
         WOQ_EUNSUPPORTED);
  EXPECT(woq_linear_int4_groups(NULL, 1, a16, a16, a16, NULL, NULL, 64, 256, 32, 1, a16, NULL, 0, NULL),
         WOQ_EINVAL);
  EXPECT(woq_linear_int4_groups(a16, 1, a16, a16, a16, NULL, NULL, 64, 256, 32, 7, a16, NULL, 0, NULL),
         WOQ_EINVAL);
  EXPECT(woq_linear_int4_groups(odd, 1, a16, a16, a16, NULL, NULL, 64, 256, 32, 1, a16, NULL, 0, NULL),
         WOQ_EALIGN);
  EXPECT(woq_linear_int4_groups(a16, 1, a16, a16, a16, NULL, (const int32_t*)a16, 64, 256, 32, 1, a16, NULL, 0,
                                NULL),
         WOQ_EWORKSPACE);
  EXPECT(woq_linear_int4_groups(a16, 200, a16, a16, a16, NULL, NULL, 64, 256, 32, 1, a16, a16, 16, NULL),
         WOQ_EWORKSPACE);
  EXPECT(woq_linear_int4_groups(a16, 48, a16, a16, a16, NULL, NULL, 64, 4096, 32, 1, a16, a16, 16, NULL),
         WOQ_EWORKSPACE);   /* the small-M path's K-range partials need their buffer */
  EXPECT(woq_linear_int4_groups(a16, 48, a16, a16, a16, NULL, NULL, 14336, 256, 32, 1, a16, a16, 16, NULL),
         WOQ_EWORKSPACE);   /* the small-M fragment pre-pass needs its buffer */
  EXPECT(woq_linear_int4_groups(NULL, 0, NULL, NULL, NULL, NULL, NULL, 64, 256, 32, 1, NULL, NULL, 0, NULL),
         WOQ_OK);
  EXPECT(woq_linear_int4_groups_noalloc(a16, 2048, a16, a16, a16, NULL, NULL, 4096, 14336, 128, 1, a16, NULL),
         WOQ_EWORKSPACE);
  EXPECT(woq_linear_int4_groups_zp4(a16, 200, a16, a16, NULL, NULL, NULL, 64, 256, 128, 1, a16, a16, 1 << 20,
                                    NULL),
         WOQ_EINVAL);
  EXPECT(woq_linear_int4_groups_zp4(a16, 200, a16, a16, a16, NULL, NULL, 64, 256, 128, 1, a16, a16, 16, NULL),
         WOQ_EWORKSPACE);

  /* grouped calls: count, tables, per-matrix checks */
  {
    const uint8_t* pk[3] = {a16, a16, a16};
    const float* sc[3] = {a16, a16, a16};
    const uint8_t* zr[3] = {a16, a16, (const uint8_t*)odd};
    void* ys[3] = {a16, a16, a16};
    int64_t nn[3] = {64, 32, 16};
    EXPECT(woq_linear_int4_groups_grouped(a16, 1, 0, pk, sc, zr, NULL, nn, 256, 32, 0, 1, ys, NULL, 0, NULL),
           WOQ_EINVAL);
    EXPECT(woq_linear_int4_groups_grouped(a16, 1, 5, pk, sc, zr, NULL, nn, 256, 32, 0, 1, ys, NULL, 0, NULL),
           WOQ_EINVAL);
    EXPECT(woq_linear_int4_groups_grouped(a16, 1, 3, NULL, sc, zr, NULL, nn, 256, 32, 0, 1, ys, NULL, 0, NULL),
           WOQ_EINVAL);
    EXPECT(woq_linear_int4_groups_grouped(a16, 1, 3, pk, sc, zr, NULL, nn, 256, 32, 0, 1, ys, NULL, 0, NULL),
           WOQ_EALIGN);
    nn[1] = -1;
    EXPECT(woq_linear_int4_groups_grouped(a16, 1, 2, pk, sc, zr, NULL, nn, 256, 32, 0, 1, ys, NULL, 0, NULL),
           WOQ_EINVAL);
  }

  /* codecs */
  EXPECT(woq_pack_uint4(a16, 3, a16, NULL), WOQ_ESHAPE);
  EXPECT(woq_unpack_uint4(a16, -2, a16, NULL), WOQ_EINVAL);
  EXPECT(woq_quantize_groups(a16, 2, 10, 4, 0, a16, a16, a16, NULL), WOQ_EGROUP);
  EXPECT(woq_quantize_groups(a16, 2, 8, 4, 2, a16, a16, a16, NULL), WOQ_EINVAL);
  EXPECT(woq_quantize_groups(NULL, 2, 8, 4, 0, a16, a16, a16, NULL), WOQ_EINVAL);
  EXPECT(woq_dequantize_int4_groups(a16, a16, a16, 2, 12, 3, 0, a16, NULL), WOQ_EGROUP);
  EXPECT(woq_dequantize_int4_groups(a16, a16, NULL, 2, 12, 4, 0, a16, NULL), WOQ_EINVAL);
  EXPECT(woq_pack_zero_points(NULL, 4, 8, a16, NULL), WOQ_EINVAL);
  EXPECT(woq_unpack_zero_points(a16, 4, 8, NULL, NULL), WOQ_EINVAL);
  EXPECT(woq_prepare_int4(a16, 64, 48, a16, NULL), WOQ_ESHAPE);

  /* quantizers */
  EXPECT(woq_gptq_quantize(a16, a16, 16, 64, 256, 32, 2, 0.01, a16, a16, a16, NULL, NULL), WOQ_EINVAL);
  EXPECT(woq_gptq_quantize(a16, a16, 16, 64, 256, 32, 0, -1.0, a16, a16, a16, NULL, NULL), WOQ_EINVAL);
  EXPECT(woq_gptq_quantize(a16, a16, 16, 64, 250, 32, 0, 0.01, a16, a16, a16, NULL, NULL), WOQ_EGROUP);
  EXPECT(woq_gptq_quantize(a16, a16, 16, 64, 256, 32, 1, 0.01, a16, a16, a16, NULL, NULL), WOQ_EINVAL);
  EXPECT(woq_awq_search(a16, a16, 0, 64, 256, 32, 20, a16, a16, a16, a16, NULL, NULL, NULL), WOQ_EINVAL);
  EXPECT(woq_awq_search(a16, a16, 8, 64, 256, 32, 1001, a16, a16, a16, a16, NULL, NULL, NULL), WOQ_EINVAL);
  EXPECT(woq_awq_search((const float*)(uintptr_t)((1u << 20) + 2), a16, 8, 64, 256, 32, 20, a16, a16, a16, a16,
                        NULL, NULL, NULL),
         WOQ_EALIGN);

  if (failures) {
    fprintf(stderr, "%d unexpected statuses\n", failures);
    return 1;
  }
  printf("abi validation: all checks passed\n");
  return 0;
}
