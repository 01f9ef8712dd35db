/*
 * Host-side check of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer
 * (built by tests/test_host_sanitizers.py with every library source, host code
 * instrumented).  Every call below carries at least one invalid argument, so each
 * must be rejected before anything is enqueued: nothing here touches a GPU, and the
 * fake device pointers are never dereferenced.  The workspace-size queries also run
 * with extreme sizes, where an overflow in the size arithmetic would be undefined
 * behaviour.  Exit status 0 with "ok" printed when every call was rejected.
 */
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include "swattn.h"

static int failures = 0;
static int calls = 0;

#define REJECT(expr)                                                              \
  do {                                                                            \
    int rc_ = (expr);                                                             \
    ++calls;                                                                      \
    if (rc_ == 0) {                                                               \
      fprintf(stderr, "accepted (should be rejected): %s\n", #expr);              \
      ++failures;                                                                 \
    }                                                                             \
  } while (0)

#define EXPECT(cond)                                                              \
  do {                                                                            \
    ++calls;                                                                      \
    if (!(cond)) {                                                                \
      fprintf(stderr, "failed: %s\n", #cond);                                     \
      ++failures;                                                                 \
    }                                                                             \
  } while (0)

int main(void) {
  void *F = (void *)(uintptr_t)0x100000;       /* aligned, never dereferenced */
  void *M = (void *)(uintptr_t)0x100002;       /* misaligned */
  float *Ff = (float *)F;
  const int *Fi = (const int *)F;
  const float nan_ = NAN, inf_ = INFINITY;
  const int big = INT_MAX;

  /* status strings and version */
  for (int s = -3; s < 8; ++s) EXPECT(swattn_status_string(s) != NULL);
  EXPECT(swattn_status_string(99) != NULL);
  EXPECT(swattn_version() >= 100);

  /* workspace sizes: valid, invalid and extreme arguments */
  EXPECT(swattn_bwd_workspace_size(8, 6, 2048, 128) == (size_t)8 * 6 * 2048 * 4);
  EXPECT(swattn_bwd_workspace_size(0, 6, 2048, 128) == 0);
  EXPECT(swattn_bwd_workspace_size(8, 6, 2048, 96) == 0);
  (void)swattn_bwd_workspace_size(big, big, big, 128);
  (void)swattn_bwd_workspace_size(-1, big, -big, 64);
  (void)swattn_bwd_gqa_workspace_size(big, big, 1, big, 128);
  (void)swattn_bwd_gqa_workspace_size(big, big, big, big, 128);
  EXPECT(swattn_bwd_gqa_workspace_size(2, 6, 4, 64, 128) == 0); /* 4 does not divide 6 */
  EXPECT(swattn_decode_workspace_size(32, 12, 128, 4096, -1) > 0);
  EXPECT(swattn_decode_workspace_size(32, 12, 128, 4096, 0) == 0);
  (void)swattn_decode_workspace_size(big, big, 128, big, -1);
  (void)swattn_decode_workspace_size(big, big, 128, big, big);
  (void)swattn_decode_workspace_size(-big, 1, 64, 1, 1);

  /* forward */
  REJECT(swattn_fwd(NULL, F, F, F, Ff, 1, 1, 8, 64, -1, 1.f, NULL));
  REJECT(swattn_fwd(F, F, F, F, NULL, 1, 1, 8, 64, -1, 1.f, NULL));
  REJECT(swattn_fwd(M, F, F, F, Ff, 1, 1, 8, 64, -1, 1.f, NULL));
  REJECT(swattn_fwd(F, F, F, F, Ff, 0, 1, 8, 64, -1, 1.f, NULL));
  REJECT(swattn_fwd(F, F, F, F, Ff, 1, -1, 8, 64, -1, 1.f, NULL));
  REJECT(swattn_fwd(F, F, F, F, Ff, 1, 1, 0, 64, -1, 1.f, NULL));
  REJECT(swattn_fwd(F, F, F, F, Ff, 1, 1, 8, 96, -1, 1.f, NULL));
  REJECT(swattn_fwd(F, F, F, F, Ff, 1, 1, 8, 64, 0, 1.f, NULL));
  REJECT(swattn_fwd(F, F, F, F, Ff, 1, 1, 8, 64, -1, 0.f, NULL));
  REJECT(swattn_fwd(F, F, F, F, Ff, 1, 1, 8, 64, -1, -1.f, NULL));
  REJECT(swattn_fwd(F, F, F, F, Ff, 1, 1, 8, 64, -1, nan_, NULL));
  REJECT(swattn_fwd(F, F, F, F, Ff, 1, 1, 8, 64, -1, inf_, NULL));
  EXPECT(swattn_fwd(F, F, F, F, Ff, big, big, big, 128, -1, 1.f, NULL) == SWATTN_ERR_INVALID_ARG);
  EXPECT(swattn_fwd(F, F, F, F, Ff, 1, 1 << 16, 1 << 16, 128, -1, 1.f, NULL) ==
         SWATTN_ERR_INVALID_ARG);
  /* one sequence's [T + 128, H, D] block past 2^31 bytes */
  EXPECT(swattn_fwd(F, F, F, F, Ff, 1, 64, 1 << 17, 128, -1, 1.f, NULL) ==
         SWATTN_ERR_UNSUPPORTED);
  REJECT(swattn_fwd_f32(NULL, Ff, Ff, Ff, Ff, 1, 1, 8, 64, -1, 1.f, NULL));
  REJECT(swattn_fwd_f32(Ff, Ff, Ff, Ff, Ff, 1, 1, 8, 64, 0, 1.f, NULL));
  REJECT(swattn_fwd_f32(Ff, Ff, Ff, Ff, Ff, 1, 1, 8, 64, -1, nan_, NULL));
  REJECT(swattn_fwd_gqa(F, F, F, F, Ff, 1, 6, 4, 8, 64, -1, 1.f, NULL));
  REJECT(swattn_fwd_gqa(F, F, F, F, Ff, 1, 6, 0, 8, 64, -1, 1.f, NULL));
  REJECT(swattn_fwd_gqa(F, F, F, F, Ff, 1, 6, -2, 8, 64, -1, 1.f, NULL));
  REJECT(swattn_fwd_gqa(F, F, F, F, Ff, big, big, 1, big, 128, -1, 1.f, NULL));

  /* backward and its stages */
  REJECT(swattn_bwd(F, F, F, F, F, Ff, F, F, F, 1, 1, 8, 64, -1, 1.f, NULL, NULL));
  REJECT(swattn_bwd(F, F, F, F, NULL, Ff, F, F, F, 1, 1, 8, 64, -1, 1.f, F, NULL));
  REJECT(swattn_bwd(F, F, F, F, F, Ff, F, F, F, 1, 1, 8, 64, 0, 1.f, F, NULL));
  REJECT(swattn_bwd(F, F, F, F, F, Ff, F, F, F, 1, 1, 8, 64, -1, -2.f, F, NULL));
  REJECT(swattn_bwd(F, F, F, F, F, Ff, F, F, F, big, big, big, 128, -1, 1.f, F, NULL));
  REJECT(swattn_bwd_f32(Ff, Ff, Ff, Ff, Ff, Ff, Ff, Ff, Ff, 1, 1, 8, 64, -1, 1.f, NULL, NULL));
  REJECT(swattn_bwd_f32(Ff, Ff, Ff, Ff, Ff, Ff, Ff, Ff, Ff, 1, 1, 8, 96, -1, 1.f, F, NULL));
  REJECT(swattn_bwd_gqa(F, F, F, F, F, Ff, F, F, F, 1, 6, 4, 8, 64, -1, 1.f, F, NULL));
  REJECT(swattn_bwd_gqa(F, F, F, F, F, Ff, F, F, F, 1, 6, 2, 8, 64, -1, 1.f, NULL, NULL));
  REJECT(swattn_bwd_gqa(F, F, F, F, F, Ff, F, F, F, 1, 6, 2, 8, 64, -1, nan_, F, NULL));
  REJECT(swattn_bwd_preprocess(NULL, F, F, 1, 1, 8, 64, NULL));
  REJECT(swattn_bwd_preprocess(F, F, F, 1, 1, 8, 96, NULL));
  REJECT(swattn_bwd_preprocess(F, F, F, big, big, big, 128, NULL));
  REJECT(swattn_bwd_preprocess_f32(Ff, Ff, NULL, 1, 1, 8, 64, NULL));
  REJECT(swattn_bwd_dkdv(F, F, F, F, Ff, F, F, F, 1, 1, 8, 64, 0, 1.f, NULL));
  REJECT(swattn_bwd_dkdv(F, F, F, F, Ff, NULL, F, F, 1, 1, 8, 64, -1, 1.f, NULL));
  REJECT(swattn_bwd_dkdv(F, F, F, F, Ff, F, F, F, 1, 1, 8, 64, -1, 0.f, NULL));
  REJECT(swattn_bwd_dkdv_f32(Ff, Ff, Ff, Ff, Ff, F, Ff, Ff, 1, 1, 8, 64, -1, inf_, NULL));
  REJECT(swattn_bwd_dq(F, F, F, F, F, Ff, F, F, 1, 1, 8, 64, -1, nan_, NULL));
  REJECT(swattn_bwd_dq(F, F, F, F, F, Ff, NULL, F, 1, 1, 8, 64, -1, 1.f, NULL));
  REJECT(swattn_bwd_dq_f32(Ff, Ff, Ff, Ff, Ff, Ff, F, Ff, 1, 1, 8, 64, 0, 1.f, NULL));

  /* prefill */
  REJECT(swattn_prefill(F, F, F, F, F, Fi, F, Ff, 1, 1, 1, 16, 64, 8, -1, 1.f, NULL));  /* Tq > Tmax */
  REJECT(swattn_prefill(F, F, F, F, F, Fi, F, Ff, 1, 1, 1, 0, 64, 8, -1, 1.f, NULL));
  REJECT(swattn_prefill(F, F, F, F, F, NULL, F, Ff, 1, 1, 1, 4, 64, 8, -1, 1.f, NULL));
  REJECT(swattn_prefill(F, F, F, F, F, Fi, F, Ff, 1, 6, 4, 4, 64, 8, -1, 1.f, NULL));
  REJECT(swattn_prefill(F, F, F, F, F, Fi, F, Ff, 1, 1, 1, 4, 64, 8, 0, 1.f, NULL));
  REJECT(swattn_prefill(F, F, F, F, F, Fi, F, Ff, 1, 1, 1, 4, 64, 8, -1, -1.f, NULL));
  REJECT(swattn_prefill(F, F, F, F, F, Fi, F, Ff, big, big, 1, 4, 128, big, -1, 1.f, NULL));

  /* decode */
  REJECT(swattn_decode(F, F, F, Fi, F, Ff, 1, 1, 64, 8, -1, 1.f, NULL, NULL));
  REJECT(swattn_decode(F, F, F, NULL, F, Ff, 1, 1, 64, 8, -1, 1.f, F, NULL));
  REJECT(swattn_decode(F, F, F, Fi, F, Ff, 1, 1, 64, 0, -1, 1.f, F, NULL));
  REJECT(swattn_decode(F, F, F, Fi, F, Ff, 1, 1, 64, 8, 0, 1.f, F, NULL));
  REJECT(swattn_decode(F, F, F, Fi, F, Ff, 1, 1, 96, 8, -1, 1.f, F, NULL));
  REJECT(swattn_decode(F, F, F, Fi, F, Ff, 70000, 1, 64, 8, -1, 1.f, F, NULL));
  REJECT(swattn_decode(F, F, F, Fi, F, Ff, big, big, 128, big, -1, 1.f, F, NULL));
  REJECT(swattn_decode(F, F, F, Fi, F, Ff, 1, 1, 64, 8, -1, nan_, F, NULL));
  REJECT(swattn_decode_f32(Ff, Ff, Ff, Fi, Ff, Ff, 1, 1, 64, 8, -1, 0.f, F, NULL));
  REJECT(swattn_decode_gqa(F, F, F, Fi, F, Ff, 1, 6, 4, 64, 8, -1, 1.f, F, NULL));
  REJECT(swattn_decode_gqa(F, F, F, Fi, F, Ff, 1, 6, 0, 64, 8, -1, 1.f, F, NULL));
  REJECT(swattn_decode_noalloc(F, F, F, Fi, F, Ff, 1, 1, 64, 8, 0, 1.f, NULL));
  REJECT(swattn_decode_noalloc(NULL, F, F, Fi, F, Ff, 1, 1, 64, 8, -1, 1.f, NULL));
  /* more partials than the scratch array holds */
  EXPECT(swattn_decode_noalloc(F, F, F, Fi, F, Ff, 64, 64, 128, 8192, -1, 1.f, NULL) ==
         SWATTN_ERR_TOO_LARGE);

  /* QK-norm + rotary prologue, and the fused entry points */
  REJECT(swattn_qk_norm_rope(F, F, F, F, Fi, 1, 8, 2, 2, 64, 0.f, 1e-6f, NULL));
  REJECT(swattn_qk_norm_rope(F, F, F, F, Fi, 1, 8, 2, 2, 64, 1e4f, -1.f, NULL));
  REJECT(swattn_qk_norm_rope(F, F, F, F, Fi, 1, 8, 2, 2, 64, nan_, 1e-6f, NULL));
  REJECT(swattn_qk_norm_rope(F, F, F, F, Fi, 1, 8, 0, 0, 64, 1e4f, 1e-6f, NULL));
  REJECT(swattn_qk_norm_rope(F, F, F, F, Fi, big, big, big, 1, 128, 1e4f, 1e-6f, NULL));
  /* one token row, but q and k vectors per row past what the kernel counts */
  EXPECT(swattn_qk_norm_rope(F, F, F, F, Fi, 1, 1, big, 1, 64, 1e4f, 1e-6f, NULL) ==
         SWATTN_ERR_INVALID_ARG);
  EXPECT(swattn_qk_norm_rope_bwd(F, F, F, F, F, F, Fi, 1, 1, 1 << 30, 1 << 30, 64, 1e4f, 1e-6f,
                                 NULL) == SWATTN_ERR_INVALID_ARG);
  REJECT(swattn_qk_norm_rope_bwd(F, F, F, F, F, F, Fi, 1, 8, 2, 2, 96, 1e4f, 1e-6f, NULL));
  REJECT(swattn_qk_norm_rope_bwd(F, F, NULL, F, F, F, Fi, 1, 8, 2, 2, 64, 1e4f, 1e-6f, NULL));
  REJECT(swattn_fwd_rope(F, F, F, F, Ff, F, Fi, 1, 2, 8, 64, -1, 1.f, 0.f, 1e-6f, NULL));
  REJECT(swattn_fwd_rope(F, F, F, F, Ff, F, Fi, 1, 2, 8, 64, 0, 1.f, 1e4f, 1e-6f, NULL));
  REJECT(swattn_fwd_rope(F, F, F, F, Ff, F, Fi, 1, 2, 8, 64, -1, nan_, 1e4f, 1e-6f, NULL));
  REJECT(swattn_bwd_rope(F, F, F, F, F, F, F, Ff, F, F, F, Fi, 1, 2, 8, 64, -1, 1.f, 1e4f,
                         inf_, F, NULL));
  REJECT(swattn_bwd_rope(F, F, F, F, F, F, F, Ff, F, F, F, Fi, 1, 2, 8, 64, -1, 1.f, 1e4f,
                         1e-6f, NULL, NULL));
  REJECT(swattn_fwd_rope_gqa(F, F, F, F, Ff, F, Fi, 1, 6, 4, 8, 64, -1, 1.f, 1e4f, 1e-6f, NULL));
  REJECT(swattn_fwd_rope_gqa(F, F, F, F, Ff, F, Fi, 1, 6, 0, 8, 64, -1, 1.f, 1e4f, 1e-6f, NULL));
  REJECT(swattn_fwd_rope_gqa(F, F, F, F, Ff, F, Fi, 1, 6, 3, 8, 64, -1, 1.f, -1.f, 1e-6f, NULL));
  REJECT(swattn_fwd_rope_gqa(F, F, F, F, Ff, F, Fi, big, big, big, big, 128, -1, 1.f, 1e4f,
                             1e-6f, NULL));
  REJECT(swattn_bwd_rope_gqa(F, F, F, F, F, F, F, Ff, F, F, F, Fi, 1, 6, 5, 8, 64, -1, 1.f,
                             1e4f, 1e-6f, F, NULL));
  REJECT(swattn_bwd_rope_gqa(F, F, F, F, F, F, F, Ff, F, F, F, Fi, 1, 6, 3, 8, 64, -1, 1.f,
                             1e4f, nan_, F, NULL));
  REJECT(swattn_bwd_rope_gqa(F, F, F, F, F, F, F, Ff, F, F, F, Fi, 1, 6, 3, 8, 64, -1, 1.f,
                             1e4f, 1e-6f, NULL, NULL));

  /* measurement probes */
  REJECT(swattn_probe_mfma(NULL, 1, 1, NULL));
  REJECT(swattn_probe_mfma(Ff, 0, 1, NULL));
  REJECT(swattn_probe_mfma(Ff, 1, 0, NULL));
  REJECT(swattn_probe_mfma(Ff, big, 1, NULL));
  REJECT(swattn_probe_read(F, 0, (unsigned int *)F, 1, NULL));
  REJECT(swattn_probe_read(M, 16, (unsigned int *)F, 1, NULL));
  REJECT(swattn_probe_read(F, 24, (unsigned int *)F, 1, NULL));
  REJECT(swattn_probe_read(F, 16, (unsigned int *)F, -1, NULL));

  if (failures) {
    fprintf(stderr, "%d of %d checks failed\n", failures, calls);
    return 1;
  }
  printf("ok %d checks\n", calls);
  return 0;
}
