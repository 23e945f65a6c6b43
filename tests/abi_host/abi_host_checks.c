/* Host argument checks of every fq.h entry point, with no GPU: each call must
 * answer with the documented status and touch nothing it was not given.  Built
 * with AddressSanitizer and UndefinedBehaviorSanitizer on the host code of the
 * boundary (see test_abi_sanitize.py); any sanitizer report fails the run. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fq.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      failures++;                                                      \
    }                                                                  \
  } while (0)

int main(void) {
  /* status strings: every value, including ones outside the enum */
  for (int st = -3; st < 10; st++) EXPECT(fq_status_string((fq_status)st) != NULL);
  EXPECT(strcmp(fq_status_string(FQ_OK), "ok") == 0);

  /* calls on a NULL handle answer on the host */
  char* p = (char*)aligned_alloc(16, 1 << 16);
  memset(p, 0, 1 << 16);
  void* v = p;
  EXPECT(fq_code_bytes(NULL, 10) == -1);
  EXPECT(fq_encode_kernel(NULL, FQ_F16, 10) == NULL);
  EXPECT(fq_encode(NULL, v, FQ_F16, 1, (uint8_t*)v, v, FQ_F16, NULL) == FQ_ERR_ARG);
  EXPECT(fq_encode_scatter(NULL, v, FQ_F16, 1, (const int64_t*)v, 4, (uint8_t*)v, v, FQ_F16, NULL) == FQ_ERR_ARG);
  EXPECT(fq_decode(NULL, (const uint8_t*)v, v, FQ_F16, 1, v, FQ_F16, NULL) == FQ_ERR_ARG);
  EXPECT(fq_attn_workspace_bytes(NULL, 1, 8, 1, 10) == 0);
  EXPECT(fq_attn_decode(NULL, v, (const uint8_t*)v, v, (const uint8_t*)v, v, 1, 8, 1, 10, 0.125f, (float*)v, v,
                        1 << 16, NULL) == FQ_ERR_ARG);
  EXPECT(fq_attn_decode_varlen(NULL, v, (const uint8_t*)v, v, (const uint8_t*)v, v, (const int32_t*)v, 1, 8, 1, 10,
                               0.125f, (float*)v, v, 1 << 16, NULL) == FQ_ERR_ARG);
  EXPECT(fq_attn_decode_noalloc(NULL, v, (const uint8_t*)v, v, (const uint8_t*)v, v, NULL, 1, 8, 1, 10, 0.125f,
                                (float*)v, NULL) == FQ_ERR_ARG);
  EXPECT(fq_attn_noalloc_max_workspace_bytes() == ((size_t)16 << 20));
  EXPECT(fq_attn_prefill_workspace_bytes(NULL, 1, 8, 1, 4, 10) == 0);
  EXPECT(fq_attn_prefill(NULL, v, (const uint8_t*)v, v, (const uint8_t*)v, v, 1, 8, 1, 4, 10, 1, 0.125f, (float*)v,
                         v, 1 << 16, NULL) == FQ_ERR_ARG);
  fq_codebook_free(NULL);

  /* training: sizes, including ones whose products overflow 32 bits */
  EXPECT(fq_codebook_train_workspace_bytes(3, 16, 100, 100) == 0);
  EXPECT(fq_codebook_train_workspace_bytes(4, 16, 100, 100) > 0);
  EXPECT(fq_codebook_train_workspace_bytes(64, 65536, 2147483647LL, 2147483647LL) > 0);
  EXPECT(fq_codebook_train_workspace_bytes(64, 65537, 100, 100) == 0);
  EXPECT(fq_codebook_train_workspace_bytes(4, 16, 2147483648LL, 100) == 0);
  EXPECT(fq_codebook_train_workspace_bytes(4, 16, 0, 100) == 0);
  double mse[4], vmse, hist[11];
  int hlen;
  const double* dv = (const double*)v;
  EXPECT(fq_codebook_train(4, 16, NULL, 100, dv, 100, dv, 1, 10, 1e-6, (float*)v, NULL, mse, &vmse, hist, &hlen, v,
                           1 << 16, NULL) == FQ_ERR_ARG);
  EXPECT(fq_codebook_train(4, 16, dv, 100, dv, 100, dv, 1, 10, -1.0, (float*)v, NULL, mse, &vmse, hist, &hlen, v,
                           1 << 16, NULL) == FQ_ERR_ARG);
  EXPECT(fq_codebook_train(4, 16, dv, 100, dv, 100, dv, 1, 10, NAN, (float*)v, NULL, mse, &vmse, hist, &hlen, v,
                           1 << 16, NULL) == FQ_ERR_ARG);
  EXPECT(fq_codebook_train(4, 16, dv, 100, dv, 100, dv, 0, 10, 1e-6, (float*)v, NULL, mse, &vmse, hist, &hlen, v,
                           1 << 16, NULL) == FQ_ERR_ARG);
  EXPECT(fq_codebook_train(4, 16, dv, 100, dv, 100, dv, 1, 10, 1e-6, (float*)v, NULL, mse, &vmse, hist, &hlen, v,
                           16, NULL) == FQ_ERR_WORKSPACE);
  EXPECT(fq_codebook_train(4, 16, (const double*)(p + 4), 100, dv, 100, dv, 1, 10, 1e-6, (float*)v, NULL, mse, &vmse,
                           hist, &hlen, v, 1 << 16, NULL) == FQ_ERR_ARG); /* misaligned */

  /* codebook load: every rejection happens before the first HIP call */
  enum { N = 16, K = 2, D = 64 };
  float* cw = (float*)malloc(sizeof(float) * N * K);
  float* rot = (float*)malloc(sizeof(float) * D * D);
  for (int i = 0; i < N * K; i++) cw[i] = 0.25f * (float)((i % 7) - 3);
  for (int i = 0; i < D * D; i++) rot[i] = (i % (D + 1)) == 0 ? 1.0f : 0.0f;
  fq_codebook* h = (fq_codebook*)0x1;
  EXPECT(fq_codebook_load(D, K, N, cw, rot, NULL) == FQ_ERR_ARG);
  EXPECT(fq_codebook_load(D, K, N, NULL, rot, &h) == FQ_ERR_ARG && h == (fq_codebook*)0x1);
  EXPECT(fq_codebook_load(D, K, N, cw, rot, &h) != FQ_OK || h != NULL); /* no GPU here: FQ_ERR_HIP, nothing leaked */
  EXPECT(fq_codebook_load(63, K, N, cw, rot, &h) == FQ_ERR_UNSUPPORTED && h == NULL);
  EXPECT(fq_codebook_load(D, 3, N, cw, rot, &h) == FQ_ERR_ARG);
  EXPECT(fq_codebook_load(D, 0, N, cw, rot, &h) == FQ_ERR_ARG);
  EXPECT(fq_codebook_load(D, K, 12, cw, rot, &h) == FQ_ERR_ARG);
  EXPECT(fq_codebook_load(D, K, 1, cw, rot, &h) == FQ_ERR_ARG);
  EXPECT(fq_codebook_load(D, K, 131072, cw, rot, &h) == FQ_ERR_ARG);
  EXPECT(fq_codebook_load(D, K, -16, cw, rot, &h) == FQ_ERR_ARG);
  cw[5] = 0.1f; /* not an fp16 value */
  EXPECT(fq_codebook_load(D, K, N, cw, rot, &h) == FQ_ERR_ARG);
  cw[5] = 1.0f / 1048576.0f; /* an fp16 subnormal */
  EXPECT(fq_codebook_load(D, K, N, cw, rot, &h) == FQ_ERR_ARG);
  cw[5] = INFINITY;
  EXPECT(fq_codebook_load(D, K, N, cw, rot, &h) == FQ_ERR_ARG);
  cw[5] = 0.5f;
  rot[70] = NAN;
  EXPECT(fq_codebook_load(D, K, N, cw, rot, &h) == FQ_ERR_ARG);
  EXPECT(h == NULL);
  free(cw);
  free(rot);
  free(p);
  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("abi host checks: ok\n");
  return 0;
}
