/* Drives the argument validation of every libfp8g entry point from plain C, for a build whose host
 * code carries AddressSanitizer and UndefinedBehaviorSanitizer (device code is not instrumented).
 * Every call here is rejected by validation or is an empty problem, so no GPU is touched; a
 * sanitizer report (overflow in a size product, an out-of-bounds or use-after-free in the error
 * path, ...) aborts the program. Prints "ok" and the number of calls made. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fp8g.h"

static int calls = 0;

#define EXPECT(expr, want)                                                                  \
  do {                                                                                      \
    fp8g_status_t st_ = (expr);                                                             \
    ++calls;                                                                                \
    if (st_ != (want)) {                                                                    \
      fprintf(stderr, "line %d: status %d, expected %d (%s)\n", __LINE__, (int)st_, (int)(want), \
              fp8g_last_error());                                                           \
      return 1;                                                                             \
    }                                                                                       \
    (void)strlen(fp8g_last_error());                                                        \
  } while (0)

int main(void) {
  static char buf[256] __attribute__((aligned(256)));
  void* p = buf;                  /* aligned dummy, never dereferenced */
  void* odd = buf + 1;            /* misaligned */
  const float* f = (const float*)buf;
  const int32_t* ip = (const int32_t*)buf;
  const int64_t huge = (int64_t)1 << 40, neg = -5;
  const int INV = FP8G_INVALID_ARGUMENT, NS = FP8G_NOT_SUPPORTED, OK = FP8G_OK;

  if (fp8g_version() < 100) return 2;
  /* plain form */
  EXPECT(fp8_gemm_nt_groupwise(p, p, f, f, p, 0, 4, 128, 100, 0, 1, 128, 128, NULL), INV);
  EXPECT(fp8_gemm_nt_groupwise(p, p, f, f, p, 0, neg, 128, 128, 0, 1, 128, 128, NULL), INV);
  EXPECT(fp8_gemm_nt_groupwise(p, p, f, f, p, 0, huge, huge, huge, 0, 1, 128, 128, NULL), INV);
  EXPECT(fp8_gemm_nt_groupwise(p, p, f, f, p, 0, INT64_MAX, 128, 128, 0, 1, 128, 128, NULL), INV);
  EXPECT(fp8_gemm_nt_groupwise(p, p, f, f, p, 0, 4, INT64_MAX, INT64_MAX / 2 + 1, 0, 1, 128, 128, NULL), INV);
  EXPECT(fp8_gemm_nt_groupwise(p, p, f, f, p, 0, 4, 128, 128, 0, 1, 64, 128, NULL), NS);
  EXPECT(fp8_gemm_nt_groupwise(p, p, f, f, p, 7, 4, 128, 128, 0, 1, 128, 128, NULL), INV);
  EXPECT(fp8_gemm_nt_groupwise(p, p, f, f, p, 0, 4, 128, 128, 3, 1, 128, 128, NULL), INV);
  EXPECT(fp8_gemm_nt_groupwise(odd, p, f, f, p, 0, 4, 128, 128, 0, 1, 128, 128, NULL), INV);
  EXPECT(fp8_gemm_nt_groupwise(NULL, p, f, f, p, 0, 4, 128, 128, 0, 1, 128, 128, NULL), INV);
  EXPECT(fp8_gemm_nt_groupwise(p, p, f, f, NULL, 0, 4, 128, 128, 0, 1, 128, 128, NULL), INV);
  EXPECT(fp8_gemm_nt_groupwise(NULL, NULL, NULL, NULL, NULL, 0, 0, 128, 128, 0, 1, 128, 128, NULL), OK);
  EXPECT(fp8_gemm_nt_groupwise(p, p, f, f, p, 0, 2147483647, 2147483647, 0, 0, 1, 128, 128, NULL), INV);
  EXPECT(fp8_gemm_nt_groupwise_fp8_out(p, p, f, f, p, NULL, 4, 128, 128, 0, 1, 128, 128, NULL), INV);
  EXPECT(fp8_gemm_nt_groupwise_fp8_out(p, p, f, f, p, (const float*)(buf + 2), 4, 128, 128, 0, 1, 128, 128, NULL), INV);
  /* contiguous forms */
  EXPECT(fp8_group_gemm_contiguous(p, p, f, f, ip, p, 0, 100, 128, 128, 2, 0, 1, 128, 128, NULL), INV);
  EXPECT(fp8_group_gemm_contiguous(p, p, f, f, ip, p, 0, 128, 100, 128, 2, 0, 1, 128, 128, NULL), INV);
  EXPECT(fp8_group_gemm_contiguous(p, p, f, f, ip, p, 0, huge * 128, 128, huge, 2, 0, 1, 128, 128, NULL), INV);
  EXPECT(fp8_group_gemm_contiguous(p, p, f, f, ip, p, 0, 128, 128, 128, neg, 0, 1, 128, 128, NULL), INV);
  EXPECT(fp8_group_gemm_contiguous(p, p, f, f, NULL, p, 0, 128, 128, 128, 2, 0, 1, 128, 128, NULL), INV);
  EXPECT(fp8_group_gemm_contiguous(p, p, f, f, ip, p, 0, 0, 128, 128, 2, 0, 1, 128, 128, NULL), OK);
  EXPECT(fp8_group_gemm_contiguous_gather(p, f, 10, NULL, p, f, ip, p, 0, 128, 128, 128, 2, 0, 1, 128, 128, NULL), INV);
  EXPECT(fp8_group_gemm_contiguous_gather(p, f, neg, ip, p, f, ip, p, 0, 128, 128, 128, 2, 0, 1, 128, 128, NULL), INV);
  EXPECT(fp8_group_gemm_contiguous_per_tensor(p, 128, NULL, p, NULL, ip, p, 0, 128, 128, 128, 2, NULL), INV);
  EXPECT(fp8_moe_fc1_silu_quant(p, f, 128, ip, p, f, ip, p, (float*)f, 128, 100, 128, 2, 0, 1, 128, 128, NULL), INV);
  EXPECT(fp8_moe_fc1_silu_quant(p, f, 128, ip, p, f, ip, NULL, (float*)f, 128, 128, 128, 2, 0, 1, 128, 128, NULL), INV);
  EXPECT(fp8_moe_fc1_silu_quant(p, f, 128, ip, p, f, ip, p, (float*)f, 128, huge, 128, 2, 0, 1, 128, 128, NULL), INV);
  EXPECT(fp8_moe_fc1_silu_quant_per_tensor(p, 128, ip, p, f, f, 2, ip, p, 128, 128, 128, 2, NULL), INV);
  EXPECT(fp8_moe_fc1_silu_quant_per_tensor(p, 128, ip, p, NULL, f, 0, ip, p, 128, 128, 128, 2, NULL), INV);
  /* masked form */
  EXPECT(fp8_batch_gemm_masked(p, p, f, f, ip, -1, p, 0, 2, 64, 128, 128, 0, 1, 128, 128, NULL), INV);
  EXPECT(fp8_batch_gemm_masked(p, p, f, f, ip, 8, p, 0, 70000, 64, 128, 128, 0, 1, 128, 128, NULL), INV);
  EXPECT(fp8_batch_gemm_masked(p, p, f, f, NULL, 8, p, 0, 2, 64, 128, 128, 0, 1, 128, 128, NULL), INV);
  EXPECT(fp8_batch_gemm_masked(p, p, f, f, ip, 8, p, 0, 2, huge, huge, 128, 0, 1, 128, 128, NULL), INV);
  EXPECT(fp8_batch_gemm_masked(p, p, f, f, ip, 8, p, 0, 0, 64, 128, 128, 0, 1, 128, 128, NULL), OK);
  /* bmm */
  EXPECT(fp8_bmm(p, p, f, 0, f, 0, p, 0, 2, 64, 100, 128, NULL), INV);
  EXPECT(fp8_bmm(p, p, f, 0, f, 0, p, 0, 2, 64, 128, 100, NULL), INV);
  EXPECT(fp8_bmm(p, p, f, 2, f, 0, p, 0, 2, 64, 128, 128, NULL), INV);
  EXPECT(fp8_bmm(p, p, f, 0, f, 0, p, 0, 70000, 64, 128, 128, NULL), INV);
  EXPECT(fp8_bmm(p, p, f, 0, f, 0, p, 0, 2, huge, huge, 128, NULL), INV);
  EXPECT(fp8_bmm(p, NULL, f, 0, f, 0, p, 0, 2, 64, 128, 128, NULL), INV);
  /* producers */
  EXPECT(fp8_quantize_1x128(p, 4, 100, p, (float*)f, 0, NULL), INV);
  EXPECT(fp8_quantize_1x128(p, huge, huge * 128, p, (float*)f, 0, NULL), INV);
  EXPECT(fp8_quantize_1x128(odd, 4, 128, p, (float*)f, 0, NULL), INV);
  EXPECT(fp8_quantize_1x128(p, 4, 128, p, (float*)f, 5, NULL), INV);
  EXPECT(fp8_fused_add_rmsnorm_quant(p, (float*)f, p, p, p, p, -1.0f, 4, 128, 0, NULL), INV);
  EXPECT(fp8_fused_add_rmsnorm_quant(p, (float*)f, p, p, p, p, 1e-6f, huge, huge, 0, NULL), INV);
  EXPECT(fp8_fused_add_rmsnorm_quant(p, (float*)f, p, p, p, p, 1e-6f, 4, 128, 0, NULL), INV); /* aliasing */
  /* expert-FFN steps */
  EXPECT(fp8_moe_build_permutation(ip, 4, 2, 3, 256, (int32_t*)ip, (int32_t*)ip, (int32_t*)ip, p, 1 << 20, NULL), INV);
  EXPECT(fp8_moe_build_permutation(ip, huge, huge, 3, 256, (int32_t*)ip, (int32_t*)ip, (int32_t*)ip, p, 0, NULL), INV);
  EXPECT(fp8_moe_build_permutation(ip, 4, 2, 2000, 1 << 20, (int32_t*)ip, (int32_t*)ip, (int32_t*)ip, p, 0, NULL), INV);
  EXPECT(fp8_moe_build_permutation(ip, 4, 2, 3, 512, (int32_t*)ip, (int32_t*)ip, (int32_t*)ip, p, 11, NULL), INV);
  EXPECT(fp8_moe_build_permutation(ip, 4, 2, 3, 512, (int32_t*)ip, (int32_t*)ip, (int32_t*)ip, NULL, 1 << 20, NULL), INV);
  EXPECT(fp8_moe_build_permutation(ip, 0, 2, 3, 0, NULL, NULL, NULL, NULL, 0, NULL), INV); /* room for padding */
  EXPECT(fp8_moe_build_permutation(ip, 0, 2, 3, 384, NULL, NULL, NULL, NULL, 0, NULL), INV); /* null outputs */
  EXPECT(fp8_moe_build_permutation_noalloc(ip, 1 << 18, 8, 1024, (int64_t)1 << 22, (int32_t*)ip, (int32_t*)ip,
                                           (int32_t*)ip, NULL), INV);
  if (fp8_moe_permutation_workspace_size(huge, huge, 3) != -1 || fp8_moe_permutation_workspace_size(4, 2, 3) != 12)
    return 4;
  EXPECT(fp8_moe_gather_quant(p, ip, 4, 100, 128, p, (float*)f, NULL), INV);
  EXPECT(fp8_moe_gather_quant(p, ip, huge, huge, huge, p, (float*)f, NULL), INV);
  EXPECT(fp8_moe_silu_mul_quant(p, ip, 128, 100, p, (float*)f, NULL), INV);
  EXPECT(fp8_moe_silu_mul_quant(p, ip, huge, huge, p, (float*)f, NULL), INV);
  EXPECT(fp8_moe_combine(p, ip, f, 4, 65, 128, 128, p, 0, NULL), INV);
  EXPECT(fp8_moe_combine(p, ip, f, huge, 8, huge, 128, p, 0, NULL), INV);
  EXPECT(fp8_moe_combine(p, ip, f, 0, 8, 128, 128, p, 0, NULL), OK);
  /* measurement aids */
  EXPECT(fp8g_clock_probe(NULL, 10, NULL), INV);
  EXPECT(fp8g_clock_probe((unsigned long long*)buf, -1, NULL), INV);
  EXPECT(fp8g_gemm_clock_record(NULL), INV);
  printf("ok %d\n", calls);
  return 0;
}
