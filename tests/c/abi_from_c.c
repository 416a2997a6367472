/* Uses the library from plain C through include/fp8g.h: version, argument validation and the
 * thread's last-error message. No GPU is touched (every call here fails validation or is empty). */
#include <stdio.h>
#include <string.h>

#include "fp8g.h"

int main(void) {
  if (fp8g_version() < 100) return 1;
  /* k = 100 is not a multiple of 128: rejected before any device work */
  char dummy[64] __attribute__((aligned(16)));
  fp8g_status_t st = fp8_gemm_nt_groupwise(dummy, dummy, (const float*)dummy, (const float*)dummy, dummy,
                                           FP8G_OUT_BF16, 4, 128, 100, FP8G_SCALE_K_MAJOR, 1, 128, 128, NULL);
  if (st != FP8G_INVALID_ARGUMENT || strstr(fp8g_last_error(), "k (100)") == NULL) return 2;
  /* an empty problem succeeds and clears the message */
  st = fp8_gemm_nt_groupwise(NULL, NULL, NULL, NULL, NULL, FP8G_OUT_BF16, 0, 128, 128, FP8G_SCALE_K_MAJOR,
                             1, 128, 128, NULL);
  if (st != FP8G_OK || fp8g_last_error()[0] != '\0') return 3;
  printf("ok\n");
  return 0;
}
