/* The C-ABI from plain C (C99): include/lmhead.h compiles as C, the library
 * links, and host-side validation answers with the documented status codes
 * before anything would be queued (no pointer is dereferenced, no GPU used).
 * Prints "ok" and exits 0, or names the first failed check and exits 1. */
#include <stdint.h>
#include <stdio.h>

#include "lmhead.h"

#define CHECK(cond)                                    \
  do {                                                 \
    if (!(cond)) {                                     \
      printf("failed: %s (line %d)\n", #cond, __LINE__); \
      return 1;                                        \
    }                                                  \
  } while (0)

int main(void) {
  const void *a = (const void *)(uintptr_t)0x10000; /* aligned, never dereferenced */
  void *out = (void *)(uintptr_t)0x20000;
  CHECK(lmhead_packed_w_bytes(2048, 32000) == (size_t)250 * (128 * 4096 + 16384));
  CHECK(lmhead_packed_w_bytes(100, 32000) == 0);
  CHECK(lmhead_workspace_bytes(LMHEAD_MODE_BF16, 512, 2048, 32000) ==
        lmhead_workspace_bytes(LMHEAD_MODE_BF16_PACKED, 512, 2048, 32000));
  CHECK(lmhead_logits(LMHEAD_MODE_BF16, LMHEAD_ROUND_F32, NULL, a, 4, 64, 1000, out, NULL) ==
        LMHEAD_E_NULL);
  CHECK(lmhead_logits(3, LMHEAD_ROUND_F32, a, a, 4, 64, 1000, out, NULL) == LMHEAD_E_MODE);
  CHECK(lmhead_logits(LMHEAD_MODE_INT8, LMHEAD_ROUND_BF16, a, a, 4, 64, 1000, out, NULL) ==
        LMHEAD_E_MODE);
  CHECK(lmhead_logits(LMHEAD_MODE_BF16_PACKED, LMHEAD_ROUND_F32, a, a, 4, 96, 1000, out, NULL) ==
        LMHEAD_E_SHAPE);
  CHECK(lmhead_pack_w(a, 64, 1000, (void *)(uintptr_t)0x20008, NULL) == LMHEAD_E_ALIGN);
  CHECK(lmhead_greedy_top2(LMHEAD_MODE_INT8, LMHEAD_ROUND_F32, a, a, 4, 131072, 1000, NULL, out,
                           out, out, NULL, out, 1 << 20, NULL) == LMHEAD_E_OVERFLOW);
  CHECK(lmhead_status_string(LMHEAD_OK)[0] != '\0');
  CHECK(lmhead_source_digest()[0] != '\0');
  printf("ok\n");
  return 0;
}
