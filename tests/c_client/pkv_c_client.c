/* A plain C99 client of libpkv: includes pkv.h, links libpkv.so, and calls
 * entry points whose arguments the host checks reject (or that carry no
 * work), so it runs without a GPU.  Exit status 0 when every status code
 * and message is the one pkv.h documents; otherwise the number of the
 * failed check. */
#include "pkv.h"

#include <stdio.h>
#include <string.h>

static int expect(int got, int want, const char *needle, int check) {
  const char *msg = pkv_last_error();
  if (got != want || (needle && !strstr(msg, needle)) || (!needle && msg[0] != '\0')) {
    fprintf(stderr, "check %d: status %d (want %d), message \"%s\"\n", check, got, want, msg);
    return check;
  }
  return 0;
}

int main(void) {
  /* 16-byte aligned stand-ins for device addresses; never dereferenced */
  void *const A = (void *)(uintptr_t)(1u << 20);
  int bad = 0;
  if (pkv_abi_version() != PKV_ABI_VERSION) return 1;
  bad = bad ? bad : expect(pkv_gather_indexer_k_fp8(A, A, A, A, A, 2, 4, 57, 8, 64 * 132, 64, 100, NULL),
                           PKV_EUNSUPPORTED, "multiple of 16", 2);
  bad = bad ? bad : expect(pkv_gather_indexer_k_fp8(A, A, A, A, A, 0, 4, 57, 8, 64 * 132, 64, 128, NULL),
                           PKV_OK, NULL, 3);
  bad = bad ? bad : expect(pkv_store_indexer_k_fp8(A, 128, PKV_DTYPE_BF16, A, 0, A, 4, 64 * 132, 64, 128, NULL),
                           PKV_OK, NULL, 4);
  bad = bad ? bad : expect(pkv_store_indexer_k_fp8(A, 128, 7, A, 10, A, 4, 64 * 132, 64, 128, NULL),
                           PKV_EINVAL, "k_dtype", 5);
  bad = bad ? bad : expect(pkv_store_kv_fp4(A, 256, A, 256, PKV_DTYPE_BF16, A, A, A, 10, 2, 128, 6, 8,
                                            2 * 2 * 6 * 72, PKV_LAYOUT_HND, (const float *)A,
                                            (const float *)A, NULL),
                           PKV_EUNSUPPORTED, "multiple of 4", 6);
  bad = bad ? bad : expect(pkv_paged_attention_decode(A, (float *)A, (float *)A, (float *)A, A, A, A,
                                                      (const int32_t *)A, (const int32_t *)A, 4, 64, 8,
                                                      128, 16, 8, 100, 64, 0.1f, 1.0f, 1.0f, 100, NULL),
                           PKV_EUNSUPPORTED, "partition_size", 7);
  bad = bad ? bad : expect(pkv_fp8_mqa_logits(A, 8192, A, (const float *)A, (const float *)A,
                                              (const int32_t *)A, (const int32_t *)A, (float *)A, 8, 8,
                                              4, 64, 16, 128, NULL),
                           PKV_EUNSUPPORTED, "not enabled", 8);
  if (!bad) printf("c client ok\n");
  return bad;
}
