/*
 * The C ABI used from plain C99: this file includes include/jscan.h, takes the
 * address of every entry point (so that linking against libjscan.so resolves
 * each one) and calls the entry points that do no GPU work.  Built and run by
 * tests/test_c_abi.py.  Exit status 0 on success; a message on stderr otherwise.
 */
#include <stdio.h>
#include <string.h>

#include "jscan.h"

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                       \
    }                                                                 \
  } while (0)

int main(void) {
  /* every entry point, as a generic function pointer (a conversion ISO C allows) */
  typedef void (*fn)(void);
  const fn entry[] = {
      (fn)&jscan_prefill_workspace_size, (fn)&jscan_prefill,          (fn)&jscan_step,
      (fn)&jscan_prefill_noalloc,
      (fn)&jscan_step_batch,             (fn)&jscan_prefill_fused,    (fn)&jscan_step_batch_fused,
      (fn)&jscan_prefill_trap,           (fn)&jscan_step_batch_trap,  (fn)&jscan_backward_workspace_size,
      (fn)&jscan_backward,               (fn)&jscan_backward_saved,   (fn)&jscan_status_string,
      (fn)&jscan_last_error,             (fn)&jscan_prefill_plan,     (fn)&jscan_set_plan_override,
      (fn)&jscan_time_next_prefill,      (fn)&jscan_prefill_stats,    (fn)&jscan_step_workspace_size,
      (fn)&jscan_step_batch_fused_ws};
  size_t i;
  int waves = 0, chunks = 0;
  for (i = 0; i < sizeof(entry) / sizeof(entry[0]); ++i) CHECK(entry[i] != NULL);

  CHECK(strcmp(jscan_status_string(JSCAN_OK), "") != 0);
  CHECK(jscan_prefill_workspace_size(1, 65536, 8192, 16, JSCAN_IO_BF16) > 0);
  CHECK(jscan_prefill_workspace_size(1, 65536, 8192, 15, JSCAN_IO_BF16) == 0);
  CHECK(jscan_backward_workspace_size(1, 65536, 8192, 16, JSCAN_IO_BF16) >
        jscan_prefill_workspace_size(1, 65536, 8192, 16, JSCAN_IO_BF16));
  CHECK(jscan_prefill_plan(1, 65536, 8192, 16, &waves, &chunks) == JSCAN_OK);
  CHECK(waves >= 1 && chunks > 1);
  /* a rejected call names its reason */
  CHECK(jscan_prefill(1, 8, 64, 8, JSCAN_IO_BF16, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                      NULL, 0, NULL) == JSCAN_ERR_UNSUPPORTED);
  CHECK(strlen(jscan_last_error()) > 0);
  CHECK(jscan_set_plan_override(3, 1) == JSCAN_ERR_UNSUPPORTED);
  {
    double stats[3];
    CHECK(jscan_prefill_stats(NULL, 0, 1, 65536, 8192, stats, NULL) == JSCAN_ERR_NULL);
  }
  {
    /* the decode step's workspace: only RMSNorm needs one */
    jscan_prologue pro;
    memset(&pro, 0, sizeof pro);
    CHECK(jscan_step_workspace_size(256, 8192, 16, JSCAN_IO_BF16, &pro) == 0);
    CHECK(jscan_step_workspace_size(256, 8192, 16, JSCAN_IO_BF16, NULL) == 0);
    pro.rms_B_weight = (const float*)(size_t)256;   /* only tested against NULL here */
    CHECK(jscan_step_workspace_size(256, 8192, 16, JSCAN_IO_BF16, &pro) >= 256 * 132);
    CHECK(jscan_step_workspace_size(256, 8192, 15, JSCAN_IO_BF16, &pro) == 0);
  }
  printf("c abi ok: %d waves, %d chunks at 1 x 65536 x 8192\n", waves, chunks);
  return 0;
}
