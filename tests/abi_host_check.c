/*
 * Host-only paths of the C ABI, run under AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_abi_sanitized.py builds the library's host code with both and links this driver).
 * Nothing here launches a kernel or touches device memory: configuration checks, workspace
 * sizing (the split-K planners run here), the argument and call-order errors of dllm_create and
 * of every call on a NULL handle.
 *
 * cfgs.h (written by the test) defines GOOD_CFGS[] / N_GOOD and BAD_CFGS[] / N_BAD.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dllm.h"
#include "cfgs.h"

static int failures = 0;
#define CHECK(cond)                                                        \
  do {                                                                     \
    if (!(cond)) {                                                         \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                          \
    }                                                                      \
  } while (0)

int main(void) {
  for (int i = 0; i < N_GOOD; ++i) {
    CHECK(dllm_validate_cfg(&GOOD_CFGS[i]) == DLLM_OK);
    size_t n = 0;
    CHECK(dllm_workspace_bytes(&GOOD_CFGS[i], &n) == DLLM_OK);
    CHECK(n > 0);
    CHECK(dllm_workspace_bytes(&GOOD_CFGS[i], NULL) == DLLM_EINVAL);
    /* dllm_create rejects every bad argument before any device work */
    const void *layer[9 * 64];
    for (int j = 0; j < 9 * 64; ++j) layer[j] = (const void *)(uintptr_t)0x1000;
    dllm_weights w = {(const void *)(uintptr_t)0x1000, (const void *)(uintptr_t)0x1000,
                      (const void *)(uintptr_t)0x1000, layer};
    dllm_t *h = (dllm_t *)(uintptr_t)0x1;
    CHECK(dllm_create(&w, &GOOD_CFGS[i], NULL, n, &h) == DLLM_EINVAL);
    CHECK(h == NULL);
    CHECK(strlen(dllm_last_error(NULL)) > 0);
    CHECK(dllm_create(&w, &GOOD_CFGS[i], (void *)(uintptr_t)0x1010, n, &h) == DLLM_EINVAL);
    CHECK(dllm_create(&w, &GOOD_CFGS[i], (void *)(uintptr_t)0x100000, n - 1, &h) == DLLM_ENOSPACE);
    CHECK(strstr(dllm_last_error(NULL), "workspace") != NULL);
    CHECK(dllm_create(NULL, &GOOD_CFGS[i], (void *)(uintptr_t)0x100000, n, &h) == DLLM_EINVAL);
    CHECK(dllm_create(&w, NULL, (void *)(uintptr_t)0x100000, n, &h) == DLLM_EINVAL);
    CHECK(dllm_create(&w, &GOOD_CFGS[i], (void *)(uintptr_t)0x100000, n, NULL) == DLLM_EINVAL);
    layer[3] = NULL;
    CHECK(dllm_create(&w, &GOOD_CFGS[i], (void *)(uintptr_t)0x100000, n, &h) == DLLM_EINVAL);
  }
  for (int i = 0; i < N_BAD; ++i) {
    CHECK(dllm_validate_cfg(&BAD_CFGS[i]) == DLLM_EINVAL);
    size_t n = 0;
    CHECK(dllm_workspace_bytes(&BAD_CFGS[i], &n) == DLLM_EINVAL);
  }
  CHECK(dllm_validate_cfg(NULL) == DLLM_EINVAL);
  /* every call on a NULL handle fails cleanly */
  int32_t buf[4];
  float fbuf[4];
  uint8_t ubuf[4];
  dllm_stats st;
  dllm_kernel_prof kp[DLLM_KC_COUNT];
  CHECK(dllm_prefill(NULL, buf) == DLLM_EINVAL);
  CHECK(dllm_block_begin(NULL, 0) == DLLM_EINVAL);
  CHECK(dllm_denoise_step(NULL, buf, buf) == DLLM_EINVAL);
  CHECK(dllm_generate(NULL, buf, buf, &st) == DLLM_EINVAL);
  CHECK(dllm_get_tokens(NULL, buf) == DLLM_EINVAL);
  CHECK(dllm_set_tokens(NULL, buf) == DLLM_EINVAL);
  CHECK(dllm_get_step_info(NULL, buf, fbuf, fbuf, ubuf) == DLLM_EINVAL);
  CHECK(dllm_debug_block_logits(NULL, fbuf) == DLLM_EINVAL);
  CHECK(dllm_get_stats(NULL, &st) == DLLM_EINVAL);
  CHECK(dllm_get_position(NULL, buf, buf) == DLLM_EINVAL);
  CHECK(dllm_set_profiling(NULL, 1) == DLLM_EINVAL);
  CHECK(dllm_get_profile(NULL, kp) == DLLM_EINVAL);
  dllm_destroy(NULL);
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("abi host checks ok (%d good, %d bad configurations)\n", N_GOOD, N_BAD);
  return 0;
}
