/* Host-only check of the C ABI's argument validation, built with the host
 * library (ipttt.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_host_asan.py. Device pointers are fake (aligned host buffers):
 * every call below must be rejected, or be a no-op, before any device work,
 * so no GPU is needed. Exits 0 when every expectation holds. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ipttt.h"

static int failures = 0;

#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expectation failed: %s (last error: %s)\n", __FILE__, __LINE__, \
              #cond, ipttt_last_error());                              \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static unsigned char arena[1 << 20];
static size_t arena_used = 0;

/* 256-byte aligned fake device buffer */
static void *fake(size_t bytes) {
  uintptr_t base = ((uintptr_t)(arena + arena_used) + 255u) & ~(uintptr_t)255u;
  arena_used = (size_t)(base - (uintptr_t)arena) + bytes;
  if (arena_used > sizeof arena) {
    fprintf(stderr, "arena exhausted\n");
    exit(2);
  }
  return (void *)base;
}

static ipttt_layer_desc make_desc(void) {
  ipttt_layer_desc d;
  memset(&d, 0, sizeof d);
  d.d = 64;
  d.d_ff = 256;
  d.conv_k = 4;
  d.chunk = 128;
  d.max_batch = 2;
  d.eta = 0.01f;
  d.update = IPTTT_UPDATE_LINEAR;
  d.in_dtype = IPTTT_BF16;
  d.w_gate = fake(4096);
  d.w_up = fake(4096);
  d.proj = fake(4096);
  d.conv_w = fake(4096);
  d.w0 = (const float *)fake(4096);
  d.w_state = (float *)fake(4096);
  d.workspace = fake(4096);
  d.workspace_bytes = ipttt_workspace_bytes(&d, 1, 1);
  return d;
}

int main(void) {
  EXPECT(strcmp(ipttt_status_str(IPTTT_E_WORKSPACE), "IPTTT_E_WORKSPACE") == 0);
  EXPECT(strcmp(ipttt_status_str((ipttt_status)7), "IPTTT_E_UNKNOWN") == 0);

  ipttt_layer_desc d = make_desc();
  EXPECT(d.workspace_bytes > 0);
  EXPECT(ipttt_workspace_bytes(&d, 0, 1) == 0);
  EXPECT(ipttt_workspace_bytes(&d, 1, 0) == 0);
  EXPECT(ipttt_workspace_bytes(NULL, 1, 1) == 0);
  EXPECT(ipttt_backward_workspace_bytes(&d, 1, 128) > 0);

  ipttt_layer *h = NULL;
  EXPECT(ipttt_init(NULL, &h) == IPTTT_E_INVALID);
  EXPECT(ipttt_init(&d, NULL) == IPTTT_E_INVALID);
  {
    ipttt_layer_desc bad = d;
    bad.conv_k = 9;
    EXPECT(ipttt_init(&bad, &h) == IPTTT_E_UNSUPPORTED);
    bad = d;
    bad.w_up = (const char *)d.w_up + 8;
    EXPECT(ipttt_init(&bad, &h) == IPTTT_E_INVALID);
    bad = d;
    bad.workspace_bytes -= 1;
    EXPECT(ipttt_init(&bad, &h) == IPTTT_E_WORKSPACE);
    bad = d;
    bad.eta = 1.0f / 0.0f;
    EXPECT(ipttt_init(&bad, &h) == IPTTT_E_INVALID);
  }

  EXPECT(ipttt_init(&d, &h) == IPTTT_OK);
  EXPECT(h != NULL);
  void *x = fake(4096), *e = fake(4096);
  float *o = (float *)fake(4096);
  /* batch beyond max_batch, never-reset sequences, null and misaligned buffers */
  EXPECT(ipttt_prefill_layer(h, x, e, o, 3, 128, NULL) == IPTTT_E_INVALID);
  EXPECT(ipttt_prefill_layer(h, x, e, o, 1, 128, NULL) == IPTTT_E_STATE);
  EXPECT(ipttt_prefill_layer(h, NULL, e, o, 1, 128, NULL) == IPTTT_E_INVALID);
  EXPECT(ipttt_prefill_layer(h, (char *)x + 2, e, o, 1, 128, NULL) == IPTTT_E_INVALID);
  EXPECT(ipttt_prefill_layer(h, x, e, o, 0, 128, NULL) == IPTTT_OK);
  EXPECT(ipttt_prefill_layer(h, x, e, o, 1, 0, NULL) == IPTTT_OK);
  EXPECT(ipttt_prefill_layer_noalloc(h, x, e, o, 3, 128, NULL) == IPTTT_E_INVALID);
  EXPECT(ipttt_prefill_layer_noalloc(h, x, e, o, 1, 128, NULL) == IPTTT_E_STATE);
  EXPECT(ipttt_prefill_layer_noalloc(h, x, e, o, -1, 128, NULL) == IPTTT_E_INVALID);
  EXPECT(ipttt_prefill_layer_noalloc(h, x, e, o, 0, 128, NULL) == IPTTT_OK);
  {
    int64_t starts[2] = {9, 3};
    EXPECT(ipttt_prefill_packed(h, x, e, o, 0, 128, starts, 2, NULL) == IPTTT_E_INVALID);
    starts[0] = 7;
    EXPECT(ipttt_prefill_packed(h, x, e, o, 0, 128, starts, 1, NULL) == IPTTT_E_STATE);
    EXPECT(ipttt_prefill_packed(h, x, e, o, 2, 128, starts, 0, NULL) == IPTTT_E_INVALID);
  }
  EXPECT(ipttt_decode_step(h, x, e, 128 * 64, 128, o, 1, NULL) == IPTTT_E_INVALID);
  EXPECT(ipttt_decode_step(h, x, e, 128 * 64, 3, o, 1, NULL) == IPTTT_E_STATE);
  EXPECT(ipttt_reset_fast_weights(h, 1, 2, NULL) == IPTTT_E_INVALID);
  EXPECT(ipttt_reset_fast_weights(h, 1, 0, NULL) == IPTTT_OK);
  {
    ipttt_grads g;
    g.dx = g.de = g.dw_gate = g.dw_up = g.dproj = g.dconv_w = g.dw0 = (float *)fake(4096);
    size_t need = ipttt_backward_workspace_bytes(&d, 1, 128);
    void *ws = fake(256);
    EXPECT(ipttt_backward_layer(h, x, e, o, NULL, 1, 128, &g, ws, need - 1, NULL) ==
           IPTTT_E_WORKSPACE);
    EXPECT(ipttt_backward_layer(h, x, e, o, NULL, 1, 128, NULL, ws, need, NULL) == IPTTT_E_INVALID);
    g.dproj = NULL;
    EXPECT(ipttt_backward_layer(h, x, e, o, NULL, 1, 128, &g, ws, need, NULL) == IPTTT_E_INVALID);
  }
  EXPECT(ipttt_profile_begin(h) == IPTTT_OK);
  {
    int32_t n[IPTTT_K_COUNT];
    double ms[IPTTT_K_COUNT];
    EXPECT(ipttt_profile_end(h, n, ms) == IPTTT_OK);
    EXPECT(ipttt_profile_end(h, NULL, ms) == IPTTT_E_INVALID);
  }
  ipttt_destroy(h);
  ipttt_destroy(NULL);
  EXPECT(ipttt_prefill_layer(NULL, x, e, o, 1, 1, NULL) == IPTTT_E_INVALID);
  EXPECT(ipttt_prefill_layer_noalloc(NULL, x, e, o, 1, 1, NULL) == IPTTT_E_INVALID);

  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("abi_asan: all checks passed\n");
  return 0;
}
