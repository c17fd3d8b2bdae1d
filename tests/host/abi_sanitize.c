/* Host-side exercise of the C ABI, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer over a host-only build of the library (no
 * device code, no GPU).  It drives every path that runs on the host before
 * the first device call: config checks and buffer sizing over the whole
 * accepted range and past it, argument checks of create/route/forward/
 * stack/trace, the NULL-handle paths and the per-thread error message.
 * Where no HIP device is present it also lets create run into the failing
 * runtime call, which exercises the clean-up of a half-made handle (the leak
 * checker sees it).  Prints "ok <n checks>" and exits 0 when every check
 * holds. */
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "strata_moe.h"

extern int hipGetDeviceCount(int* count);   /* from the HIP runtime */

static int n_checks, n_failed;

#define CHECK(cond)                                                         \
  do {                                                                      \
    ++n_checks;                                                             \
    if (!(cond)) {                                                          \
      ++n_failed;                                                           \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
    }                                                                       \
  } while (0)

static strata_moe_config cfg(int H, int I, int E, int k, int shared, int fmt, int T) {
  strata_moe_config c;
  memset(&c, 0, sizeof c);
  c.hidden = H; c.inter = I; c.n_experts = E; c.top_k = k;
  c.n_shared = shared; c.qfmt = fmt; c.max_tokens = T;
  return c;
}

static size_t block_bytes(int fmt) { return fmt == STRATA_MXFP4 ? 17 : (size_t)(4 * fmt + 2); }

static void sizes_of_valid_configs(void) {
  static const int fmts[] = {STRATA_Q2, STRATA_Q3, STRATA_Q4, STRATA_MXFP4};
  static const int widths[] = {32, 96, 256, 800, 2560, 2592, 7168};
  static const int tokens[] = {1, 8, 9, 8192, 32768};
  for (size_t f = 0; f < sizeof fmts / sizeof *fmts; ++f)
    for (size_t a = 0; a < sizeof widths / sizeof *widths; ++a)
      for (size_t b = 0; b < sizeof widths / sizeof *widths; b += 2)
        for (size_t t = 0; t < sizeof tokens / sizeof *tokens; t += 2) {
          const strata_moe_config c = cfg(widths[a], widths[b], 512, 10, (int)(t & 1), fmts[f], tokens[t]);
          const size_t eb = strata_moe_expert_bytes(&c);
          CHECK(eb == 3 * (size_t)c.inter * (size_t)(c.hidden / 32) * block_bytes(c.qfmt));
          CHECK(strata_moe_packed_bytes(&c) >= (size_t)(c.n_experts + c.n_shared) * eb);
          CHECK(strata_moe_workspace_bytes(&c) > 0);
        }
  /* the edges of the accepted ranges */
  const strata_moe_config edge[] = {
      cfg(32, 32, 1, 1, 0, STRATA_Q2, 1),        cfg(32, 32, 4096, 4096, 0, STRATA_Q2, 4),
      cfg(65536, 1024, 8, 2, 0, STRATA_Q2, 1),   cfg(7168, 2048, 256, 8, 1, STRATA_MXFP4, 2048),
      cfg(2560, 512, 512, 512, 0, STRATA_Q3, 64),
  };
  for (size_t i = 0; i < sizeof edge / sizeof *edge; ++i) {
    CHECK(strata_moe_expert_bytes(&edge[i]) > 0);
    CHECK(strata_moe_packed_bytes(&edge[i]) > 0);
    CHECK(strata_moe_workspace_bytes(&edge[i]) > 0);
  }
}

static void invalid_configs(void) {
  const strata_moe_config bad[] = {
      cfg(2560, 512, 512, 10, 0, 1, 8),      cfg(2560, 512, 512, 10, 0, 6, 8),
      cfg(2500, 512, 512, 10, 0, 2, 8),      cfg(2560, 100, 512, 10, 0, 2, 8),
      cfg(0, 512, 512, 10, 0, 2, 8),         cfg(-32, 512, 512, 10, 0, 2, 8),
      cfg(65568, 512, 512, 10, 0, 2, 8),     cfg(2560, 512, 0, 1, 0, 2, 8),
      cfg(2560, 512, 4097, 10, 0, 2, 8),     cfg(2560, 512, 512, 0, 0, 2, 8),
      cfg(2560, 512, 512, 513, 0, 2, 8),     cfg(2560, 512, 512, 10, 2, 2, 8),
      cfg(2560, 512, 512, 10, -1, 2, 8),     cfg(2560, 512, 512, 10, 0, 2, 0),
      cfg(2560, 512, 512, 512, 0, 2, 1 << 20),                 /* T * k past 2^28 */
      cfg(65536, 512, 512, 10, 0, 2, 1 << 15),                 /* token rows past 4 GiB */
      cfg(65536, 65536, 8, 2, 0, STRATA_Q4, 1),                /* one expert past 2 GiB */
      cfg(2147483616, 512, 512, 10, 0, 2, 8),                  /* int overflow bait */
      cfg(2560, 2147483616, 512, 10, 0, 2, 8),
  };
  for (size_t i = 0; i < sizeof bad / sizeof *bad; ++i) {
    CHECK(strata_moe_expert_bytes(&bad[i]) == 0);
    CHECK(strata_moe_packed_bytes(&bad[i]) == 0);
    CHECK(strata_moe_workspace_bytes(&bad[i]) == 0);
    strata_moe* h = (strata_moe*)1;
    void* p = (void*)(uintptr_t)4096;
    const int rc = strata_moe_create(&bad[i], (const float*)p, NULL, p, NULL, p, p, NULL, &h);
    CHECK(rc == STRATA_E_INVALID || rc == STRATA_E_UNSUPPORTED);
    CHECK(strlen(strata_moe_last_error()) > 0);
  }
  CHECK(strata_moe_expert_bytes(NULL) == 0);
  CHECK(strata_moe_packed_bytes(NULL) == 0);
  CHECK(strata_moe_workspace_bytes(NULL) == 0);
}

static void create_argument_checks(void) {
  const strata_moe_config c = cfg(2560, 512, 512, 10, 0, STRATA_Q2, 8);
  void* p = (void*)(uintptr_t)4096;
  const float* w = (const float*)p;
  strata_moe* h = NULL;
  CHECK(strata_moe_create(&c, w, NULL, p, NULL, p, p, NULL, NULL) == STRATA_E_INVALID);
  CHECK(strata_moe_create(&c, NULL, NULL, p, NULL, p, p, NULL, &h) == STRATA_E_INVALID && h == NULL);
  CHECK(strstr(strata_moe_last_error(), "non-NULL") != NULL);
  CHECK(strata_moe_create(&c, w, NULL, NULL, NULL, p, p, NULL, &h) == STRATA_E_INVALID);
  CHECK(strata_moe_create(&c, w, NULL, p, NULL, NULL, p, NULL, &h) == STRATA_E_INVALID);
  CHECK(strata_moe_create(&c, w, NULL, p, NULL, p, NULL, NULL, &h) == STRATA_E_INVALID);
  CHECK(strata_moe_create(&c, w, NULL, p, p, p, p, NULL, &h) == STRATA_E_INVALID);      /* shared, n_shared 0 */
  CHECK(strstr(strata_moe_last_error(), "shared") != NULL);
  const strata_moe_config cs = cfg(2560, 512, 512, 10, 1, STRATA_Q2, 8);
  CHECK(strata_moe_create(&cs, w, NULL, p, NULL, p, p, NULL, &h) == STRATA_E_INVALID);  /* no shared record */
  void* mis = (void*)(uintptr_t)(4096 + 16);
  CHECK(strata_moe_create(&c, w, NULL, p, NULL, mis, p, NULL, &h) == STRATA_E_INVALID);
  CHECK(strstr(strata_moe_last_error(), "aligned") != NULL);
  CHECK(strata_moe_create(&c, w, NULL, p, NULL, p, mis, NULL, &h) == STRATA_E_INVALID);
  CHECK(strata_moe_create(&c, (const float*)(uintptr_t)4100, NULL, p, NULL, p, p, NULL, &h) == STRATA_E_INVALID);
  CHECK(strata_moe_create(&c, w, (const float*)(uintptr_t)4098, p, NULL, p, p, NULL, &h) == STRATA_E_INVALID);
  CHECK(h == NULL);
}

/* With no device, create gets past every argument check and fails at its
 * first runtime call; the half-made handle must be released. */
static void create_without_device(void) {
  int n = 0;
  if (hipGetDeviceCount(&n) == 0 && n > 0) return;     /* never hand fake addresses to a device */
  const strata_moe_config c = cfg(2560, 512, 512, 10, 1, STRATA_Q3, 64);
  void* p = (void*)(uintptr_t)4096;
  for (int i = 0; i < 3; ++i) {
    strata_moe* h = (strata_moe*)1;
    const int rc = strata_moe_create(&c, (const float*)p, NULL, p, p, p, p, NULL, &h);
    CHECK(rc == STRATA_E_HIP);
    CHECK(h == NULL);
    CHECK(strstr(strata_moe_last_error(), "create") != NULL);
  }
}

static void null_handle_calls(void) {
  void* p = (void*)(uintptr_t)4096;
  CHECK(strata_moe_forward(NULL, p, STRATA_BF16, 1, (float*)p, 0, NULL) == STRATA_E_INVALID);
  CHECK(strstr(strata_moe_last_error(), "handle") != NULL);
  CHECK(strata_moe_forward_static(NULL, p, STRATA_BF16, 1, (float*)p, 0, NULL) == STRATA_E_INVALID);
  CHECK(strata_moe_route(NULL, p, STRATA_BF16, 1, (int32_t*)p, (float*)p, (int32_t*)p, (int32_t*)p, 0, NULL) ==
        STRATA_E_INVALID);
  CHECK(strata_moe_stack_forward(NULL, 0, NULL, 0, 1, NULL, NULL, NULL) == STRATA_E_INVALID);
  strata_moe* layers[2] = {NULL, NULL};
  CHECK(strata_moe_stack_forward(layers, 2, p, STRATA_BF16, 1, (float*)p, (float*)p, NULL) == STRATA_E_INVALID);
  CHECK(strata_moe_trace_next_call(NULL, NULL, 0) == STRATA_E_INVALID);
  strata_moe_destroy(NULL);
}

/* The error message is per thread: each thread sees its own last failure. */
static void* thread_errors(void* arg) {
  const int id = (int)(intptr_t)arg;
  for (int i = 0; i < 2000; ++i) {
    const strata_moe_config c = cfg(2560, 512, 512, id & 1 ? 513 : 10, 0, id & 1 ? STRATA_Q2 : 6, 8);
    strata_moe* h = NULL;
    strata_moe_create(&c, NULL, NULL, NULL, NULL, NULL, NULL, NULL, &h);
    const char* msg = strata_moe_last_error();
    if (!strstr(msg, id & 1 ? "top_k" : "qfmt")) return (void*)1;
    if (strata_moe_workspace_bytes(&c) != 0) return (void*)1;
  }
  return NULL;
}

static void per_thread_errors(void) {
  pthread_t th[4];
  for (int i = 0; i < 4; ++i) pthread_create(&th[i], NULL, thread_errors, (void*)(intptr_t)i);
  for (int i = 0; i < 4; ++i) {
    void* r = NULL;
    pthread_join(th[i], &r);
    CHECK(r == NULL);
  }
}

int main(void) {
  sizes_of_valid_configs();
  invalid_configs();
  create_argument_checks();
  create_without_device();
  null_handle_calls();
  per_thread_errors();
  if (n_failed) {
    fprintf(stderr, "%d of %d checks failed\n", n_failed, n_checks);
    return 1;
  }
  printf("ok %d\n", n_checks);
  return 0;
}
