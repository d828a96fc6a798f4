/* Host-side checks of the C ABI without a GPU, built with AddressSanitizer
 * and UndefinedBehaviorSanitizer on the host code (tests/test_abi_sanitized_cpu.py
 * builds and runs it).  Every call below is either a validation failure,
 * which must return before any HIP call, or a size query; with no GPU the
 * one well-formed call must fail in its first HIP call.  Device pointers are
 * fake, never dereferenced addresses.  Exit status 0 = every check held. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fwpkm.h"

static int failures = 0;
#define CHECK(cond)                                                                \
  do {                                                                             \
    if (!(cond)) {                                                                 \
      fprintf(stderr, "check failed at line %d: %s (last error: %s)\n", __LINE__, \
              #cond, fwpkm_last_error());                                          \
      ++failures;                                                                  \
    }                                                                              \
  } while (0)

#define FAKE(x) ((void*)(uintptr_t)(x))

static fwpkm_config base_cfg(void) {
  fwpkm_config c;
  memset(&c, 0, sizeof(c));
  c.sqrt_slots = 32;
  c.dim_qk = 64;
  c.dim_v = 64;
  c.topk = 4;
  c.chunk_size = 64;
  c.num_heads = 1;
  c.max_batch = 2;
  c.eps = 1e-3f;
  c.score_mode = FWPKM_SCORE_IDW;
  c.addr_weight = 0.0f;
  return c;
}

static fwpkm_state state(uintptr_t k1, uintptr_t k2, uintptr_t v, int64_t sk, int64_t sv) {
  fwpkm_state s;
  s.k1 = (float*)FAKE(k1);
  s.k2 = (float*)FAKE(k2);
  s.v = (float*)FAKE(v);
  s.batch_stride_k = sk;
  s.batch_stride_v = sv;
  return s;
}

int main(void) {
  const uintptr_t Q = 0x1000000000ull, Y = 0x2000000000ull, R = 0x3000000000ull;
  const uintptr_t PK1 = 0x4000000000ull, PK2 = 0x5000000000ull, PV = 0x6000000000ull;
  const uintptr_t NK1 = 0x7000000000ull, NK2 = 0x8000000000ull, NV = 0x9000000000ull;
  const int64_t SK = 32 * 32, SV = 1024 * 64;

  /* configurations */
  fwpkm_handle* h = NULL;
  fwpkm_config c = base_cfg();
  CHECK(fwpkm_create(NULL, &h) == FWPKM_ERR_INVALID_ARG);
  CHECK(fwpkm_create(&c, NULL) == FWPKM_ERR_INVALID_ARG);
  c.dim_qk = 63;
  CHECK(fwpkm_create(&c, &h) == FWPKM_ERR_INVALID_ARG && h == NULL);
  c = base_cfg();
  c.topk = 33;
  CHECK(fwpkm_create(&c, &h) == FWPKM_ERR_INVALID_ARG);
  c = base_cfg();
  c.eps = NAN;
  CHECK(fwpkm_create(&c, &h) == FWPKM_ERR_INVALID_ARG);
  c = base_cfg();
  c.sqrt_slots = FWPKM_MAX_SQRT_SLOTS + 1;
  c.topk = 4;
  CHECK(fwpkm_create(&c, &h) == FWPKM_ERR_UNSUPPORTED);
  CHECK(strlen(fwpkm_last_error()) > 0);
  c = base_cfg();
  CHECK(fwpkm_workspace_bytes(&c) > 0);
  CHECK(fwpkm_workspace_bytes(NULL) == 0);
  CHECK(fwpkm_sequence_workspace_bytes(&c, 2, 100) > 0);
  CHECK(fwpkm_sequence_workspace_bytes(&c, 0, 100) == 0);
  CHECK(fwpkm_create(&c, &h) == FWPKM_OK && h != NULL);

  /* chunk calls: validation failures */
  fwpkm_state past = state(PK1, PK2, PV, SK, SV), nxt = past;
  CHECK(fwpkm_forward_chunk(NULL, (float*)FAKE(Q), (float*)FAKE(Y), 2, 64, 1.f, &past, &nxt,
                            (float*)FAKE(R), NULL, NULL, NULL) == FWPKM_ERR_INVALID_ARG);
  CHECK(fwpkm_forward_chunk(h, NULL, (float*)FAKE(Y), 2, 64, 1.f, &past, &nxt, (float*)FAKE(R),
                            NULL, NULL, NULL) == FWPKM_ERR_INVALID_ARG);
  CHECK(fwpkm_forward_chunk(h, (float*)FAKE(Q), (float*)FAKE(Y), 3, 64, 1.f, &past, &nxt,
                            (float*)FAKE(R), NULL, NULL, NULL) == FWPKM_ERR_INVALID_ARG);
  CHECK(fwpkm_forward_chunk(h, (float*)FAKE(Q), (float*)FAKE(Y), 2, 65, 1.f, &past, &nxt,
                            (float*)FAKE(R), NULL, NULL, NULL) == FWPKM_ERR_INVALID_ARG);
  CHECK(fwpkm_forward_chunk(h, (float*)FAKE(Q), (float*)FAKE(Y), 2, 64, INFINITY, &past, &nxt,
                            (float*)FAKE(R), NULL, NULL, NULL) == FWPKM_ERR_INVALID_ARG);
  CHECK(fwpkm_forward_chunk(h, (float*)FAKE(Q), (float*)FAKE(Y), 2, 64, 1.f, &past, NULL,
                            (float*)FAKE(R), NULL, NULL, NULL) == FWPKM_ERR_INVALID_ARG);
  fwpkm_state part = state(PK1 + 4, NK2, NV, SK, SV);
  CHECK(fwpkm_forward_chunk(h, (float*)FAKE(Q), (float*)FAKE(Y), 2, 64, 1.f, &past, &part,
                            (float*)FAKE(R), NULL, NULL, NULL) == FWPKM_ERR_ALIAS);
  CHECK(fwpkm_forward_chunk(h, (float*)FAKE(Q), (float*)FAKE(Y), 2, 64, 1.f, &past, &nxt,
                            (float*)FAKE(Q + 16), NULL, NULL, NULL) == FWPKM_ERR_ALIAS);
  CHECK(fwpkm_forward_chunk_weighted(h, (float*)FAKE(Q), (float*)FAKE(Y), (float*)FAKE(R + 64), 2,
                                     64, 1.f, &past, &nxt, (float*)FAKE(R), NULL, NULL,
                                     NULL) == FWPKM_ERR_ALIAS);
  CHECK(fwpkm_forward_chunk_noalloc(h, (float*)FAKE(Q), (float*)FAKE(Y), 0, 64, 1.f, &past, &nxt,
                                    (float*)FAKE(R), NULL, NULL, NULL) == FWPKM_ERR_INVALID_ARG);
  CHECK(fwpkm_forward_sequence(h, NULL, (float*)FAKE(Q), (float*)FAKE(Y), NULL, 2, 10, 1.f, &past,
                               &nxt, (float*)FAKE(R), NULL, NULL, FAKE(NV), 1 << 20,
                               NULL) == FWPKM_ERR_INVALID_ARG);

  /* a well-formed call reaches its first HIP call, which fails without a GPU */
  fwpkm_state shared = state(PK1, PK2, PV, 0, 0), expanded = state(NK1, NK2, NV, SK, SV);
  const int rc = fwpkm_forward_chunk(h, (float*)FAKE(Q), (float*)FAKE(Y), 2, 64, 1.f, &shared,
                                     &expanded, (float*)FAKE(R), NULL, NULL, NULL);
  CHECK(rc == FWPKM_ERR_HIP);

  /* timing support and names */
  CHECK(fwpkm_profile_enable(NULL, 1) == FWPKM_ERR_INVALID_ARG);
  CHECK(fwpkm_profile_enable(h, 1) == FWPKM_OK);
  double ms[FWPKM_NUM_TIMED];
  int64_t launches[FWPKM_NUM_TIMED];
  CHECK(fwpkm_profile_read(h, ms, launches) == FWPKM_OK);
  CHECK(launches[0] == 0);
  CHECK(strcmp(fwpkm_kernel_name(0), "score") == 0);
  CHECK(strcmp(fwpkm_kernel_name(-1), "") == 0);
  CHECK(strcmp(fwpkm_kernel_name(FWPKM_NUM_TIMED), "") == 0);
  CHECK(fwpkm_checked_build() == 0);

  fwpkm_destroy(h);
  fwpkm_destroy(NULL);
  if (failures == 0) printf("abi host checks ok\n");
  return failures == 0 ? 0 : 1;
}
