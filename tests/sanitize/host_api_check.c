/* Sanitizer driver for the host code of libeqlinear, in C as a C caller of
 * the ABI would be (built with AddressSanitizer and UndefinedBehaviorSanitizer
 * on the host side): every plan kind is created and destroyed, workspace
 * sizes are queried over a range of shapes, and every call is made with
 * invalid arguments (out-of-range enumeration values included, which C
 * callers may pass), checking the documented status codes.  No call needs a
 * GPU: validation returns before the first HIP call, and calls that reach the
 * HIP runtime on a host without one report EQL_ERR_HIP or EQL_ERR_ALLOC.
 * Prints "ok" and exits 0 on success. */
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>

#include "eqconv.h"
#include "eqlinear.h"

static int failures = 0;
#define CHECK(cond)                                                             \
  do {                                                                          \
    if (!(cond)) {                                                              \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond);  \
      ++failures;                                                               \
    }                                                                           \
  } while (0)

int main(void) {
  void* a16 = (void*)(uintptr_t)(1 << 20);         /* aligned, never dereferenced */
  void* mis = (void*)((uintptr_t)(1 << 20) + 8);   /* misaligned */
  const int64_t widths[] = {1, 2, 7, 16, 33, 96, 130, 384, 1000, 65536};
  const int64_t rows[] = {0, 1, 12608, (int64_t)1 << 30};
  const size_t nw = sizeof(widths) / sizeof(widths[0]);
  for (int dt = 0; dt < 2; ++dt) {
    for (size_t ic = 0; ic < nw; ++ic) {
      for (size_t id = 0; id < nw; ++id) {
        const int64_t C = widths[ic], D = widths[id];
        for (int g = 0; g < 2; ++g) {
          const int64_t hi = g == 0 ? 16 : 8;
          for (int64_t n = 2; n <= hi; n += 3) {
            eqlinear_plan_t p = NULL;
            const eqlinear_status_t st = eqlinear_plan_create_group(C, D, g, n, dt, &p);
            CHECK(st == EQL_OK && p != NULL);
            if (st != EQL_OK) continue;
            for (size_t ir = 0; ir < 4; ++ir) {
              const size_t ws = eqlinear_backward_weight_workspace(p, rows[ir]);
              CHECK(rows[ir] > 0 || ws == 0);
            }
            int64_t s = -1, d = -1;
            CHECK(eqlinear_mac_counts(p, 12608, &s, &d) == EQL_OK && s > 0 && d >= s);
            CHECK(eqlinear_forward(p, a16, a16, 4, NULL) == EQL_ERR_NO_WEIGHT);
            CHECK(eqlinear_backward_input(p, a16, a16, 4, NULL) == EQL_ERR_NO_WEIGHT);
            CHECK(eqlinear_forward(p, a16, a16, -1, NULL) == EQL_ERR_INVALID_ARG);
            CHECK(eqlinear_forward_act(p, a16, a16, 4, 9, NULL) == EQL_ERR_INVALID_ARG);
            CHECK(eqlinear_forward_act(p, a16, a16, 4, -1, NULL) == EQL_ERR_INVALID_ARG);
            CHECK(eqlinear_backward_weight(p, a16, a16, NULL, NULL, 4, a16, 1 << 20, NULL) ==
                  EQL_ERR_INVALID_ARG);
            CHECK(eqlinear_backward_weight(p, mis, a16, (float*)a16, NULL, 4, a16, 1 << 20, NULL) ==
                  EQL_ERR_MISALIGNED);
            CHECK(eqlinear_backward_weight(p, a16, a16, (float*)a16, NULL, -5, a16, 1 << 20, NULL) ==
                  EQL_ERR_INVALID_ARG);
            CHECK(eqlinear_backward_weight_noalloc(p, a16, mis, (float*)a16, NULL, 4, NULL) ==
                  EQL_ERR_MISALIGNED);
            CHECK(eqlinear_set_weight(p, NULL, NULL, NULL) == EQL_ERR_INVALID_ARG);
            CHECK(eqlinear_set_weight(p, mis, NULL, NULL) == EQL_ERR_MISALIGNED);
            CHECK(eqlinear_plan_destroy(p) == EQL_OK);
          }
        }
      }
    }
  }
  /* unsupported groups, orders, dtypes and widths */
  eqlinear_plan_t p = NULL;
  CHECK(eqlinear_plan_create(8, 8, 17, EQL_F32, &p) == EQL_ERR_UNSUPPORTED && p == NULL);
  CHECK(eqlinear_plan_create(8, 8, 1, EQL_F32, &p) == EQL_ERR_UNSUPPORTED);
  CHECK(eqlinear_plan_create(0, 8, 4, EQL_F32, &p) == EQL_ERR_INVALID_ARG);
  CHECK(eqlinear_plan_create(8, (int64_t)1 << 40, 4, EQL_F32, &p) == EQL_ERR_INVALID_ARG);
  CHECK(eqlinear_plan_create(8, 8, 4, 5, &p) == EQL_ERR_UNSUPPORTED);
  CHECK(eqlinear_plan_create(8, 8, 4, -3, &p) == EQL_ERR_UNSUPPORTED);
  CHECK(eqlinear_plan_create_group(8, 8, 7, 4, EQL_F32, &p) == EQL_ERR_UNSUPPORTED);
  CHECK(eqlinear_plan_create(8, 8, 4, EQL_F32, NULL) == EQL_ERR_INVALID_ARG);
  CHECK(eqlinear_plan_destroy(NULL) == EQL_OK);
  CHECK(eqlinear_backward_weight_workspace(NULL, 4) == 0);
  CHECK(eqlinear_forward(NULL, a16, a16, 4, NULL) == EQL_ERR_INVALID_ARG);
  for (int st = -1; st <= 9; ++st) CHECK(eqlinear_status_string(st) != NULL);
  CHECK(eqlinear_last_error() != NULL);
  /* a call that reaches the HIP runtime: without a GPU it reports an error */
  CHECK(eqlinear_plan_create(96, 384, 4, EQL_F16, &p) == EQL_OK);
  const eqlinear_status_t sw = eqlinear_set_weight(p, a16, NULL, NULL);
  CHECK(sw == EQL_ERR_HIP || sw == EQL_ERR_ALLOC || sw == EQL_OK);
  CHECK(eqlinear_plan_destroy(p) == EQL_OK);
  CHECK(eqlinear_plan_create(2048, 2048, 4, EQL_F16, &p) == EQL_OK);
  CHECK(eqlinear_backward_weight_noalloc(p, a16, a16, (float*)a16, NULL, (int64_t)1 << 16, NULL) ==
        EQL_ERR_WORKSPACE);
  CHECK(eqlinear_plan_destroy(p) == EQL_OK);
  /* group convolution plans */
  const int64_t ks[] = {1, 3, 5, 7}, cs[] = {4, 8, 48}, pix[] = {0, 2, 64};
  for (int dt = 0; dt < 2; ++dt) {
    for (int ik = 0; ik < 4; ++ik) {
      for (int icc = 0; icc < 3; ++icc) {
        eqconv_plan_t cp = NULL;
        CHECK(eqconv_plan_create(cs[icc], 12, ks[ik], dt, &cp) == EQL_OK);
        if (cp == NULL) continue;
        for (int ip = 0; ip < 3; ++ip) (void)eqconv_backward_weight_workspace(cp, pix[ip], 56, 56);
        int64_t s = 0, d = 0;
        CHECK(eqconv_mac_counts(cp, 2, 8, 8, &s, &d) == EQL_OK && d > s);
        CHECK(eqconv_forward(cp, a16, a16, 2, 8, 8, EQL_ACT_NONE, NULL) == EQL_ERR_NO_WEIGHT);
        CHECK(eqconv_forward(cp, a16, a16, 2, 8, 8, 11, NULL) == EQL_ERR_INVALID_ARG);
        CHECK(eqconv_forward(cp, a16, a16, -2, 8, 8, EQL_ACT_NONE, NULL) == EQL_ERR_INVALID_ARG);
        CHECK(eqconv_plan_destroy(cp) == EQL_OK);
      }
    }
    eqconv_plan_t cp = NULL;
    CHECK(eqconv_plan_create(8, 12, 2, dt, &cp) == EQL_ERR_UNSUPPORTED);
    CHECK(eqconv_plan_create(8, 12, 9, dt, &cp) == EQL_ERR_UNSUPPORTED);
    CHECK(eqconv_plan_create(6, 12, 3, dt, &cp) == EQL_ERR_UNSUPPORTED);
    CHECK(eqconv_plan_create(8, 12, 3, 4, &cp) == EQL_ERR_UNSUPPORTED);
  }
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
