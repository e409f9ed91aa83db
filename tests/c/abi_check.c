/* The C ABI used from plain C: include/carve.h compiles as C99 and the library links and
 * answers its host-side calls (sizes, status strings, argument checks) without a GPU.
 * No call here reaches a kernel: every checked call is rejected before any launch. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "carve.h"

static int failures = 0;
#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                    \
    }                                                                \
  } while (0)

int main(void) {
  /* a 16-byte aligned placeholder address: never dereferenced by a rejected call */
  void* fake = (void*)(uintptr_t)0x100000;
  carve_shape s;
  s.B = 2; s.H = 4; s.T = 300; s.Dk = 128; s.Dv = 128; s.L = 64; s.dtype = CARVE_BF16;

  CHECK(carve_abi_version() == CARVE_ABI_VERSION);
  CHECK(strcmp(carve_status_string(CARVE_OK), "CARVE_OK") == 0);
  CHECK(strncmp(carve_status_string(CARVE_ERR_WORKSPACE), "CARVE_", 6) == 0);

  size_t fwd = carve_fwd_workspace_size(&s, NULL);
  size_t bwd = carve_bwd_workspace_size(&s);
  size_t saved = carve_saved_size(&s);
  CHECK(fwd > 0 && bwd > fwd && saved > 0 && carve_bwd_saved_workspace_size(&s) > 0);

  /* argument checks before any launch */
  CHECK(carve_fwd(&s, fake, fake, fake, (const float*)fake, NULL, (const float*)fake, NULL, NULL, fake, NULL,
                  fake, fwd - 1, NULL) == CARVE_ERR_WORKSPACE);
  CHECK(carve_fwd(&s, NULL, fake, fake, (const float*)fake, NULL, (const float*)fake, NULL, NULL, fake, NULL,
                  fake, fwd, NULL) == CARVE_ERR_INVALID_ARG);
  carve_shape bad = s;
  bad.Dk = 96;
  CHECK(carve_fwd_workspace_size(&bad, NULL) == 0);
  CHECK(carve_fwd(&bad, fake, fake, fake, (const float*)fake, NULL, (const float*)fake, NULL, NULL, fake, NULL,
                  fake, (size_t)1 << 40, NULL) == CARVE_ERR_UNSUPPORTED);
  CHECK(carve_bwd(&s, fake, fake, fake, (const float*)fake, (const float*)fake, (const float*)fake, NULL, fake,
                  NULL, fake, fake, fake, (float*)fake, NULL, (float*)fake, NULL, fake, bwd, NULL) ==
        CARVE_ERR_INVALID_ARG);   /* b given without db */

  /* unequal key and value widths size their padded operands */
  carve_shape un = s;
  un.Dk = 64;
  CHECK(carve_fwd_workspace_size(&un, NULL) > fwd);

  /* an empty problem needs no workspace and launches nothing */
  carve_shape empty = s;
  empty.T = 0;
  CHECK(carve_fwd_workspace_size(&empty, NULL) == 0);
  CHECK(carve_fwd(&empty, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == CARVE_OK);

  if (failures) return 1;
  printf("carve C ABI: ok (fwd workspace %zu bytes, bwd %zu, saved %zu)\n", fwd, bwd, saved);
  return 0;
}
