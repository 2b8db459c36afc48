/* The library's C ABI used from plain C (no torch, no C++): the host-side
 * entry points that need no device.  Prints one line per check and exits
 * non-zero on the first failure. */
#include <stdio.h>
#include <string.h>

#include "gla.h"

static int fails = 0;
#define CHECK(cond, what)                                        \
  do {                                                           \
    if (!(cond)) {                                               \
      printf("FAIL %s\n", what);                                 \
      fails++;                                                   \
    } else {                                                     \
      printf("ok %s\n", what);                                   \
    }                                                            \
  } while (0)

int main(void) {
  gla_dims d;
  size_t bytes = 1;
  gla_state* pool = NULL;
  d.B = 8; d.T = 2048; d.H = 16; d.dk = 96; d.dv = 192; d.chunk = 128;
  d.in_dtype = GLA_BF16; d.out_dtype = GLA_BF16; d.segments = 0;

  CHECK(strcmp(gla_status_str(GLA_OK), "GLA_OK") == 0, "status string");
  CHECK(gla_workspace_size(GLA_OP_FWD, &d, &bytes) == GLA_OK && bytes == 0,
        "forward workspace of the training shape is empty (one walk per CU)");
  d.B = 1; d.T = 65536;
  CHECK(gla_workspace_size(GLA_OP_FWD, &d, &bytes) == GLA_OK && bytes > 0,
        "long context needs segment-state workspace");
  d.segments = 4;
  CHECK(gla_workspace_size(GLA_OP_FWD, &d, &bytes) == GLA_OK && bytes > 0,
        "a caller's segment count needs segment-state workspace");
  d.segments = -1;
  CHECK(gla_workspace_size(GLA_OP_FWD, &d, &bytes) == GLA_ERR_INVALID_ARGUMENT, "negative segments are rejected");
  d.segments = 0;
  d.dk = 64;
  CHECK(gla_workspace_size(GLA_OP_FWD, &d, &bytes) == GLA_ERR_UNSUPPORTED, "dk = 64 is unsupported");
  CHECK(strlen(gla_last_error()) > 0, "the failure leaves a message");
  CHECK(gla_state_alloc_q16(0, 16, 96, 192, NULL, &pool) == GLA_ERR_INVALID_ARGUMENT && pool == NULL,
        "a pool of no slots is rejected");
  CHECK(gla_state_format(NULL) == -1, "format of no pool");
  CHECK(gla_state_slot_bytes(16, 96, 192) == 1179648u, "float32 slot bytes");
  CHECK(gla_state_free(NULL) == GLA_OK, "freeing no pool");
  return fails != 0;
}
