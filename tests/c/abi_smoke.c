/* A plain C99 caller of the library: host-only entry points and argument
 * checks that return before any device work, so it runs without a GPU. */
#include <stdio.h>
#include <string.h>

#include "pmoe.h"

static int failures = 0;

static void expect(int cond, const char* what) {
  if (!cond) {
    printf("FAIL %s (last error: %s)\n", what, pmoe_last_error());
    ++failures;
  }
}

int main(void) {
  size_t sizes[4];
  size_t offs[PMOE_WS_NUM_FIELDS];
  expect(pmoe_version() > 0, "version");
  expect(pmoe_weight_bytes(4, 256, 256, 128, sizes) == PMOE_OK, "weight_bytes swiglu");
  expect(sizes[0] == (size_t)4 * 256 * 256 / 2, "FC1 code bytes");
  expect(pmoe_weight_bytes(4, 200, 256, 128, sizes) == PMOE_ERR_SHAPE, "N1 neither I nor 2I");
  expect(pmoe_moe_workspace_bytes(16, 2, 4, 256, 128, PMOE_ACT_RELU2) > 0, "workspace bytes");
  expect(pmoe_moe_workspace_bytes(16, 5, 4, 256, 128, PMOE_ACT_RELU2) == 0, "K > E");
  expect(pmoe_moe_workspace_layout(16, 2, 4, 256, 128, PMOE_ACT_RELU2, offs) == PMOE_OK, "layout");
  expect(offs[PMOE_WS_ROW_OF_ROUTE] == 0 && offs[PMOE_WS_Z] > offs[PMOE_WS_H], "layout order");
  /* T == 0 is a no-op that touches nothing */
  expect(pmoe_quantize_input_per_token(NULL, 0, 256, NULL, NULL, NULL, NULL) == PMOE_OK, "T = 0");
  expect(pmoe_quantize_input_per_token(NULL, 4, 100, NULL, NULL, NULL, NULL) == PMOE_ERR_SHAPE,
         "H not a multiple of 16");
  expect(strlen(pmoe_last_error()) > 0, "error message");
  printf(failures ? "abi_smoke: %d failures\n" : "abi_smoke: ok\n", failures);
  return failures != 0;
}
