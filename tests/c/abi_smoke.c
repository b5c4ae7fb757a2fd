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
  expect(pmoe_moe_workspace_bytes(16, 2, 4, 256, 128, PMOE_ACT_RELU2) > 0 && pmoe_last_error()[0] == 0,
         "a successful call clears the error");
  /* argument errors found before any device work */
  expect(pmoe_weight_bytes(4, 256, 256, 128, NULL) == PMOE_ERR_ARG, "null sizes");
  expect(pmoe_moe_workspace_layout(16, 2, 4, 256, 128, PMOE_ACT_RELU2, NULL) == PMOE_ERR_ARG,
         "null offsets");
  expect(pmoe_moe_workspace_bytes(16, 2, 4, 100, 128, PMOE_ACT_RELU2) == 0, "H not a multiple of 64");
  expect(pmoe_moe_workspace_bytes(16, 2, 4, 32768, 128, PMOE_ACT_RELU2) == 0, "H too long");
  expect(pmoe_moe_workspace_bytes(16, 2, 2000, 256, 128, PMOE_ACT_RELU2) == 0, "E too large");
  expect(pmoe_finalize(NULL, NULL, NULL, 4, 2, 60, NULL, NULL) == PMOE_ERR_SHAPE, "finalize H");
  expect(pmoe_router_topk(NULL, 0, 64, 6, 0, NULL, NULL, NULL) == PMOE_OK, "router T = 0");
  expect(pmoe_router_topk(NULL, 4, 64, 0, 0, NULL, NULL, NULL) == PMOE_ERR_SHAPE, "router K = 0");
  {
    pmoe_moe_options o;
    float a1 = 1.0f;
    memset(&o, 0, sizeof o);
    o.recipe = 3;
    expect(pmoe_routed_moe_ex(NULL, NULL, NULL, NULL, 0, NULL, 8, 2, 4, 256, 128, 256, 0, NULL, NULL,
                              NULL, NULL, NULL, NULL, PMOE_ACT_SWIGLU, &o, NULL, 0, NULL, NULL) ==
               PMOE_ERR_ARG,
           "unknown recipe");
    o.recipe = PMOE_RECIPE_PER_TOKEN;
    o.a1_scale = &a1;
    expect(pmoe_moe_forward(NULL, NULL, 0, NULL, 8, 2, 4, 256, 128, 256, 0, NULL, NULL, NULL, NULL,
                            NULL, NULL, PMOE_ACT_SWIGLU, &o, NULL, 0, NULL, NULL) == PMOE_ERR_ARG,
           "a1 scale with the per-token recipe");
  }
  printf(failures ? "abi_smoke: %d failures\n" : "abi_smoke: ok\n", failures);
  return failures != 0;
}
