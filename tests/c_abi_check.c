/* A plain C caller of libattn.so (no Python, no HIP headers): the header must
 * compile as C99 with every warning enabled, and the host-only calls and the
 * argument checks must work without a GPU.  Built and run by
 * tests/test_abi.py::test_plain_c_caller. */
#include <stdio.h>
#include <string.h>

#include "attn.h"

static int fails = 0;

static void expect(int ok, const char* what) {
  if (!ok) {
    printf("FAIL %s\n", what);
    ++fails;
  }
}

int main(void) {
  int n = attn_variant_count();
  expect(n > 0, "variant count");
  for (int i = 0; i < n; ++i) {
    int id, hd, dt, bm, bn, waves, stages, ks, se;
    expect(attn_variant_info(i, &id, &hd, &dt, &bm, &bn, &waves, &stages, &ks, &se) == ATTN_OK,
           "variant info");
    expect(id > 0 && (hd == 64 || hd == 128) && (dt == ATTN_F16 || dt == ATTN_BF16), "variant fields");
    expect(bm > 0 && bn > 0 && waves > 0 && stages > 0 && (ks == 0 || ks == 1) && se >= 0,
           "variant tile");
  }
  expect(attn_variant_info(n, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL) != ATTN_OK,
         "variant index past the end");

  /* Argument checks happen before anything touches a device. */
  char q[64], k[64], v[64], o[64];
  expect(attn_fwd(q, k, v, o, NULL, 1, 1, 16, 64, 0.125f, 7, NULL) == ATTN_ERR_DTYPE, "bad dtype");
  expect(attn_fwd(q, k, v, o, NULL, 1, 1, 16, 96, 0.125f, ATTN_BF16, NULL) == ATTN_ERR_SHAPE, "bad D");
  expect(attn_fwd(q, k, v, o, NULL, -1, 1, 16, 64, 0.125f, ATTN_BF16, NULL) == ATTN_ERR_SHAPE, "bad B");
  expect(strlen(attn_last_error()) > 0, "last error text");
  expect(strlen(attn_strerror(ATTN_ERR_SHAPE)) > 0, "strerror");
  attn_fwd_options_t opts;
  memset(&opts, 0, sizeof(opts));
  opts.rescale_threshold = 16.0f;
  expect(attn_fwd_ex(q, k, v, o, NULL, 1, 1, 16, 64, 0.125f, ATTN_F16, NULL, &opts) == ATTN_ERR_ARG,
         "fp16 threshold above 15");
  expect(attn_fwd_split_workspace_size(1, 1, 4096, 64, 4) > 0, "workspace size");
  expect(attn_fwd_split_workspace_size(1, 1, 4096, 96, 4) == 0, "workspace size of a bad D");
  printf("%s\n", fails ? "c abi check failed" : "c abi check ok");
  return fails ? 1 : 0;
}
