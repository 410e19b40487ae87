// Host-side checks of libmoe under AddressSanitizer, with no GPU: every call here
// is answered by the library's host code (configuration checks, sizes, argument
// checks) before anything would be launched.  Prints "ok" and exits 0 when every
// expectation holds; AddressSanitizer aborts on a host memory error.
#include <stdio.h>
#include <string.h>

#include "moe.h"

static int failures = 0;
#define EXPECT(cond)                                              \
  do {                                                            \
    if (!(cond)) {                                                \
      fprintf(stderr, "line %d: expected %s\n", __LINE__, #cond); \
      ++failures;                                                 \
    }                                                             \
  } while (0)

static moe_config cfg(int T, int d, int H, int dh, int E, int k, int groups, int tkg, int renorm, int drop,
                      int C, int kn, int kd, int dff, int act, int shared, int latent, int act_dt, int r_dt,
                      int mode) {
  moe_config c;
  memset(&c, 0, sizeof c);
  c.T = T; c.d_model = d; c.n_heads = H; c.d_head = dh; c.n_experts = E; c.top_k = k; c.n_groups = groups;
  c.topk_groups = tkg; c.renorm = renorm; c.drop = drop; c.capacity = C; c.keep_num = kn; c.keep_den = kd;
  c.d_ff = dff; c.act = act; c.n_shared = shared; c.latent_proj = latent; c.residual = 1; c.act_dtype = act_dt;
  c.router_dtype = r_dt; c.route_mode = mode;
  return c;
}

int main() {
  // the five workloads of the benchmark (shapes and rules)
  const moe_config w[5] = {
      cfg(256, 128, 1, 128, 8, 2, 0, 0, 0, MOE_DROP_CAPACITY, 80, 1, 1, 256, MOE_ACT_RELU, 0, 0, MOE_F32, MOE_F32, 0),
      cfg(4096, 4096, 1, 4096, 8, 2, 0, 0, 1, MOE_DROP_NONE, 0, 1, 1, 14336, MOE_ACT_SWIGLU, 0, 0, MOE_BF16, MOE_F32, 0),
      cfg(8192, 2048, 1, 2048, 64, 6, 0, 0, 0, MOE_DROP_CAPACITY, 768, 1, 1, 1408, MOE_ACT_SWIGLU, 2, 0, MOE_BF16,
          MOE_BF16, 0),
      cfg(8192, 5120, 1, 5120, 160, 6, 8, 3, 0, MOE_DROP_AFFINITY, 0, 9, 10, 1536, MOE_ACT_SWIGLU, 2, 0, MOE_BF16,
          MOE_BF16, 0),
      cfg(16384, 2048, 8, 256, 128, 1, 0, 0, 0, MOE_DROP_NONE, 0, 1, 1, 512, MOE_ACT_SWIGLU, 0, 1, MOE_BF16, MOE_BF16,
          0),
  };
  for (int i = 0; i < 5; ++i) {
    EXPECT(moe_check_config(&w[i]) == MOE_OK);
    EXPECT(moe_workspace_bytes(&w[i]) > 0);
    EXPECT(moe_rows_upper_bound(&w[i]) > 0);
    EXPECT(moe_backward_workspace_bytes(&w[i]) > 0);
  }
  // invalid configurations
  moe_config b = w[2];
  b.d_ff = 100;
  EXPECT(moe_check_config(&b) == MOE_ERR_ARG && moe_workspace_bytes(&b) == 0 && moe_rows_upper_bound(&b) == -1);
  b = w[2];
  b.top_k = 0;
  EXPECT(moe_check_config(&b) == MOE_ERR_ARG);
  b = w[2];
  b.n_experts = 3000;
  EXPECT(moe_check_config(&b) != MOE_OK);
  EXPECT(moe_check_config(NULL) == MOE_ERR_ARG);
  for (int s = 0; s >= -4; --s) EXPECT(strncmp(moe_status_str(s), "MOE_", 4) == 0);
  EXPECT(moe_status_str(7) != NULL);
  // argument checks of every entry point (pointers are never dereferenced: each call fails first)
  void *f = (void *)0x1000;
  int32_t *fi = (int32_t *)0x1000;
  float *ff = (float *)0x1000;
  const moe_config *c2 = &w[2], *c3 = &w[3], *c4 = &w[4];
  EXPECT(moe_route(NULL, f, f, NULL, NULL, 0, fi, ff, NULL, f, (size_t)1 << 40, NULL) == MOE_ERR_ARG);
  EXPECT(moe_route(c2, f, f, NULL, NULL, 0, NULL, ff, NULL, f, (size_t)1 << 40, NULL) == MOE_ERR_ARG);
  EXPECT(moe_route(c2, f, f, NULL, NULL, 0, fi, ff, NULL, f, 16, NULL) == MOE_ERR_WORKSPACE);
  EXPECT(moe_route(c4, f, f, NULL, NULL, 0, fi, ff, ff, f, (size_t)1 << 40, NULL) == MOE_ERR_UNSUPPORTED);
  EXPECT(moe_route_ex(c2, f, f, NULL, NULL, NULL, 5, fi, ff, NULL, NULL, f, (size_t)1 << 40, NULL) == MOE_ERR_ARG);
  EXPECT(moe_dispatch(c3, fi, NULL, f, fi, fi, fi, fi, fi, f, f, (size_t)1 << 40, NULL) == MOE_ERR_ARG);
  EXPECT(moe_dispatch_noalloc(c3, fi, NULL, f, fi, fi, fi, fi, fi, NULL, NULL) == MOE_ERR_ARG);
  EXPECT(moe_check_topk(c2, fi, NULL, NULL) == MOE_ERR_ARG);
  EXPECT(moe_expert_ffn(c2, f, fi, f, NULL, f, f, f, f, f, f, f, f, (size_t)1 << 40, NULL) == MOE_ERR_ARG);
  EXPECT(moe_expert_ffn_gather(c2, f, fi, fi, f, NULL, f, f, f, f, f, f, f, f, (size_t)1 << 40, NULL) ==
         MOE_ERR_ARG);
  EXPECT(moe_combine(c2, f, NULL, ff, f, f, f, NULL) == MOE_ERR_ARG);
  EXPECT(moe_layer_fwd(c2, NULL, f, f, NULL, f, (size_t)1 << 40, NULL) == MOE_ERR_ARG);
  EXPECT(moe_sel_bias_update(c2, NULL, ff, 0.001f, NULL) == MOE_ERR_ARG);
  EXPECT(moe_transpose_weights(c2, NULL, NULL, NULL) == MOE_ERR_ARG);
  EXPECT(moe_layer_bwd(c2, NULL, NULL, f, f, 0.f, 0.f, NULL, NULL, f, (size_t)1 << 40, NULL) == MOE_ERR_ARG);
  if (failures) return 1;
  printf("ok\n");
  return 0;
}
