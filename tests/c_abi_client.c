/*
 * c_abi_client.c — a plain C99 client of include/decode_attn.h: it plans both layer kinds of the
 * 32K-context workload and checks the host-side validation, with no device work (num_cus is given,
 * so no device is queried and nothing is launched). Built and run by tests/test_c_client.py.
 */
#include <stdio.h>
#include <string.h>

#include "decode_attn.h"

static int failures = 0;

#define CHECK(cond)                                             \
  do {                                                          \
    if (!(cond)) {                                              \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                               \
    }                                                           \
  } while (0)

static decode_attn_problem long_ctx_problem(int32_t kv_heads, int32_t head_dim, int32_t window) {
  decode_attn_problem p;
  memset(&p, 0, sizeof p);
  p.batch = 4;
  p.num_q_heads = 16;
  p.num_kv_heads = kv_heads;
  p.head_dim = head_dim;
  p.page_size = 16;
  p.max_pages_per_seq = 2112;
  p.num_pages = 16896;
  p.max_ctx_len = 33792;
  p.window = window;
  p.num_cus = 256;
  return p;
}

int main(void) {
  decode_attn_plan_t plan;
  decode_attn_problem p = long_ctx_problem(2, 512, 0);

  CHECK(decode_attn_version() == DECODE_ATTN_VERSION);
  CHECK(decode_attn_plan(&p, &plan) == DECODE_ATTN_OK);
  CHECK(plan.kind == 1);
  CHECK(plan.group_size == 8);
  CHECK(plan.num_splits >= 16 && plan.num_splits <= 64);
  CHECK(plan.workspace_bytes >= (uint64_t)4 * 16 * plan.num_splits * (512 + 1) * 4);
  CHECK(plan.partial_lse_offset % 256 == 0);
  const int global_splits = plan.num_splits;

  p = long_ctx_problem(8, 256, 1024);
  CHECK(decode_attn_plan(&p, &plan) == DECODE_ATTN_OK);
  CHECK(plan.kind == 2);
  CHECK(plan.group_size == 2);

  /* Host-side rejections: nothing is launched. */
  p = long_ctx_problem(3, 512, 0); /* 16 % 3 != 0 */
  CHECK(decode_attn_plan(&p, &plan) == DECODE_ATTN_ERR_SHAPE);
  p = long_ctx_problem(2, 384, 0); /* no kernel for head_dim 384 */
  CHECK(decode_attn_plan(&p, &plan) == DECODE_ATTN_ERR_UNSUPPORTED);
  CHECK(decode_attn_plan(NULL, &plan) == DECODE_ATTN_ERR_NULL);
  p = long_ctx_problem(2, 512, 0);
  CHECK(decode_attn_plan(&p, &plan) == DECODE_ATTN_OK);
  CHECK(decode_attn_global(&plan, NULL, NULL, NULL, NULL, NULL, 1, 0.04f, NULL, NULL, NULL, 0,
                           NULL) == DECODE_ATTN_ERR_NULL);
  CHECK(decode_attn_global(&plan, NULL, NULL, NULL, NULL, NULL, 0, 0.04f, NULL, NULL, NULL, 0,
                           NULL) == DECODE_ATTN_OK); /* batch 0: nothing to do */
  CHECK(decode_attn_rope_cache(NULL, 16, 64, 0, 1e4, NULL) == DECODE_ATTN_ERR_NULL);
  CHECK(strncmp(decode_attn_status_str(DECODE_ATTN_ERR_ALIGN), "DECODE_ATTN_ERR_ALIGN", 21) == 0);

  if (failures == 0)
    printf("c client ok: global layer %d splits, workspace %llu bytes\n", global_splits,
           (unsigned long long)plan.workspace_bytes);
  return failures == 0 ? 0 : 1;
}
