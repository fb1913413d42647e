/* Host-only use of the C ABI from C: compiled against include/vsa.h and
 * linked to libvsa.so by tests/test_c_abi.py.  Prints struct layouts and
 * the sizing answers of the query entry points for the Wan2.1-1.3B shape,
 * one "key value" pair per line.  No device is touched. */
#include <stddef.h>
#include <stdio.h>

#include "vsa.h"

int main(void) {
  vsa_shape s = {1, 12, 128, 21, 30, 52, 4, 4, 8, VSA_BF16};
  float density = 0.2f;
  int64_t rl = 0, cap = 0;
  size_t pws = 0, aws = 0;
  printf("sizeof_shape %zu\n", sizeof(vsa_shape));
  printf("sizeof_index %zu\n", sizeof(vsa_index));
  printf("offsetof_index_row_ptr %zu\n", offsetof(vsa_index, row_ptr));
  printf("offsetof_index_capacity %zu\n", offsetof(vsa_index, capacity));
  printf("offsetof_index_equal_heads %zu\n", offsetof(vsa_index, equal_heads));
  printf("sizeof_select %zu\n", sizeof(vsa_select));
  printf("offsetof_select_value %zu\n", offsetof(vsa_select, value));
  printf("offsetof_select_estimator %zu\n", offsetof(vsa_select, estimator));
  printf("sizeof_head_option %zu\n", sizeof(vsa_head_option));

  vsa_status st = vsa_query(&s, &density, 1, -1, &rl, &cap, &pws, &aws);
  printf("query %d %lld %lld %zu %zu\n", (int)st, (long long)rl, (long long)cap, pws, aws);

  float p = 0.25f;
  vsa_select sel = {VSA_TOPP, 1, &p, -1, 2, 0.0f, VSA_EST_DSA};
  st = vsa_query_select(&s, &sel, &rl, &cap, &pws);
  printf("query_select %d %lld %lld %zu\n", (int)st, (long long)rl, (long long)cap, pws);

  vsa_head_option opts[12];
  for (int h = 0; h < 12; ++h) {
    opts[h].kind = h % 3;
    opts[h].value = 0.2f;
    opts[h].window_t = (h % 4) - 1;
  }
  st = vsa_query_mixed(&s, opts, VSA_EST_MEAN, &rl, &cap, &pws);
  printf("query_mixed %d %lld %lld %zu\n", (int)st, (long long)rl, (long long)cap, pws);

  int32_t cands[6] = {4, 4, 8, 1, 8, 16};
  size_t sws = 0;
  st = vsa_scheme_workspace(&s, cands, 2, &sws);
  printf("scheme_workspace %d %zu\n", (int)st, sws);

  size_t mws = 0, moff[4] = {0, 0, 0, 0};
  st = vsa_scheme_means_workspace(&s, cands, 2, &mws, moff);
  printf("scheme_means_workspace %d %zu %zu %zu %zu %zu\n", (int)st, mws, moff[0], moff[1], moff[2], moff[3]);
  printf("noalloc_max_ws %zu\n", (size_t)VSA_PLAN_NOALLOC_MAX_WS);
  printf("calib_limits %zu %d %d\n", (size_t)VSA_CALIB_POOL_BYTES, VSA_CALIB_MAX_WORKGROUPS, VSA_CALIB_MAX_ITERS);

  /* error paths: each fails a host check before anything is enqueued */
  printf("bad_density %d\n", (int)vsa_query(&s, &density, 2, -1, NULL, NULL, NULL, NULL));
  vsa_index idx = {s, 0, 0, NULL, NULL, 0, 0};
  int32_t heads[2] = {0, 0};
  printf("plan_heads_no_list %d\n", (int)vsa_plan_heads(NULL, NULL, NULL, NULL, &s, NULL, 1, &density, 1, -1,
                                                        &idx, NULL, 0, NULL));
  printf("plan_heads_repeated %d\n", (int)vsa_plan_heads(NULL, NULL, NULL, NULL, &s, heads, 2, &density, 1, -1,
                                                         &idx, NULL, 0, NULL));
  printf("attn_heads_null %d\n", (int)vsa_attn_heads(NULL, NULL, NULL, &idx, heads, 12, 0.0f, NULL, NULL, 0, NULL));
  printf("plan_noalloc_null %d\n", (int)vsa_plan_noalloc(NULL, NULL, &s, &density, 1, -1, &idx, NULL));
  printf("calib_null %d\n", (int)vsa_calib_mfma_bf16(NULL, VSA_CALIB_POOL_BYTES, NULL, 1, 1, NULL));
  printf("status_str %s\n", vsa_status_str(VSA_ERR_CAPACITY));
  return 0;
}
