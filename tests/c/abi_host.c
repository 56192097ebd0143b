/* A plain C11 program against include/rpkv.h: capability query, plan creation,
 * host planning of a small mixed batch, the plan summary and item lists, and
 * error reporting.  Host-only calls, so it runs without a GPU.  Prints one
 * "key value" pair per line for the test to check. */
#include <stdio.h>
#include <string.h>

#include "rpkv.h"

int main(void) {
  rpkv_shape s;
  memset(&s, 0, sizeof s);
  s.num_q_heads = 32;
  s.num_kv_heads = 8;
  s.head_dim = 128;
  s.page_size = 16;
  s.dtype = RPKV_BF16;
  s.max_batch = 4;
  s.num_pages = 256;
  s.max_tokens = 1024;
  s.max_pages_per_req = 64;
  printf("supports %d\n", (int)rpkv_supports(&s));

  rpkv_shape bad = s;
  bad.head_dim = 96;
  rpkv_status st = rpkv_supports(&bad);
  printf("supports_bad %d %s\n", (int)st, rpkv_status_string(st));

  rpkv_plan *plan = NULL;
  if (rpkv_plan_create(&s, &plan) != RPKV_OK) return 1;
  /* a 300-token prefill, a chunked prefill of 40 over 200 cached, two decodes */
  const int32_t cu[5] = {0, 300, 340, 341, 342};
  const int32_t L[4] = {300, 240, 777, 1000};
  st = rpkv_plan_batch(plan, 4, cu, L, 64, NULL, NULL, 0);
  printf("plan %d\n", (int)st);
  rpkv_plan_info info;
  if (rpkv_plan_get_info(plan, &info) != RPKV_OK) return 1;
  printf("tokens %d\n", info.num_tokens);
  printf("max_seqlen_k %d\n", info.max_seqlen_k);
  printf("prefill_items %d\n", info.num_prefill_items);
  printf("decode_items %d\n", info.num_decode_items);
  int32_t last[4];
  if (rpkv_last_indices(plan, last) != RPKV_OK) return 1;
  printf("last %d %d %d %d\n", last[0], last[1], last[2], last[3]);
  int32_t count = 0;
  rpkv_plan_get_items(plan, 1, NULL, 0, &count);
  printf("decode_list %d\n", count);
  printf("tiles_per_block %d\n", info.tiles_per_block);

  /* the same batch with the MFMA tiles forced into ping-pong pairs: the field
   * after prefix_detect_keys reaches the planner and the summary reports it */
  rpkv_shape sp = s;
  sp.tiles_per_block = 2;
  rpkv_plan *pair_plan = NULL;
  if (rpkv_plan_create(&sp, &pair_plan) != RPKV_OK) return 1;
  if (rpkv_plan_batch(pair_plan, 4, cu, L, 64, NULL, NULL, 0) != RPKV_OK) return 1;
  rpkv_plan_info pinfo;
  if (rpkv_plan_get_info(pair_plan, &pinfo) != RPKV_OK) return 1;
  int32_t npre = 0;
  rpkv_plan_get_items(pair_plan, 0, NULL, 0, &npre);
  printf("pairs %d %d %d\n", pinfo.tiles_per_block, pinfo.num_prefill_items, npre % 16);
  rpkv_plan_destroy(pair_plan);
  sp.tiles_per_block = 3;
  st = rpkv_supports(&sp);
  printf("tpb_bad %d\n", (int)st);

  /* a request with more new tokens than KV length is rejected with a message */
  const int32_t Lbad[4] = {300, 20, 777, 1000};
  st = rpkv_plan_batch(plan, 4, cu, Lbad, 64, NULL, NULL, 0);
  printf("plan_bad %d %s\n", (int)st, rpkv_last_error()[0] ? "msg" : "nomsg");
  rpkv_plan_destroy(plan);
  printf("done\n");
  return 0;
}
