/* A plain C11 client of libsinkattn.so: includes only include/sink_attn.h
 * and calls the host-side entry points (no GPU). It builds the tile
 * schedule of a small packed problem with the two-call protocol and prints
 * the sizes and every table word, then the status of a call the library
 * must refuse. tests/test_c_client.py compiles it with gcc, runs it and
 * compares the output with the same calls made through the Python
 * binding. */
#include <stdio.h>
#include <stdlib.h>

#include "sink_attn.h"

int main(void) {
  /* three sequences (5, 130 and 64 query rows against 5, 200 and 64 keys),
   * 8 q-heads over 2 kv-heads, head_dim 128, causal, bf16 */
  const int32_t cu_q[4] = {0, 5, 135, 199};
  const int32_t cu_k[4] = {0, 5, 205, 269};
  sink_attn_problem p = {0};
  p.batch = 3;
  p.num_heads_q = 8;
  p.num_heads_k = 2;
  p.head_dim = 128;
  p.total_q = 199;
  p.total_k = 269;
  p.max_seqlen_q = 130;
  p.max_seqlen_k = 200;
  p.causal = 1;
  p.win_left = -1;
  p.win_right = -1;
  p.dtype = SINK_ATTN_BF16;
  p.layout_q = SINK_ATTN_TND;
  p.layout_out = SINK_ATTN_TND;

  int64_t words = 0, fws = 0, bws = 0;
  sink_attn_status st = sink_attn_metadata(&p, cu_q, cu_k, NULL, 0, &words, &fws, &bws);
  if (st != SINK_ATTN_OK || words <= 0) {
    fprintf(stderr, "size query: %s\n", sink_attn_status_string(st));
    return 1;
  }
  int32_t* meta = (int32_t*)malloc((size_t)words * sizeof(int32_t));
  if (!meta) return 1;
  int64_t words2 = 0;
  st = sink_attn_metadata(&p, cu_q, cu_k, meta, words, &words2, &fws, &bws);
  if (st != SINK_ATTN_OK || words2 != words) {
    fprintf(stderr, "table: %s\n", sink_attn_status_string(st));
    free(meta);
    return 1;
  }
  printf("abi %d\n", sink_attn_abi_version());
  printf("sizes %lld %lld %lld\n", (long long)words, (long long)fws, (long long)bws);
  printf("table");
  for (int64_t i = 0; i < words; ++i) printf(" %d", (int)meta[i]);
  printf("\n");

  /* 8 q-heads over 3 kv-heads: not a GQA grouping, refused */
  p.num_heads_k = 3;
  st = sink_attn_metadata(&p, cu_q, cu_k, NULL, 0, &words, &fws, &bws);
  printf("refused %d %s\n", (int)st, sink_attn_status_string(st));
  free(meta);
  return 0;
}
