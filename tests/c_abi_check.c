/* The library boundary used from plain C: compiled by a C compiler against
 * include/dsa.h alone and linked to libdsa.so. Only calls that return before
 * any device work are made (argument checks, workspace sizes, empty work), so
 * no GPU is needed. Exit status 0 when every check holds. */
#include <stdio.h>

#include "dsa.h"

static int fails = 0;
#define CHECK(cond)                           \
  do {                                        \
    if (!(cond)) {                            \
      printf("FAIL line %d: %s\n", __LINE__, #cond); \
      ++fails;                                \
    }                                         \
  } while (0)

int main(void) {
  /* a non-NULL address that is never dereferenced */
  void* const P = (void*)(size_t)16;
  const size_t BIG = (size_t)1 << 40;
  dsa_shape sh = {1, 4, 2, 256, 128, DSA_BF16};

  CHECK(dsa_status_string(DSA_OK) != NULL);
  CHECK(dsa_status_string(DSA_ERR_HIP) != NULL);

  /* argument errors come back before any HIP call */
  CHECK(dsa_vertical_slash_sparse_attention(NULL, P, P, P, &sh, 8, 8, 64, 0.f, NULL, 0, P, BIG, NULL) ==
        DSA_ERR_INVALID_ARG);
  CHECK(dsa_vertical_slash_sparse_attention(P, P, P, P, &sh, 8, 0, 64, 0.f, NULL, 0, P, BIG, NULL) ==
        DSA_ERR_INVALID_ARG);
  dsa_shape gqa = sh;
  gqa.q_heads = 3;
  CHECK(dsa_block_sparse_attention(P, P, P, P, &gqa, 4, 0.f, NULL, 0, P, BIG, NULL) == DSA_ERR_INVALID_ARG);
  dsa_shape odd_dim = sh;
  odd_dim.head_dim = 96;
  CHECK(dsa_block_sparse_attention(P, P, P, P, &odd_dim, 4, 0.f, NULL, 0, P, BIG, NULL) ==
        DSA_ERR_UNSUPPORTED);
  CHECK(dsa_streaming_attention(P, P, P, P, &sh, 1, 0, 0.f, NULL, 0, NULL) == DSA_ERR_INVALID_ARG);
  const int32_t dup[2] = {1, 1};
  CHECK(dsa_streaming_attention(P, P, P, P, &sh, 1, 2, 0.f, dup, 2, NULL) == DSA_ERR_INVALID_ARG);

  /* workspace sizes are host arithmetic; too small a workspace is refused */
  const size_t ws_vs = dsa_vertical_slash_workspace_bytes(&sh, 8, 8, 4);
  CHECK(ws_vs > 0);
  CHECK(dsa_vertical_slash_sparse_attention(P, P, P, P, &sh, 8, 8, 64, 0.f, NULL, 0, P, ws_vs - 1, NULL) ==
        DSA_ERR_WORKSPACE);
  CHECK(dsa_block_sparse_workspace_bytes(&sh, 4, 4) > 0);
  CHECK(dsa_topk_workspace_bytes(4, 1000, 10) == 0); /* one pass: no workspace */

  /* nothing to do: zero batch, or no listed head */
  dsa_shape none = sh;
  none.batch = 0;
  CHECK(dsa_vertical_slash_sparse_attention(P, P, P, P, &none, 8, 8, 64, 0.f, NULL, 0, NULL, 0, NULL) == DSA_OK);
  const int32_t one[1] = {0};
  CHECK(dsa_block_sparse_attention(P, P, P, P, &sh, 4, 0.f, one, 0, NULL, 0, NULL) == DSA_OK);

  /* shapes the checks refuse: no shape, no kv head, a ragged GQA group, a
     negative size, a head slab past 32-bit offsets, an unknown dtype */
  CHECK(dsa_streaming_attention(P, P, P, P, NULL, 1, 2, 0.f, NULL, 0, NULL) == DSA_ERR_INVALID_ARG);
  dsa_shape bad = sh;
  bad.kv_heads = 0;
  CHECK(dsa_streaming_attention(P, P, P, P, &bad, 1, 2, 0.f, NULL, 0, NULL) == DSA_ERR_INVALID_ARG);
  bad = sh;
  bad.seq_len = -1;
  CHECK(dsa_block_sparse_attention(P, P, P, P, &bad, 4, 0.f, NULL, 0, P, BIG, NULL) == DSA_ERR_INVALID_ARG);
  bad = sh;
  bad.seq_len = (int32_t)1 << 23; /* 2^23 rows x 128 dims x 2 bytes = 2^31 */
  CHECK(dsa_vertical_slash_sparse_attention(P, P, P, P, &bad, 8, 8, 64, 0.f, NULL, 0, P, BIG, NULL) ==
        DSA_ERR_UNSUPPORTED);
  bad = sh;
  bad.dtype = 7;
  CHECK(dsa_streaming_attention(P, P, P, P, &bad, 1, 2, 0.f, NULL, 0, NULL) == DSA_ERR_UNSUPPORTED);
  CHECK(dsa_vertical_slash_workspace_bytes(NULL, 8, 8, 4) == 0);

  /* head lists: out of range, negative count, too many heads */
  const int32_t out_of_range[1] = {4};
  CHECK(dsa_streaming_attention(P, P, P, P, &sh, 1, 2, 0.f, out_of_range, 1, NULL) == DSA_ERR_INVALID_ARG);
  CHECK(dsa_streaming_attention(P, P, P, P, &sh, 1, 2, 0.f, one, -1, NULL) == DSA_ERR_INVALID_ARG);

  /* parameters: estimator window, slash count, top-k, window sizes */
  CHECK(dsa_vertical_slash_sparse_attention(P, P, P, P, &sh, 8, 8, 65, 0.f, NULL, 0, P, BIG, NULL) ==
        DSA_ERR_UNSUPPORTED);
  CHECK(dsa_vertical_slash_sparse_attention(P, P, P, P, &sh, -1, 8, 64, 0.f, NULL, 0, P, BIG, NULL) ==
        DSA_ERR_INVALID_ARG);
  CHECK(dsa_block_sparse_attention(P, P, P, P, &sh, 0, 0.f, NULL, 0, P, BIG, NULL) == DSA_ERR_INVALID_ARG);
  CHECK(dsa_streaming_attention(P, P, P, P, &sh, -1, 2, 0.f, NULL, 0, NULL) == DSA_ERR_INVALID_ARG);
  CHECK(dsa_kv_retention(P, P, &sh, 0, 8, 0.f, NULL, 0, P, P, P, BIG, NULL) == DSA_ERR_INVALID_ARG);
  CHECK(dsa_kv_retention(P, P, &sh, 8, -1, 0.f, NULL, 0, P, P, P, BIG, NULL) == DSA_ERR_INVALID_ARG);

  /* mixed layer: unknown pattern, no pattern list */
  const int32_t pats[4] = {DSA_PATTERN_VS, DSA_PATTERN_BS, 9, DSA_PATTERN_NONE};
  CHECK(dsa_mixed_sparse_attention(P, P, P, P, &sh, pats, 8, 8, 64, 4, 1, 2, 0.f, P, BIG, NULL) ==
        DSA_ERR_INVALID_ARG);
  CHECK(dsa_mixed_sparse_attention(P, P, P, P, &sh, NULL, 8, 8, 64, 4, 1, 2, 0.f, P, BIG, NULL) ==
        DSA_ERR_INVALID_ARG);

  /* stage calls */
  int32_t dummy = 0;
  CHECK(dsa_topk((const float*)P, 2, 100, -1, -1, &dummy, P, BIG, NULL) == DSA_ERR_INVALID_ARG);
  CHECK(dsa_topk((const float*)P, 2, 100, 5, 100, &dummy, P, BIG, NULL) == DSA_ERR_INVALID_ARG);
  CHECK(dsa_topk((const float*)P, 2, 100, 5, -2, &dummy, P, BIG, NULL) == DSA_ERR_INVALID_ARG);
  CHECK(dsa_topk(NULL, 2, 100, 5, 0, &dummy, P, BIG, NULL) == DSA_ERR_INVALID_ARG);
  CHECK(dsa_vs_build_index(P, -1, P, 4, 1, 100, &dummy, &dummy, &dummy, &dummy, NULL) == DSA_ERR_INVALID_ARG);
  CHECK(dsa_bs_pool(P, DSA_BF16, 1, 4, 256, 96, NULL, 0, (float*)P, NULL) == DSA_ERR_UNSUPPORTED);
  CHECK(dsa_bs_pool(P, 5, 1, 4, 256, 64, NULL, 0, (float*)P, NULL) == DSA_ERR_UNSUPPORTED);
  CHECK(dsa_bs_pool(NULL, DSA_BF16, 1, 4, 256, 64, NULL, 0, (float*)P, NULL) == DSA_ERR_INVALID_ARG);
  CHECK(dsa_bs_select((const float*)P, (const float*)P, 1, 10, 64, 0.f, 0, &dummy, &dummy, NULL, P, BIG,
                      NULL) == DSA_ERR_INVALID_ARG);
  CHECK(dsa_bs_select((const float*)P, (const float*)P, 1, 10, 64, 0.f, 4, &dummy, &dummy, NULL, P, 0, NULL) ==
        DSA_ERR_WORKSPACE);
  CHECK(dsa_sparse_attention_vs(P, P, P, P, &sh, 0.f, NULL, 0, P, P, -1, P, P, 4, NULL) == DSA_ERR_INVALID_ARG);
  CHECK(dsa_sparse_attention_vs(P, P, P, P, &sh, 0.f, NULL, 0, NULL, P, 4, P, P, 4, NULL) ==
        DSA_ERR_INVALID_ARG);
  CHECK(dsa_sparse_attention_blocks(P, P, P, P, &sh, 0.f, NULL, 0, P, P, -1, NULL) == DSA_ERR_INVALID_ARG);
  CHECK(dsa_sparse_attention_blocks(P, P, P, P, &sh, 0.f, NULL, 0, NULL, P, 4, NULL) == DSA_ERR_INVALID_ARG);

  /* decode: a negative list width, counts missing, too large for the static scratch */
  CHECK(dsa_sparse_decode(P, P, P, P, &sh, 0.f, NULL, 0, P, -1, P, P, BIG, NULL) == DSA_ERR_INVALID_ARG);
  CHECK(dsa_sparse_decode(P, P, P, P, &sh, 0.f, NULL, 0, P, 4, NULL, P, BIG, NULL) == DSA_ERR_INVALID_ARG);
  dsa_shape longd = sh;
  longd.batch = 512; /* 65536 decode rows: one split each, 34 MB of partials */
  longd.q_heads = 128;
  longd.kv_heads = 8;
  longd.seq_len = 4096;
  CHECK(dsa_sparse_decode_noalloc(P, P, P, P, &longd, 0.f, NULL, 0, NULL, 0, NULL, NULL) == DSA_ERR_WORKSPACE);

  /* workspace sizes at the largest accepted shape stay finite and grow with it */
  dsa_shape big = {64, 128, 8, ((int32_t)1 << 23) - 64, 128, DSA_BF16};
  CHECK(dsa_vertical_slash_workspace_bytes(&big, 1 << 20, 1 << 20, 128) >
        dsa_vertical_slash_workspace_bytes(&sh, 8, 8, 4));
  CHECK(dsa_block_sparse_workspace_bytes(&big, 1 << 16, 128) > dsa_block_sparse_workspace_bytes(&sh, 4, 4));
  CHECK(dsa_vs_estimate_workspace_bytes(&big, 128) > 0);
  CHECK(dsa_kv_retention_workspace_bytes(&big, 1 << 20, 128) > 0);
  CHECK(dsa_sparse_decode_workspace_bytes(&big, 1 << 20, 128) > 0);
  CHECK(dsa_bs_select_workspace_bytes(8192, 1 << 17) > 0);
  CHECK(dsa_topk_workspace_bytes(8192, (1 << 23) - 64, 1000) > 0); /* chunked two-pass rows */

  printf("%s\n", fails ? "c abi: failures" : "c abi: ok");
  return fails != 0;
}
