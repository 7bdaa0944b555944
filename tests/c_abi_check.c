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

  printf("%s\n", fails ? "c abi: failures" : "c abi: ok");
  return fails != 0;
}
