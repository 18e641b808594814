/* Plain C99 client of the library's host-only calls: the header compiles as
 * C, the symbols link, and planning statistics, the tile classifier and the
 * error path answer as documented. Needs no GPU. Prints "ok" on success. */
#include <stdio.h>
#include <string.h>

#include "magi_attn.h"

static int fails = 0;

static void check(int cond, const char* what) {
  if (!cond) {
    printf("FAIL: %s (%s)\n", what, magi_attn_last_error());
    ++fails;
  }
}

int main(void) {
  /* One video of three 64-token chunks, no KV cache. */
  const int32_t offsets[4] = {0, 64, 128, 192};
  const int32_t seqs[2] = {0, 3};
  magi_attn_layout_t lay;
  magi_attn_stats_t st;
  int8_t cls[9];
  int qt, kt;

  check(magi_attn_abi_version() == MAGI_ATTN_ABI_VERSION, "ABI version");
  check(strcmp(magi_attn_status_str(MAGI_ERR_UNSUPPORTED), "unsupported") == 0, "status string");

  memset(&lay, 0, sizeof lay);
  lay.n_seqs = 1;
  lay.seq_chunks = seqs;
  lay.n_chunks = 3;
  lay.q_offsets = offsets;
  lay.kv_offsets = NULL; /* = q_offsets */
  lay.n_q_heads = 4;
  lay.n_kv_heads = 2;
  lay.head_dim = 128;
  lay.dtype = MAGI_DTYPE_BF16;

  /* Chunk c's 64 rows see the 64 (c + 1) keys of chunks 0..c. */
  check(magi_attn_plan_stats(&lay, &st) == MAGI_OK, "plan stats");
  check(st.unmasked_pairs == 64 * 64 * (1 + 2 + 3), "unmasked pairs");
  check(st.n_items > 0, "work items");

  /* 64 x 64 tiles line up with the chunks: full (2) on and below the diagonal, empty (0) above. */
  check(magi_attn_classify_host(&lay, 64, 64, cls) == MAGI_OK, "classify");
  for (qt = 0; qt < 3; ++qt)
    for (kt = 0; kt < 3; ++kt) check(cls[qt * 3 + kt] == (kt <= qt ? 2 : 0), "tile class");

  /* 3 query heads do not group onto 2 KV heads: rejected with a message. */
  lay.n_q_heads = 3;
  check(magi_attn_plan_stats(&lay, &st) == MAGI_ERR_INVALID_ARG, "invalid head grouping");
  check(strlen(magi_attn_last_error()) > 0, "error message");

  if (fails) return 1;
  printf("ok\n");
  return 0;
}
