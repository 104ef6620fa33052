/* A plain C11 client of include/segpaged.h (compiled by gcc as C, linked against
 * libsegpaged.so): the host-only calls, driven by layouts read from stdin. For each layout
 *   B Hkv P
 *   ctx_len[0..B)
 *   q_len[0..B)
 *   Hkv lines: kind sink window
 * it prints "status n_pages n_retrieval_rows" and then, on success, the seg_table and kv_len
 * entries on one line each. A final line checks argument validation and status strings. */
#include <stdio.h>
#include <stdlib.h>

#include "segpaged.h"

static int read_i32(int32_t* x) { return scanf("%d", x) == 1; }

int main(void) {
  int32_t B, Hkv, P;
  while (read_i32(&B) && read_i32(&Hkv) && read_i32(&P)) {
    int32_t* ctx = malloc(sizeof(int32_t) * (size_t)(B > 0 ? B : 1));
    int32_t* q = malloc(sizeof(int32_t) * (size_t)(B > 0 ? B : 1));
    sp_head_policy* pol = malloc(sizeof(sp_head_policy) * (size_t)Hkv);
    for (int32_t b = 0; b < B; ++b) read_i32(&ctx[b]);
    for (int32_t b = 0; b < B; ++b) read_i32(&q[b]);
    for (int32_t h = 0; h < Hkv; ++h) {
      read_i32(&pol[h].kind);
      read_i32(&pol[h].sink);
      read_i32(&pol[h].window);
    }
    int64_t n_pages = -1, n_rows = -1;
    sp_status st = segpaged_plan_pages(B, ctx, q, Hkv, pol, P, &n_pages);
    if (st == SP_OK) st = segpaged_retrieval_rows(B, ctx, q, Hkv, pol, &n_rows);
    printf("%d %lld %lld\n", (int)st, (long long)n_pages, (long long)n_rows);
    if (st == SP_OK) {
      const size_t nh = (size_t)B * (size_t)Hkv;
      int32_t* seg = malloc(sizeof(int32_t) * (nh * 8 + 1));
      int32_t* kvl = malloc(sizeof(int32_t) * (nh + 1));
      st = segpaged_layout_tables(B, ctx, q, Hkv, pol, P, seg, kvl);
      if (st != SP_OK) {
        printf("tables failed %d\n", (int)st);
        return 1;
      }
      for (size_t i = 0; i < nh * 8; ++i) printf("%d ", seg[i]);
      printf("\n");
      for (size_t i = 0; i < nh; ++i) printf("%d ", kvl[i]);
      printf("\n");
      free(seg);
      free(kvl);
    }
    free(ctx);
    free(q);
    free(pol);
  }
  /* validation: null outputs and arrays, an unsupported page size, a bad policy */
  int32_t c1[1] = {100}, q1[1] = {1};
  sp_head_policy g[1] = {{SP_GLOBAL, 0, 1}}, bad[1] = {{SP_LOCAL, 4, 0}};
  int64_t n = 0;
  printf("checks %d %d %d %d %d %s\n", (int)segpaged_plan_pages(1, c1, q1, 1, g, 64, NULL),
         (int)segpaged_plan_pages(1, NULL, q1, 1, g, 64, &n),
         (int)segpaged_plan_pages(1, c1, q1, 1, g, 48, &n),
         (int)segpaged_plan_pages(1, c1, q1, 1, bad, 64, &n),
         (int)segpaged_plan_pages(1, c1, q1, 1, g, 64, &n),
         segpaged_status_string(SP_ERR_UNSUPPORTED) != NULL ? "named" : "null");
  return 0;
}
