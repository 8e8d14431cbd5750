/* A plain C99 caller of the library: builds masks through the C ABI, reads
 * them back and checks the host-side results against closed forms, and
 * checks the argument validation of the launch entry points (which returns
 * before any device work).  Prints "ok" and exits 0 on success. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "attn_jvp.h"

#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                      \
    }                                                                \
  } while (0)

int main(void) {
  CHECK(attn_jvp_version() == ATTN_JVP_API_VERSION);
  CHECK(strcmp(attn_jvp_status_str(ATTN_JVP_OK), "ok") == 0);

  /* chunk-wise TF mask: 6 frames of 10 tokens, 2 frames per chunk:
   * F = 3 chunks of C = 20 tokens, C^2 F (F + 1) admissible pairs */
  attn_jvp_mask *m = NULL;
  CHECK(attn_jvp_mask_tf(6, 10, 2, &m) == ATTN_JVP_OK && m != NULL);
  int32_t n_q = 0, n_k = 0, n_groups = 0, n_ranges = 0;
  int64_t pairs = 0;
  CHECK(attn_jvp_mask_info(m, &n_q, &n_k, &n_groups, &n_ranges, &pairs) == ATTN_JVP_OK);
  CHECK(n_q == 120 && n_k == 120 && n_groups == 6);
  CHECK(pairs == (int64_t)20 * 20 * 3 * 4);

  int32_t *gq = malloc(sizeof(int32_t) * (n_groups + 1));
  int32_t *rp = malloc(sizeof(int32_t) * (n_groups + 1));
  int32_t *kb = malloc(sizeof(int32_t) * n_ranges);
  int32_t *ke = malloc(sizeof(int32_t) * n_ranges);
  CHECK(attn_jvp_mask_export(m, gq, rp, kb, ke) == ATTN_JVP_OK);
  /* every row of a noisy chunk u sees the clean chunks before it and itself:
   * count from the export */
  int64_t counted = 0;
  for (int g = 0; g < n_groups; ++g)
    for (int r = rp[g]; r < rp[g + 1]; ++r) counted += (int64_t)(gq[g + 1] - gq[g]) * (ke[r] - kb[r]);
  CHECK(counted == pairs);

  /* the same mask rebuilt from its CSR form is identical */
  attn_jvp_mask *m2 = NULL;
  CHECK(attn_jvp_mask_rects(n_q, n_k, n_groups, gq, rp, kb, ke, &m2) == ATTN_JVP_OK);
  int64_t pairs2 = 0;
  int32_t a, b, c, d;
  CHECK(attn_jvp_mask_info(m2, &a, &b, &c, &d, &pairs2) == ATTN_JVP_OK);
  CHECK(pairs2 == pairs && c == n_groups && d == n_ranges);

  /* the transpose has as many pairs, and transposing twice gives back the rows */
  attn_jvp_mask *t = NULL, *tt = NULL;
  CHECK(attn_jvp_mask_transpose(m, &t) == ATTN_JVP_OK);
  CHECK(attn_jvp_mask_transpose(t, &tt) == ATTN_JVP_OK);
  int64_t pt = 0, ptt = 0;
  CHECK(attn_jvp_mask_info(t, &a, &b, &c, &d, &pt) == ATTN_JVP_OK && pt == pairs);
  CHECK(attn_jvp_mask_info(tt, &a, &b, &c, &d, &ptt) == ATTN_JVP_OK && ptt == pairs);

  /* block schedule for 64-row tiles of 32-key blocks: 2 tiles */
  int32_t n_tiles = 0;
  int64_t n_entries = 0, n_partial = 0;
  CHECK(attn_jvp_mask_schedule(m, 64, 32, &n_tiles, &n_entries, &n_partial, NULL, NULL, NULL,
                               NULL, NULL) == ATTN_JVP_OK);
  CHECK(n_tiles == 2 && n_entries > 0);
  CHECK(attn_jvp_mask_schedule(m, 64, 48, &n_tiles, &n_entries, &n_partial, NULL, NULL, NULL,
                               NULL, NULL) == ATTN_JVP_ERR_SHAPE);

  /* block-causal and dense builders */
  attn_jvp_mask *bc = NULL, *dn = NULL;
  CHECK(attn_jvp_mask_block_causal(4, 5, &bc) == ATTN_JVP_OK);
  CHECK(attn_jvp_mask_info(bc, &a, &b, &c, &d, &pt) == ATTN_JVP_OK && pt == (int64_t)25 * 10);
  CHECK(attn_jvp_mask_dense(7, 9, &dn) == ATTN_JVP_OK);
  CHECK(attn_jvp_mask_info(dn, &a, &b, &c, &d, &pt) == ATTN_JVP_OK && pt == 63);

  /* launch entry points reject bad arguments before touching a device */
  attn_jvp_args args;
  memset(&args, 0, sizeof(args));
  args.dtype = ATTN_JVP_BF16;
  args.B = 1;
  args.H = 1;
  args.n_q = 120;
  args.n_k = 120;
  args.D = 96; /* unsupported head dim */
  args.q = args.k = args.v = (const void *)(uintptr_t)0x10000;
  args.o = (void *)(uintptr_t)0x20000;
  args.lse = (float *)(uintptr_t)0x30000;
  args.q_stride_n = args.k_stride_n = 128;
  args.q_stride_h = args.k_stride_h = 128;
  CHECK(attn_jvp_fwd(&args, m, NULL) == ATTN_JVP_ERR_UNSUPPORTED);
  CHECK(attn_jvp_fwd(NULL, m, NULL) == ATTN_JVP_ERR_NULL);
  args.D = 128;
  args.n_q = 119;
  CHECK(attn_jvp_fwd(&args, m, NULL) == ATTN_JVP_ERR_MASK);
  args.n_q = 120;
  uint64_t ws = 7;
  CHECK(attn_jvp_fwd_split_workspace(&args, m, 1, &ws) == ATTN_JVP_OK && ws == 0);
  CHECK(attn_jvp_fwd_split(&args, m, 0, NULL, 0, NULL) == ATTN_JVP_ERR_SHAPE);
  int32_t chosen = 0;
  CHECK(attn_jvp_split_choose(&args, m, 256, &chosen) == ATTN_JVP_OK && chosen >= 1);
  int32_t bm = 0, bn = 0;
  CHECK(attn_jvp_tile_shape(ATTN_JVP_BF16, 128, 1, &bm, &bn) == ATTN_JVP_OK && bm == 256 && bn == 32);
  CHECK(attn_jvp_tile_shape(ATTN_JVP_BF16, 128, 0, &bm, &bn) == ATTN_JVP_OK && bm == 256 && bn == 64);

  attn_jvp_bwd_args bargs;
  memset(&bargs, 0, sizeof(bargs));
  CHECK(attn_jvp_bwd(&bargs, m, NULL) == ATTN_JVP_ERR_NULL);

  attn_jvp_mask_free(dn);
  attn_jvp_mask_free(bc);
  attn_jvp_mask_free(tt);
  attn_jvp_mask_free(t);
  attn_jvp_mask_free(m2);
  attn_jvp_mask_free(m);
  attn_jvp_mask_free(NULL);
  free(gq);
  free(rp);
  free(kb);
  free(ke);
  printf("ok\n");
  return 0;
}
