/*
 * Host-side checks of libtq built with AddressSanitizer and
 * UndefinedBehaviorSanitizer (host code only, no device code): every
 * exported call on valid and malformed host arguments that is answered
 * before any device work -- codebooks, format validation, tile and
 * workspace sizes, error strings, and the argument checks of the write,
 * decode, merge, window and self-test calls.  Built and run by
 * tests/test_host_sanitizers.py; prints "ok" and exits 0 when every check
 * holds and the sanitizers report nothing.
 */
#include <stdio.h>
#include <string.h>

#include "tq.h"

static int fails = 0;
#define CHECK(c)                                                  \
  do {                                                            \
    if (!(c)) {                                                   \
      printf("FAIL line %d: %s (%s)\n", __LINE__, #c, tq_last_error()); \
      ++fails;                                                    \
    }                                                             \
  } while (0)

static void make_format(tq_format* f, int d, int ng, int b0, int b1) {
  memset(f, 0, sizeof *f);
  f->head_dim = d;
  f->num_groups = ng;
  f->group_bits[0] = b0;
  f->group_bits[1] = ng == 2 ? b1 : 0;
  for (int i = 0; i < d; ++i) {
    f->group_channels[i] = (uint8_t)i;
    f->signs[i] = (i * 7 + 3) % 5 < 2 ? -1 : 1;
  }
  tq_lloyd_max_codebook(b0, f->codebook[0]);
  if (ng == 2) tq_lloyd_max_codebook(b1, f->codebook[1]);
}

int main(void) {
  uint16_t cb[16];
  for (int b = 1; b <= 4; ++b) CHECK(tq_lloyd_max_codebook(b, cb) == TQ_OK);
  CHECK(tq_lloyd_max_codebook(0, cb) == TQ_ERR_VALUE);
  CHECK(tq_lloyd_max_codebook(5, cb) == TQ_ERR_VALUE);
  CHECK(tq_lloyd_max_codebook(3, NULL) == TQ_ERR_VALUE);
  CHECK(strlen(tq_last_error()) > 0);

  tq_format f, g;
  make_format(&f, 128, 1, 4, 0);
  CHECK(tq_format_check(&f) == TQ_OK);
  make_format(&g, 128, 2, 4, 3);
  CHECK(tq_format_check(&g) == TQ_OK);
  CHECK(tq_format_check(NULL) == TQ_ERR_VALUE);
  g = f; g.head_dim = 96;                    CHECK(tq_format_check(&g) != TQ_OK);
  g = f; g.group_bits[0] = 5;                CHECK(tq_format_check(&g) != TQ_OK);
  g = f; g.signs[5] = 0;                     CHECK(tq_format_check(&g) != TQ_OK);
  g = f; g.codebook[0][3] = g.codebook[0][2]; CHECK(tq_format_check(&g) != TQ_OK);
  g = f; g.codebook[0][0] = 0x7C00;          CHECK(tq_format_check(&g) != TQ_OK);   /* +inf level */
  g = f; g.num_groups = 3;                   CHECK(tq_format_check(&g) != TQ_OK);
  make_format(&g, 128, 2, 4, 3);
  g.group_channels[1] = 0;                   CHECK(tq_format_check(&g) != TQ_OK);   /* duplicate channel */
  make_format(&g, 128, 2, 4, 3);
  g.group_channels[0] = 1; g.group_channels[1] = 0;
  CHECK(tq_format_check(&g) != TQ_OK);                                              /* group not ascending */
  CHECK(strlen(tq_last_error()) > 0);

  int32_t rb = 0, tile = 0;
  CHECK(tq_tile_bytes(&f, 16, &rb, &tile) == TQ_OK && rb == 64 && tile == 16 * 64 + 32);
  CHECK(tq_tile_bytes(&f, 8, &rb, &tile) != TQ_OK);
  CHECK(tq_tile_bytes(&f, 16, NULL, &tile) == TQ_ERR_VALUE);
  uint64_t ws = 0;
  CHECK(tq_decode_workspace_bytes(4, 32, 128, 1, &ws) == TQ_OK && ws == 0);
  CHECK(tq_decode_workspace_bytes(4, 32, 128, 16, &ws) == TQ_OK && ws == 4ull * 32 * 16 * 129 * 4);
  CHECK(tq_decode_workspace_bytes(-1, 32, 128, 16, &ws) == TQ_ERR_VALUE);

  /* stand-in device pointers: every call below must be refused, or finish
     with nothing to do, before it touches one */
  void* dp = (void*)(uintptr_t)0x1000;
  int64_t* slots = (int64_t*)dp;
  CHECK(tq_write_kv(NULL, NULL, TQ_BF16, 4, 8, slots, dp, dp, 10, 16, &f, &f, NULL, NULL) == TQ_ERR_VALUE);
  CHECK(tq_write_kv(dp, dp, (tq_dtype)7, 4, 8, slots, dp, dp, 10, 16, &f, &f, NULL, NULL) == TQ_ERR_VALUE);
  CHECK(tq_write_kv(dp, dp, TQ_BF16, 4, 8, slots, dp, dp, 10, 8, &f, &f, NULL, NULL) == TQ_ERR_UNSUPPORTED_FORMAT);
  CHECK(tq_write_kv(dp, dp, TQ_BF16, 4, 8, NULL, dp, dp, 10, 16, &f, &f, NULL, NULL) == TQ_ERR_VALUE);
  CHECK(tq_write_kv(dp, dp, TQ_BF16, 0, 8, slots, dp, dp, 10, 16, &f, &f, NULL, NULL) == TQ_OK);

  const int32_t* ip = (const int32_t*)dp;
  const uint8_t* up = (const uint8_t*)dp;
  CHECK(tq_decode_paged(dp, TQ_BF16, 2, 7, 2, up, up, 10, 16, ip, 4, ip, &f, &f, 0.1f, 1, NULL, 0, dp, TQ_BF16,
                        NULL, NULL, NULL) == TQ_ERR_VALUE);
  CHECK(tq_decode_paged(dp, TQ_BF16, 2, 8, 2, up, up, 10, 8, ip, 4, ip, &f, &f, 0.1f, 1, NULL, 0, dp, TQ_BF16,
                        NULL, NULL, NULL) == TQ_ERR_UNSUPPORTED_FORMAT);
  CHECK(tq_decode_paged(dp, TQ_BF16, 2, 8, 2, up, up, 10, 16, ip, 4, ip, &f, &f, 0.1f, 4, NULL, 0, dp, TQ_BF16,
                        NULL, NULL, NULL) == TQ_ERR_VALUE);   /* workspace missing */
  CHECK(tq_decode_paged(dp, TQ_BF16, 0, 8, 2, up, up, 10, 16, ip, 4, ip, &f, &f, 0.1f, 1, NULL, 0, dp, TQ_BF16,
                        NULL, NULL, NULL) == TQ_OK);
  CHECK(tq_decode_paged_multi(dp, TQ_BF16, 2, 33, 8, 2, up, up, 10, 16, ip, 4, ip, &f, &f, 0.1f, 1, NULL, 0, dp,
                              TQ_BF16, NULL, NULL, NULL) == TQ_ERR_UNSUPPORTED_FORMAT);
  CHECK(tq_decode_paged_noalloc(dp, TQ_BF16, 600, 64, 8, up, up, 10, 16, ip, 4, ip, &f, &f, 0.1f, 128, dp,
                                TQ_BF16, NULL, NULL, NULL) == TQ_ERR_VALUE);
  CHECK(tq_decode_paged_window(dp, TQ_BF16, 2, 8, 2, up, up, 10, 16, ip, 4, ip, &f, &f, dp, dp, TQ_F32, 4, ip,
                               0.1f, 1, NULL, 0, dp, TQ_BF16, NULL, NULL, NULL) == TQ_ERR_UNSUPPORTED_FORMAT);
  CHECK(tq_decode_paged_window(dp, TQ_BF16, 2, 8, 2, up, up, 10, 16, ip, 4, ip, &f, &f, dp, dp, TQ_BF16, -1, ip,
                               0.1f, 1, NULL, 0, dp, TQ_BF16, NULL, NULL, NULL) == TQ_ERR_VALUE);
  CHECK(tq_decode_dense(dp, TQ_BF16, 2, 34, 2, 128, dp, dp, TQ_BF16, 4, ip, 0.1f, NULL, NULL, dp, TQ_F32, NULL,
                        NULL, NULL) == TQ_ERR_UNSUPPORTED_FORMAT);
  CHECK(tq_decode_dense(dp, TQ_BF16, 2, 8, 2, 128, dp, dp, TQ_BF16, 4, ip, 0.1f, (const float*)dp, NULL, dp,
                        TQ_F32, NULL, NULL, NULL) == TQ_ERR_VALUE);
  CHECK(tq_split_merge((const float*)dp, (const float*)dp, 2, 2, 0, 128, dp, TQ_F32, NULL, NULL) == TQ_ERR_VALUE);
  CHECK(tq_split_merge((const float*)dp, (const float*)dp, 0, 2, 2, 128, dp, TQ_F32, NULL, NULL) == TQ_OK);
  CHECK(tq_selftest_fp64((const double*)dp, (const double*)dp, -1, NULL, NULL, NULL, NULL, NULL) == TQ_ERR_VALUE);
  CHECK(tq_selftest_fp64(NULL, NULL, 0, NULL, NULL, NULL, NULL, NULL) == TQ_OK);

  if (fails) {
    printf("FAILED %d\n", fails);
    return 1;
  }
  printf("ok\n");
  return 0;
}
