/* Host-side calls of the C ABI, for a build whose host code carries the
 * address and undefined-behaviour sanitizers. Every call here fails its
 * argument checks or is a size query, so nothing is launched (no GPU is
 * needed); the sanitizers watch the host-side validation, planning and size
 * arithmetic over extreme shapes. Exit status 0 when every status is the
 * expected one. */
#include <limits.h>
#include <stdint.h>
#include <stdio.h>

#include "wedlm.h"

static int fails = 0;
#define EXPECT(c)                                                  \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "line %d: expected %s\n", __LINE__, #c);     \
      ++fails;                                                     \
    }                                                              \
  } while (0)

static const int kVals[] = {INT_MIN, -7, -1, 0, 1, 2, 7, 15, 16, 17, 63, 64, 65, 127, 128, 129,
                            255, 256, 257, 4096, 65535, 65536, 1 << 20, INT_MAX - 1, INT_MAX};
#define NV ((int)(sizeof(kVals) / sizeof(kVals[0])))

int main(void) {
  for (int s = -20; s <= 5; ++s) EXPECT(wedlm_status_string(s) != NULL);
  EXPECT((wedlm_abi_version() >> 16) == 1);

  /* size queries: each argument swept over extreme values, the others valid */
  {
    int base[9] = {WEDLM_BF16, 2, 4, 16, 32, 8, 128, 16, 4096};
    for (int a = 0; a < 9; ++a)
      for (int i = 0; i < NV; ++i) {
        int x[9];
        for (int j = 0; j < 9; ++j) x[j] = base[j];
        x[a] = kVals[i];
        size_t n = wedlm_window_attn_workspace_size(x[0], x[1], x[2], x[3], x[4], x[5], x[6],
                                                    x[7], x[8]);
        (void)n;
      }
    /* and every pair of arguments swept together */
    for (int a = 0; a < 9; ++a)
      for (int b = a + 1; b < 9; ++b)
        for (int i = 0; i < NV; ++i)
          for (int k = 0; k < NV; ++k) {
            int x[9];
            for (int j = 0; j < 9; ++j) x[j] = base[j];
            x[a] = kVals[i];
            x[b] = kVals[k];
            (void)wedlm_window_attn_workspace_size(x[0], x[1], x[2], x[3], x[4], x[5], x[6],
                                                   x[7], x[8]);
          }
    EXPECT(wedlm_window_attn_workspace_size(WEDLM_BF16, 1, 1, 16, 32, 8, 64, 16, 2048) == 0);
    EXPECT(wedlm_window_attn_workspace_size(WEDLM_BF16, 1, 4, 16, 32, 8, 128, 16, 32768) > 0);
  }
  {
    int base[4] = {WEDLM_BF16, 16, 16, 151936};
    for (int a = 0; a < 4; ++a)
      for (int i = 0; i < NV; ++i) {
        int x[4] = {base[0], base[1], base[2], base[3]};
        x[a] = kVals[i];
        (void)wedlm_entropy_select_workspace_size(x[0], x[1], x[2], x[3]);
      }
    for (int i = 0; i < NV; ++i)
      for (int k = 0; k < NV; ++k)
        for (int m = 0; m < NV; ++m)
          (void)wedlm_entropy_select_workspace_size(WEDLM_BF16, kVals[i], kVals[k], kVals[m]);
    EXPECT(wedlm_entropy_select_workspace_size(WEDLM_BF16, 16, 16, 151936) > 0);
    EXPECT(wedlm_entropy_select_workspace_size(WEDLM_BF16, 16, 65, 151936) == 0);
  }
  {
    int base[5] = {WEDLM_BF16, 16, 16, 4096, 151936};
    for (int a = 0; a < 5; ++a)
      for (int i = 0; i < NV; ++i) {
        int x[5] = {base[0], base[1], base[2], base[3], base[4]};
        x[a] = kVals[i];
        (void)wedlm_lm_head_select_workspace_size(x[0], x[1], x[2], x[3], x[4]);
        (void)wedlm_lm_head_packed_size(x[0], x[3], x[4]);
      }
    for (int a = 1; a < 5; ++a)
      for (int b = a + 1; b < 5; ++b)
        for (int i = 0; i < NV; ++i)
          for (int k = 0; k < NV; ++k) {
            int x[5] = {base[0], base[1], base[2], base[3], base[4]};
            x[a] = kVals[i];
            x[b] = kVals[k];
            (void)wedlm_lm_head_select_workspace_size(x[0], x[1], x[2], x[3], x[4]);
            (void)wedlm_lm_head_packed_size(x[0], x[3], x[4]);
          }
    EXPECT(wedlm_lm_head_packed_size(WEDLM_BF16, 4096, 151936) > 0);
    EXPECT(wedlm_lm_head_packed_size(WEDLM_BF16, 100, 151936) == 0);
  }

  /* invalid calls: each returns a negative status before any launch */
  int32_t i32[64] = {0};
  uint8_t u8[64] = {0};
  float f32[64] = {0};
  void* p = i32;
  for (int i = 0; i < NV; ++i) {
    const int v = kVals[i];
    EXPECT(wedlm_window_reorder(v, 8, NULL, i32, i32, i32, i32, i32, i32, NULL) < 0);
    EXPECT(wedlm_window_reorder_rule(1, v, 2, u8, i32, i32, i32, i32, i32, i32, NULL) < 0);
    EXPECT(wedlm_rope_logical(WEDLM_BF16, v, 1, 8, 4, 2, 128, 1e6, p, p, p, i32, i32, NULL, p, p,
                              NULL) < 0);
    EXPECT(wedlm_window_attn(WEDLM_BF16, 1, v, 16, 32, 8, 128, 16, 64, 8, 100, 0.1f, p, p, p, p,
                             p, i32, i32, NULL, NULL, 0, 0, NULL) < 0);
    EXPECT(wedlm_window_attn_rope(WEDLM_BF16, 1, 4, v, 32, 8, 128, 16, 64, 8, 100, 0.1f, 1e6, p,
                                  p, p, i32, i32, p, p, i32, i32, NULL, NULL, NULL, 0, 0,
                                  NULL) < 0);
    EXPECT(wedlm_window_attn_rope_entropy(WEDLM_BF16, 1, 4, 16, v, 8, 128, 16, 64, 8, 100, 0.1f,
                                          1e6, p, p, p, i32, i32, p, p, i32, i32, NULL, NULL,
                                          NULL, 0, 0, 151936, p, NULL, 0, NULL) < 0);
    EXPECT(wedlm_entropy_select(WEDLM_BF16, 16, 16, v, NULL, u8, 0.1f, 1.f, 1, f32, f32, i32, u8,
                                p, 64, NULL) < 0);
    EXPECT(wedlm_entropy_select_noalloc(WEDLM_BF16, v, 16, 1000, NULL, u8, 0.1f, 1.f, 1, f32,
                                        f32, i32, u8, NULL) < 0);
    EXPECT(wedlm_lm_head_pack(WEDLM_BF16, v, 1000, NULL, p, NULL) < 0);
    EXPECT(wedlm_lm_head_select(WEDLM_BF16, 1, 16, v, 1000, NULL, p, u8, 0.1f, 1.f, 1, f32, f32,
                                i32, u8, p, 64, NULL) < 0);
    EXPECT(wedlm_commit_prefix(WEDLM_BF16, 1, v, 16, 8, 128, 16, 64, 8, i32, u8, i32, p, p, i32,
                               p, p, i32, u8, i32, NULL, i32, -1, NULL) < 0);
    EXPECT(wedlm_commit_prefix_rope(WEDLM_BF16, 1, 4, v, 8, 128, 16, 64, 8, 1e6, i32, u8, i32, p,
                                    p, i32, p, p, i32, u8, i32, NULL, i32, -1, NULL) < 0);
    EXPECT(wedlm_select_commit_reorder(WEDLM_BF16, 4, 16, v, NULL, 0.1f, 1.f, 1, 16, 64, 8, 0,
                                       i32, i32, i32, u8, i32, i32, i32, -1, f32, f32, i32, u8,
                                       i32, i32, i32, i32, p, 64, NULL) < 0);
    EXPECT(wedlm_entropy_partials(WEDLM_BF16, v, 16, 1000, NULL, p, 64, NULL) < 0);
    EXPECT(wedlm_select_commit_reorder_partials(WEDLM_BF16, 4, v, 1000, 0.1f, 1.f, 1, 16, 64, 8,
                                                0, i32, i32, i32, u8, i32, i32, i32, -1, f32,
                                                f32, i32, u8, i32, i32, i32, i32, NULL, 0,
                                                NULL) < 0);
    EXPECT(wedlm_select_commit_reorder_combine(
               WEDLM_BF16, 4, 16, 1000, 0.1f, 1.f, 1, 16, 64, 8, 0, i32, i32, i32, u8, i32, i32,
               i32, -1, f32, f32, i32, u8, i32, i32, i32, i32, NULL, 0, v, 32, 8, 128, 4096,
               NULL, 0, NULL, NULL) < 0);
    EXPECT(wedlm_block_attn_rope(WEDLM_BF16, v, 256, 16, 32, 8, 128, 16, 64, 8, 0.1f, 1e6, p, p,
                                 p, i32, i32, p, p, i32, NULL, NULL) < 0);
    EXPECT(wedlm_read_probe(NULL, (size_t)v, i32, v, (uint32_t*)i32, 1, NULL) < 0);
  }
  if (fails) {
    fprintf(stderr, "%d unexpected statuses\n", fails);
    return 1;
  }
  printf("ok\n");
  return 0;
}
