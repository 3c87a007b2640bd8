/* The C ABI used from plain C (no Python, no HIP headers): the library links,
 * reports its version and status strings, and rejects bad arguments on the
 * host before launching anything (CPU only: no call reaches a kernel). */
#include <stdio.h>

#include "../../include/moelb.h"

static int fails = 0;
#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);          \
      ++fails;                                                        \
    }                                                                 \
  } while (0)

int main(void) {
  void* P = (void*)16; /* never dereferenced: validation fails first */
  size_t need;
  EXPECT(moelb_version() == 100);
  EXPECT(moelb_status_string(MOELB_EINVAL) != NULL);
  /* k > E; T not a multiple of G; L > N */
  EXPECT(moelb_gate_topk(P, 4, 8, 2, 3, MOELB_BF16, P, P, NULL, NULL, P, P, NULL, NULL, NULL) == MOELB_EINVAL);
  EXPECT(moelb_histogram(P, 10, 2, 8, 4, P, NULL, NULL) == MOELB_EINVAL);
  EXPECT(moelb_plan(P, P, 4, 8, 1, 2, P, NULL, NULL) == MOELB_EINVAL);
  /* negative passes; unknown variant; stale split over its own input */
  EXPECT(moelb_split(P, P, P, 4, 8, 1, -1, 0, P, P, NULL) == MOELB_EINVAL);
  EXPECT(moelb_split_variant(P, P, P, 4, 8, 1, 12, 0, 99, P, P, NULL) == MOELB_EINVAL);
  EXPECT(moelb_split_stale(P, P, P, 4, 8, 1, P, P, P, NULL) == MOELB_EINVAL);
  /* swap planner: gamma denominator 0 */
  EXPECT(moelb_plan_swaps(P, P, 4, 8, 0, 1, 0, 2, P, NULL, NULL, P, NULL) == MOELB_EINVAL);
  /* permutation: workspace one byte short */
  need = moelb_permute_workspace_bytes(64, 2, 8, 4);
  EXPECT(need > 0);
  EXPECT(moelb_permute(NULL, P, 64, 8, 2, 8, 4, 1, MOELB_BF16, P, P, P, P, need - 1, P, P, P, NULL, NULL) ==
         MOELB_EWORKSPACE);
  /* grouped FFN: d not a multiple of 8; combine: k above the limit */
  EXPECT(moelb_grouped_ffn(P, 8, 8, P, 8, 2, 2, 0, NULL, 1, 12, 8, MOELB_BF16, P, P, P, 1u << 30, P, NULL) ==
         MOELB_EINVAL);
  EXPECT(moelb_combine(P, 8, P, P, 4, 17, 8, MOELB_BF16, NULL, P, NULL) == MOELB_EINVAL);
  /* every status string, including unknown codes */
  for (int st = -2; st < 6; ++st) EXPECT(moelb_status_string(st) != NULL);
  /* workspace sizes: zero for invalid shapes, growing with the batch, no
     overflow at the largest shapes the entry points accept */
  EXPECT(moelb_permute_workspace_bytes(64, 2, 8, 0) == 0);
  EXPECT(moelb_permute_workspace_bytes(1 << 20, 16, 256, 64) > moelb_permute_workspace_bytes(1 << 10, 16, 256, 64));
  EXPECT(moelb_grouped_ffn_workspace_bytes(-1, 8, 8, 64, 64, MOELB_BF16) == 0);
  EXPECT(moelb_grouped_ffn_workspace_bytes(1 << 24, 32768, 256, 8192, 8192, MOELB_F32) >
         (size_t)(1 << 24) * 8192 * 4);
  /* FFN stages outside [1, MOELB_FFN_ALL]; rows without source rows */
  EXPECT(moelb_grouped_ffn_stages(0, P, 8, 8, P, 8, 2, 2, 0, NULL, 1, 8, 8, MOELB_BF16, P, P, P, 1u << 30, P, NULL) ==
         MOELB_EINVAL);
  EXPECT(moelb_grouped_ffn_stages(8, P, 8, 8, P, 8, 2, 2, 0, NULL, 1, 8, 8, MOELB_BF16, P, P, P, 1u << 30, P, NULL) ==
         MOELB_EINVAL);
  EXPECT(moelb_grouped_ffn(P, 0, 8, P, 8, 2, 2, 0, NULL, 1, 8, 8, MOELB_BF16, P, P, P, 1u << 30, P, NULL) ==
         MOELB_EINVAL);
  /* packed weights: bf16 with d and inter multiples of 64 only */
  EXPECT(moelb_grouped_ffn_stages(MOELB_FFN_ALL | MOELB_FFN_PACKED_WEIGHTS, P, 8, 8, P, 8, 2, 2, 0, NULL, 1, 8, 64,
                                  MOELB_BF16, P, P, P, 1u << 30, P, NULL) == MOELB_EINVAL);
  EXPECT(moelb_grouped_ffn_stages(MOELB_FFN_ALL | MOELB_FFN_PACKED_WEIGHTS, P, 8, 8, P, 8, 2, 2, 0, NULL, 1, 64, 64,
                                  MOELB_F32, P, P, P, 1u << 30, P, NULL) == MOELB_EINVAL);
  EXPECT(moelb_pack_weights(P, 2, 12, 64, MOELB_BF16, (void*)(1ull << 30), NULL) == MOELB_EINVAL);
  EXPECT(moelb_pack_weights(P, 2, 16, 96, MOELB_BF16, (void*)(1ull << 30), NULL) == MOELB_EINVAL);
  EXPECT(moelb_pack_weights(P, 2, 16, 64, MOELB_F32, (void*)(1ull << 30), NULL) == MOELB_EINVAL);
  EXPECT(moelb_pack_weights(P, 2, 16, 64, MOELB_BF16, (char*)P + 64, NULL) == MOELB_EINVAL);
  /* operands whose byte offsets would not fit 32 bits */
  EXPECT(moelb_grouped_ffn(P, 1 << 20, 8, P, 8, 2, 2, 0, NULL, 1, 4096, 8, MOELB_BF16, P, P, P, 1u << 30, P, NULL) ==
         MOELB_EINVAL);
  /* the no-allocation permutation: a workspace beyond its fixed array */
  EXPECT(moelb_permute_noalloc(NULL, P, 1 << 22, 64, 8, 256, 64, 1, MOELB_BF16, P, P, P, P, P, P, NULL, NULL) ==
         MOELB_EWORKSPACE);
  /* split schedule and scheduled split: bad sizes */
  EXPECT(moelb_split_schedule(P, P, 65, 8, 1, P, NULL) == MOELB_EINVAL);
  EXPECT(moelb_split_scheduled(P, P, P, NULL, 4, 8, 9, 12, 0, 0, P, P, NULL) == MOELB_EINVAL);
  printf("%s\n", fails ? "failed" : "ok");
  return fails != 0;
}
