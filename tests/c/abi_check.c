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
  printf("%s\n", fails ? "failed" : "ok");
  return fails != 0;
}
