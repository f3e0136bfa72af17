/* The C ABI from plain C99: the header compiles as C, the library links,
   and argument validation answers before any HIP call (no GPU needed). */
#include <stdint.h>
#include <stdio.h>

#include "bsattn.h"

static int fails = 0;
#define EXPECT(cond)                                              \
  do {                                                            \
    if (!(cond)) {                                                \
      fprintf(stderr, "line %d: %s\n", __LINE__, #cond);          \
      ++fails;                                                    \
    }                                                             \
  } while (0)

int main(void) {
  EXPECT(bs_version() >= 100);
  int64_t nnz = -1;
  EXPECT(bs_layout_nnz(NULL, &nnz) == BS_ERR_INVALID_ARG && nnz == -1);
  int rows = -1, stride = -1;
  EXPECT(bs_layout_kv_share(NULL, &rows, &stride) == BS_ERR_INVALID_ARG);
  EXPECT(bs_layout_set_kv_share(NULL, 1) == BS_ERR_INVALID_ARG);
  uint8_t lay[4] = {1, 1, 1, 1};
  bs_layout_t L = NULL;
  EXPECT(bs_layout_build(lay, 1, 2, 2, 8, NULL, &L) == BS_ERR_UNSUPPORTED && L == NULL);
  EXPECT(bs_last_error() != NULL && bs_last_error()[0] != '\0');
  EXPECT(bs_layout_build(NULL, 1, 2, 2, 16, NULL, &L) == BS_ERR_INVALID_ARG);
  bs_acsr_term t = {5, 2, 1, 0, 1, 1}; /* row_begin > row_end */
  EXPECT(bs_layout_build_acsr(&t, 1, 1, 8, 8, 16, NULL, &L) == BS_ERR_INVALID_ARG);
  bs_layout_free(NULL);
  if (fails == 0) printf("abi_check ok\n");
  return fails == 0 ? 0 : 1;
}
