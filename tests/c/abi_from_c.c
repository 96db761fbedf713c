/* Calls the library's host-only entry points from plain C99 through
 * include/sparge.h: the header compiles as C, the library links and loads
 * without Python, and the calls behave as the header states.  Prints "ok"
 * and returns 0, or names the first failed check and returns 1.  No call
 * here touches a GPU. */
#include <stdio.h>
#include <string.h>

#include "sparge.h"

#define CHECK(cond)                                        \
  do {                                                     \
    if (!(cond)) {                                         \
      printf("failed: %s (line %d)\n", #cond, __LINE__);   \
      return 1;                                            \
    }                                                      \
  } while (0)

static int is_permutation(const int32_t* perm, const int32_t* inv, int n) {
  static unsigned char seen[4096];
  if (n > 4096) return 0;
  memset(seen, 0, sizeof seen);
  for (int p = 0; p < n; ++p) {
    if (perm[p] < 0 || perm[p] >= n || seen[perm[p]]) return 0;
    seen[perm[p]] = 1;
    if (inv[perm[p]] != p) return 0;
  }
  return 1;
}

int main(void) {
  CHECK(sparge_version() > 0);
  CHECK(sparge_rows_per_wave() > 0 && SPARGE_BQ % sparge_rows_per_wave() == 0);

  /* the stage-2 path: AUTO unless set; -1 only reads it */
  CHECK(sparge_attn_path(-1) == SPARGE_PATH_AUTO);
  CHECK(sparge_attn_path(SPARGE_PATH_FUSED) == SPARGE_PATH_AUTO);
  CHECK(sparge_attn_path(-1) == SPARGE_PATH_FUSED);
  CHECK(sparge_attn_path(SPARGE_PATH_AUTO) == SPARGE_PATH_FUSED);
  CHECK(sparge_attn_path(7) == SPARGE_EINVAL);
  CHECK(strlen(sparge_last_error()) > 0);

  /* a 4 x 4 x 4 grid: the Hilbert order is a permutation whose consecutive
     ranks are face neighbours (a 2^k cube) */
  int32_t perm[4096], inv[4096];
  CHECK(sparge_hilbert_index(4, 4, 4, perm, inv) == SPARGE_OK);
  CHECK(is_permutation(perm, inv, 64));
  for (int p = 1; p < 64; ++p) {
    int a = perm[p - 1], b = perm[p];
    int dt = a / 16 - b / 16, dh = (a / 4) % 4 - (b / 4) % 4, dw = a % 4 - b % 4;
    int dist = (dt < 0 ? -dt : dt) + (dh < 0 ? -dh : dh) + (dw < 0 ? -dw : dw);
    CHECK(dist == 1);
  }
  /* a ragged grid is still a permutation */
  CHECK(sparge_hilbert_index(3, 5, 7, perm, inv) == SPARGE_OK);
  CHECK(is_permutation(perm, inv, 105));
  CHECK(sparge_hilbert_index(0, 4, 4, perm, inv) == SPARGE_EINVAL);
  CHECK(sparge_hilbert_index(4, 4, 4, NULL, inv) == SPARGE_EINVAL);

  /* raster order is the identity; time-major puts a pixel's frames together */
  CHECK(sparge_grid_order(2, 3, 4, SPARGE_ORDER_ROWMAJOR, perm, inv) == SPARGE_OK);
  for (int p = 0; p < 24; ++p) CHECK(perm[p] == p && inv[p] == p);
  CHECK(sparge_grid_order(2, 3, 4, SPARGE_ORDER_TIMEMAJOR, perm, inv) == SPARGE_OK);
  CHECK(is_permutation(perm, inv, 24));
  CHECK(perm[0] == 0 && perm[1] == 12);
  CHECK(sparge_grid_order(2, 3, 4, 9, perm, inv) == SPARGE_EINVAL);

  /* workspace sizes: positive for a valid problem, growing with N, 0 for a
     bad shape */
  sparge_tensor q = {1, 8, 4096, 128, 8 * 4096 * 128, 4096 * 128, 128};
  sparge_tensor k = {1, 2, 4096, 128, 2 * 4096 * 128, 4096 * 128, 128};
  size_t w1 = sparge_workspace_size(&q, &k);
  CHECK(w1 > 0);
  q.N = k.N = 8192;
  CHECK(sparge_workspace_size(&q, &k) > w1);
  k.H = 3; /* 8 query heads do not split over 3 kv heads */
  CHECK(sparge_workspace_size(&q, &k) == 0);
  CHECK(sparge_l1_workspace_size() > 0);

  printf("ok\n");
  return 0;
}
