/* Host-side checks of libpark's argument validation and workspace sizing, built with the
 * address and undefined-behaviour sanitizers on the host code (test_host_sanitizers.py).
 * Every call here fails a host-side check or only computes a size, so nothing reaches a
 * GPU; the pointers passed are never dereferenced. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "park.h"

static int failures = 0;
#define EXPECT(expr, want)                                                              \
  do {                                                                                  \
    long long got_ = (long long)(expr);                                                 \
    if (got_ != (long long)(want)) {                                                    \
      fprintf(stderr, "%s:%d: %s = %lld, want %lld\n", __FILE__, __LINE__, #expr, got_, \
              (long long)(want));                                                       \
      ++failures;                                                                       \
    }                                                                                   \
  } while (0)

int main(void) {
  void* F = (void*)(uintptr_t)0x10000;          /* non-null, 256-byte aligned, never used */
  void* U = (void*)(uintptr_t)0x10008;          /* not 256-byte aligned */
  const size_t big = (size_t)1 << 40;
  const float nanf_ = NAN, inff_ = INFINITY;

  EXPECT(park_abi_version(), PARK_ABI_VERSION);
  for (int s = -3; s < 9; ++s) EXPECT(park_status_string(s) != NULL, 1);

  /* sizes: valid, at the maxima, and invalid ones that must give 0 without overflowing */
  for (int op = 0; op < 4; ++op) {
    EXPECT(park_workspace_bytes(op, 1, 40, 75600, 128, 1024) > 0, 1);
    EXPECT(park_workspace_bytes(op, 1, 24, 119056, 128, 1536) > 0, 1);
    EXPECT(park_workspace_bytes(op, 1, 1, 1, 64, 1) > 0, 1);
    EXPECT(park_workspace_bytes(op, 1, 1, 1000, 96, 8), 0);
    EXPECT(park_workspace_bytes(op, 1, 1, 1000, 128, 2000), 0);
    EXPECT(park_workspace_bytes(op, 0, 1, 1000, 128, 8), 0);
    EXPECT(park_workspace_bytes(op, 1 << 20, 1 << 20, 1 << 20, 128, 8), 0);
    EXPECT(park_workspace_bytes(op, 2147483647, 2147483647, 2147483647, 128, 8), 0);
    EXPECT(park_workspace_bytes(op, 1, 1, -5, 128, 8), 0);
  }
  EXPECT(park_workspace_bytes(9, 1, 1, 1000, 128, 8), 0);
  for (int op = 0; op < 3; ++op) {
    EXPECT(park_workspace_bytes_clustered(op, 1, 40, 75600, 128, 1024, 128) > 0, 1);
    EXPECT(park_workspace_bytes_clustered(op, 1, 40, 75600, 128, 1024, 1536) > 0, 1);
    EXPECT(park_workspace_bytes_clustered(op, 1, 40, 75600, 128, 1024, 0), 0);
    EXPECT(park_workspace_bytes_clustered(op, 1, 40, 75600, 128, 1024, 1537), 0);
    EXPECT(park_workspace_bytes_clustered(op, 1, 1, 10, 128, 4, 11), 0);
  }
  EXPECT(park_logmass_workspace_bytes(1, 40, 75600, 128, 1024) > 0, 1);
  EXPECT(park_logmass_workspace_bytes(1, 40, 75600, 96, 1024), 0);

  /* clustering */
#define CL(Q, dt, N, d, nk, it, met, al, ws, wsb) \
  park_cluster_keys(Q, F, dt, 1, 2, N, d, nk, it, met, al, NULL, F, F, F, F, F, NULL, ws, wsb, NULL)
  EXPECT(CL(NULL, 1, 256, 128, 8, 2, 0, 0.05f, F, big), PARK_ERR_INVALID);
  EXPECT(CL(F, 7, 256, 128, 8, 2, 0, 0.05f, F, big), PARK_ERR_INVALID);
  EXPECT(CL(F, 1, 0, 128, 8, 2, 0, 0.05f, F, big), PARK_ERR_INVALID);
  EXPECT(CL(F, 1, 256, 128, 300, 2, 0, 0.05f, F, big), PARK_ERR_INVALID);
  EXPECT(CL(F, 1, 256, 128, 8, 0, 0, 0.05f, F, big), PARK_ERR_INVALID);
  EXPECT(CL(F, 1, 256, 128, 8, 2, 3, 0.05f, F, big), PARK_ERR_INVALID);
  EXPECT(CL(F, 1, 256, 128, 8, 2, 0, nanf_, F, big), PARK_ERR_INVALID);
  EXPECT(CL(F, 1, 256, 128, 8, 2, 0, 1.5f, F, big), PARK_ERR_INVALID);
  EXPECT(CL(F, 1, 256, 96, 8, 2, 0, 0.05f, F, big), PARK_ERR_UNSUPPORTED);
  EXPECT(CL(F, 1, 4000, 128, 2000, 2, 0, 0.05f, F, big), PARK_ERR_UNSUPPORTED);
  EXPECT(CL(F, 1, 256, 128, 8, 2, 0, 0.05f, NULL, big), PARK_ERR_WORKSPACE);
  EXPECT(CL(F, 1, 256, 128, 8, 2, 0, 0.05f, F, 64), PARK_ERR_WORKSPACE);
  EXPECT(CL(F, 1, 256, 128, 8, 2, 0, 0.05f, U, big), PARK_ERR_WORKSPACE);
  EXPECT(park_cluster_queries(F, 1, 1, 1, 256, 128, 0, 2, NULL, F, F, F, F, F, F, big, NULL), PARK_ERR_INVALID);
  EXPECT(park_cluster_queries(F, 1, 1, 1, 256, 128, 8, 2, NULL, F, F, F, F, F, NULL, big, NULL), PARK_ERR_WORKSPACE);

  /* retrieval, all variants */
#define RB(fn, p, k, sc, qb, ws) fn(F, 1, 1, 2, 256, 128, F, F, 8, qb, p, k, sc, F, F, F, F, ws, big, NULL)
  EXPECT(RB(park_retrieve_blocks, 1.5f, 2, -1.0f, 64, F), PARK_ERR_INVALID);
  EXPECT(RB(park_retrieve_blocks, nanf_, 2, -1.0f, 64, F), PARK_ERR_INVALID);
  EXPECT(RB(park_retrieve_blocks, 0.9f, -1, -1.0f, 64, F), PARK_ERR_INVALID);
  EXPECT(RB(park_retrieve_blocks, 0.9f, 2, inff_, 64, F), PARK_ERR_INVALID);
  EXPECT(RB(park_retrieve_blocks, 0.9f, 2, -1.0f, 32, F), PARK_ERR_UNSUPPORTED);
  EXPECT(RB(park_retrieve_blocks, 0.9f, 2, -1.0f, 64, NULL), PARK_ERR_WORKSPACE);
  EXPECT(RB(park_retrieve_blocks_pooled, -0.5f, 2, -1.0f, 64, F), PARK_ERR_INVALID);
  EXPECT(RB(park_retrieve_blocks_pooled, 0.9f, 2, -1.0f, 64, U), PARK_ERR_WORKSPACE);
  EXPECT(park_retrieve_blocks_unfused(F, 1, 1, 2, 256, 128, F, F, 8, 64, 0.9f, 2, -1.0f, NULL, F, F, F, F, F, big,
                                      NULL), PARK_ERR_INVALID);
  EXPECT(park_retrieve_blocks_clustered(F, 1, 1, 2, 256, 128, F, F, 8, NULL, F, 4, 0.9f, 2, -1.0f, F, F, F, F, F,
                                        big, NULL), PARK_ERR_INVALID);
  EXPECT(park_retrieve_blocks_clustered(F, 1, 1, 2, 256, 128, F, F, 8, F, F, 1537, 0.9f, 2, -1.0f, F, F, F, F, F,
                                        big, NULL), PARK_ERR_INVALID);
  EXPECT(park_retrieve_blocks_online(F, 1, 1, 2, 256, 128, F, F, 8, NULL, NULL, 3, 0.9f, 2, -1.0f, F, F, F, F, F,
                                     big, NULL), PARK_ERR_INVALID);
  EXPECT(park_retrieve_blocks_online(F, 1, 1, 2, 256, 128, F, F, 8, F, NULL, 4, 0.9f, 2, -1.0f, F, F, F, F, F, big,
                                     NULL), PARK_ERR_INVALID);
  EXPECT(park_retrieve_blocks_online(F, 1, 1, 2, 256, 128, F, F, 8, NULL, NULL, 4, 0.9f, 2, -1.0f, F, F, F, F, NULL,
                                     big, NULL), PARK_ERR_WORKSPACE);

  /* attention, all variants */
#define AT(V, qb, sc, d, ws, wsb) \
  park_block_sparse_attn(F, F, V, 1, 1, 2, 256, d, F, F, 8, F, F, qb, sc, F, NULL, ws, wsb, NULL)
  EXPECT(AT(NULL, 64, -1.0f, 128, F, big), PARK_ERR_INVALID);
  EXPECT(AT(F, 64, nanf_, 128, F, big), PARK_ERR_INVALID);
  EXPECT(AT(F, 128, -1.0f, 128, F, big), PARK_ERR_UNSUPPORTED);
  EXPECT(AT(F, 64, -1.0f, 32, F, big), PARK_ERR_UNSUPPORTED);
  EXPECT(AT(F, 64, -1.0f, 128, NULL, big), PARK_ERR_WORKSPACE);
  EXPECT(AT(F, 64, -1.0f, 128, F, 100), PARK_ERR_WORKSPACE);
  {
    void* evs[2] = {F, F};
    EXPECT(park_block_sparse_attn_timed(F, F, F, 1, 1, 2, 256, 128, F, F, 8, F, F, 64, -1.0f, F, NULL, NULL, 0, NULL,
                                        evs, evs, 2), PARK_ERR_WORKSPACE);
    EXPECT(park_block_sparse_attn_timed(F, F, F, 1, 1, 2, 256, 128, F, F, 8, F, F, 64, -1.0f, F, NULL, F, big, NULL,
                                        NULL, evs, 1), PARK_ERR_INVALID);
    EXPECT(park_block_sparse_attn_timed(F, F, F, 1, 1, 2, 256, 128, F, F, 8, F, F, 64, -1.0f, F, NULL, F, big, NULL,
                                        evs, evs, -1), PARK_ERR_INVALID);
  }
  /* passes over the heads: at least one for valid sizes, none for rejected ones */
  EXPECT(park_attn_passes(1, 1, 40, 75600, 128, 1024) > 1, 1);
  EXPECT(park_attn_passes(1, 1, 1, 2048, 64, 32), 1);
  EXPECT(park_attn_passes(1, 1 << 20, 1 << 20, 1 << 20, 128, 8), 0);
  EXPECT(park_attn_passes(1, 1, 1, -5, 128, 8), 0);
  EXPECT(park_block_sparse_attn_clustered(F, F, F, 1, 1, 2, 256, 128, F, F, 8, NULL, F, 4, F, F, -1.0f, F, NULL, F,
                                          big, NULL), PARK_ERR_INVALID);
  EXPECT(park_block_sparse_attn_clustered(F, F, F, 1, 1, 2, 256, 128, F, F, 8, F, F, 4, F, F, -1.0f, F, NULL, NULL,
                                          big, NULL), PARK_ERR_WORKSPACE);
  EXPECT(park_block_importance_exact(F, F, 1, 1, 2, 256, 128, F, F, 8, nanf_, F, F, big, NULL), PARK_ERR_INVALID);
  EXPECT(park_logmass_rmse(F, F, 0, 1, 2, 256, 128, F, F, 8, F, F, -1.0f, F, F, big, NULL), PARK_ERR_UNSUPPORTED);

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("sanitized host checks passed\n");
  return 0;
}
