/* Host-only use of libdion3.so from plain C99: the header compiles as C and
 * the host entry points behave as documented (no device work is done). */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "dion3.h"

#define EXPECT(c)                                                   \
  do {                                                              \
    if (!(c)) {                                                     \
      fprintf(stderr, "%s:%d: failed: %s\n", __FILE__, __LINE__, #c); \
      return 1;                                                     \
    }                                                               \
  } while (0)

int main(void) {
  dion3_ns_cfg cfg;
  size_t bytes = 0, bytes4 = 0;
  dion3_norm_cfg bad = {1.0f, 1e-8f};
  char fake[512];
  void* ws = (void*)(((size_t)fake + 255) & ~(size_t)255);   /* aligned, never dereferenced */

  EXPECT(dion3_version() >= 1);
  EXPECT(dion3_ns_cfg_size() == sizeof(dion3_ns_cfg));
  dion3_ns_cfg_default(&cfg);
  EXPECT(cfg.iters == 5 && cfg.n_restart == 1 && cfg.restart_at[0] == 3);
  EXPECT(cfg.method == DION3_NS_GRAM && cfg.path == DION3_PATH_AUTO);
  EXPECT(fabsf(cfg.abc[0][0] - 3.4445f) < 1e-6f);

  EXPECT(dion3_k_from_fraction(0.25, 128) == 32);
  EXPECT(dion3_k_from_fraction(0.07, 100) == 7);
  EXPECT(dion3_k_from_fraction(0.0, 10) == -1);

  EXPECT(dion3_workspace_size(1, 128, 512, 32, &bytes) == DION3_OK && bytes > 0);
  EXPECT(dion3_workspace_size(4, 128, 512, 32, &bytes4) == DION3_OK && bytes4 > 3 * bytes);
  EXPECT(dion3_workspace_size(1, 10, 10, 11, &bytes) == DION3_ERR_ARG);
  EXPECT(dion3_workspace_size(1, 0, 10, 1, &bytes) == DION3_ERR_ARG);
  EXPECT(dion3_workspace_size(1, 10, 10, 0, &bytes) == DION3_ERR_ARG);
  EXPECT(dion3_workspace_size(1, (1 << 20) + 1, 10, 0, &bytes) == DION3_ERR_ARG);
  EXPECT(dion3_workspace_size(1, (1 << 20) + 1, 10, 1, &bytes) == DION3_ERR_UNSUPPORTED);
  EXPECT(dion3_step((float*)ws, (float*)ws, 64, 32, 32, 0, 0.04f, 0.95f, NULL, NULL, NULL, ws,
                    1u << 30, NULL) == DION3_ERR_ARG);
  EXPECT(dion3_step((float*)ws, (float*)ws, 64, 32, 32, 65, 0.04f, 0.95f, NULL, NULL, NULL, ws,
                    1u << 30, NULL) == DION3_ERR_ARG);

  /* argument errors are reported before any launch */
  EXPECT(dion3_step(NULL, NULL, 64, 32, 32, 16, 0.04f, 0.95f, NULL, NULL, NULL, ws, 1u << 30,
                    NULL) == DION3_ERR_ARG);
  cfg.iters = 0;
  EXPECT(dion3_step((float*)ws, (float*)ws, 64, 32, 32, 16, 0.04f, 0.95f, &cfg, NULL, NULL, ws,
                    1u << 30, NULL) == DION3_ERR_ARG);
  EXPECT(dion3_step_megabatch_norm((float* const*)ws, (float* const*)ws, NULL, (float* const*)ws, 1,
                                   64, 32, 32, 16, 0.04f, 0.95f, NULL, &bad, NULL, NULL, ws,
                                   1u << 30, NULL) == DION3_ERR_ARG);
  EXPECT(strlen(dion3_status_string(DION3_ERR_WORKSPACE)) > 0);
  printf("c abi ok\n");
  return 0;
}
