/* A plain C99 caller of the library: include/moe.h compiles as C, the library links, and
 * moe_query answers without a GPU.  Prints the workspace and saved-buffer sizes of the layer
 * given on the command line (T d E k inter n_shared flags) and a rejected configuration's status. */
#include <stdio.h>
#include <stdlib.h>

#include "moe.h"

int main(int argc, char** argv) {
  if (argc != 8) return 2;
  moe_config c = {0};
  c.T = atoi(argv[1]);
  c.d = atoi(argv[2]);
  c.E = atoi(argv[3]);
  c.k = atoi(argv[4]);
  c.inter = atoi(argv[5]);
  c.n_shared = atoi(argv[6]);
  c.flags = (uint32_t)strtoul(argv[7], NULL, 10);
  c.score_fn = MOE_SCORE_SIGMOID;
  size_t ws = 0;
  moe_saved_layout sl;
  moe_workspace_layout wl;
  const moe_status st = moe_query(&c, &ws, &sl, &wl);
  moe_config bad = c;
  bad.d = 100; /* not a multiple of 128 */
  const moe_status st_bad = moe_query(&bad, &ws, NULL, NULL);
  printf("%d %zu %zu %zu %d %s\n", (int)st, ws, sl.total, wl.total, (int)st_bad, moe_strerror(st_bad));
  return st != MOE_OK;
}
