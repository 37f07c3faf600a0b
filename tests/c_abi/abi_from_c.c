/* A plain C99 program against include/svgear.h: the header must compile as C
 * and the library must be callable from C. Host side only: it queries sizes
 * and status strings and passes arguments the library refuses before it
 * looks for a device. Exit status 0 on success. */
#include <stdio.h>
#include <string.h>

#include "svgear.h"

static int fails = 0;

static void expect(int cond, const char* what) {
  if (!cond) {
    fprintf(stderr, "FAILED: %s\n", what);
    ++fails;
  }
}

int main(void) {
  expect(strcmp(svgear_status_string(SVGEAR_OK), "ok") == 0, "status string of SVGEAR_OK");
  expect(svgear_cluster_workspace(SVGEAR_BF16, 40, 75600, 128, 500) > 0,
         "workspace of the Wan2.2 key clustering");
  expect(svgear_cluster_workspace(SVGEAR_BF16, 40, 75600, 96, 500) == 0,
         "no workspace for an unsupported head dimension");
  /* null tensors: refused synchronously, nothing enqueued */
  expect(svgear_unpermute(SVGEAR_BF16, 1, 16, 64, NULL, NULL, NULL, NULL) ==
             SVGEAR_ERR_INVALID_ARG,
         "unpermute with null pointers");
  expect(svgear_cluster(SVGEAR_F32, 1, 16, 64, 4, 1, NULL, NULL, NULL, NULL, NULL, 0, NULL) ==
             SVGEAR_ERR_INVALID_ARG,
         "cluster with null pointers");
  if (fails == 0) printf("abi from C: ok\n");
  return fails == 0 ? 0 : 1;
}
