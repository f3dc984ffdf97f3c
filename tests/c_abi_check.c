/* A plain C99 caller of the library: the header compiles as C, every call it
 * makes links, and host validation answers without a GPU (a batch without
 * cu_seqlens is refused before any launch). */
#include <stdio.h>
#include <string.h>

#include "spec_verify.h"

int main(void) {
  sv_batch b = {2, 4, 8, NULL};
  int32_t result[10];
  sv_status st = spec_accept(&b, SV_ACCEPT_GREEDY, result, NULL, SV_BF16, 10, NULL, NULL,
                             NULL, result, NULL, NULL, NULL, 0, NULL, NULL);
  const char* msg = sv_last_error();
  printf("status %d: %s; version %s\n", (int)st, msg, sv_version());
  if (st != SV_EINVAL || strstr(msg, "cu_seqlens") == NULL) return 1;
  if (spec_verify_flush(-1, NULL, NULL, NULL, NULL) != SV_EINVAL) return 2;
  if (sv_workspace_bytes(0, 4, 32, 128, 1000, 8) != 0) return 3;
  return 0;
}
