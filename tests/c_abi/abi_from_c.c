/* A C program against include/ragattn.h and libragattn.so: the header is
 * valid C (and C++), the library links and its validation answers without a
 * GPU. Each line printed is "<status> <message>" or a size. An ra_dtype
 * outside the enumerators is passed as a C caller may. */
#include <stdio.h>

#include "ragattn.h"

int main(void) {
  ra_status st = ra_merge_states(NULL, NULL, 0, 4, 128, RA_BF16, NULL, NULL, NULL);
  printf("%d %s\n", (int)st, ra_last_error());
  st = ra_tree_attn(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, 0, 0, 0, 8, 8, 128,
                    (ra_dtype)7, 0, 1.0f, 1e4f, 0.1f, NULL);
  printf("%d %s\n", (int)st, ra_last_error());
  st = ra_set_workgroup_waves(0);
  printf("%d %s\n", (int)st, ra_last_error());
  printf("%zu\n", ra_paged_attn_split_workspace(16, 32, 128, 4));
  return 0;
}
