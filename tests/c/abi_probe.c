/* A C client of libqmoe: compiled as strict C99 against include/qmoe.h and linked
 * against the library, it prints the layout of the ABI structs and the status of calls
 * that the library rejects on the host (no GPU is touched). */
#include <stddef.h>
#include <stdio.h>
#include <string.h>

#include "qmoe.h"

int main(void) {
  moe_layer L;
  moe_routing r;
  moe_status s1, s2, s3;
  memset(&L, 0, sizeof L);
  memset(&r, 0, sizeof r);
  printf("sizeof moe_qmatrix %zu\n", sizeof(moe_qmatrix));
  printf("sizeof moe_layer %zu\n", sizeof(moe_layer));
  printf("offsetof moe_layer.shared_gate %zu\n", offsetof(moe_layer, shared_gate));
  printf("offsetof moe_layer.router_w %zu\n", offsetof(moe_layer, router_w));
  printf("sizeof moe_routing %zu\n", sizeof(moe_routing));
  printf("sizeof moe_debug %zu\n", sizeof(moe_debug));
  /* rejected before anything is enqueued */
  s1 = moe_route(NULL, 4, 8, 2, &r, NULL, 0, NULL);          /* no logits */
  s2 = moe_expert_ffn_decode(NULL, NULL, 4, &r, NULL, NULL, 0, NULL, NULL); /* no layer */
  L.d_model = 100; /* not a multiple of 32 */
  s3 = moe_layer_decode(&L, NULL, NULL, 4, &r, NULL, NULL, 0, NULL, NULL);
  printf("status %s %s %s\n", moe_status_string(s1), moe_status_string(s2),
         moe_status_string(s3));
  printf("workspace %zu\n", moe_ffn_workspace_bytes(&L, 4, 0));
  return 0;
}
