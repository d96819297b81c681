/* Host-only use of the C ABI from a C11 program (no GPU needed): the header
 * compiles as C, the library links, status strings and workspace queries
 * answer, and invalid calls are rejected before any launch. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "tp_mlp.h"

#define CHECK(c)                                              \
  do {                                                        \
    if (!(c)) {                                               \
      fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      return 1;                                               \
    }                                                         \
  } while (0)

int main(void) {
  CHECK(strcmp(tp_mlp_status_string(TP_MLP_OK), "ok") == 0);
  CHECK(strcmp(tp_mlp_status_string((tp_mlp_status)99), "unknown status") == 0);

  tp_mlp_shape dec = {1, 8192, 28672, 4, 0, TP_MLP_ACT_SWIGLU};
  CHECK(tp_mlp_workspace_bytes(&dec, 0) > 0);                 /* one-token decode: k-split partials */
  tp_mlp_shape big = {2048, 12288, 49152, 8, 0, TP_MLP_ACT_GELU};
  CHECK(tp_mlp_workspace_bytes(&big, 0) == 0);                /* wide tiles: none */
  tp_mlp_shape bad = {4, 64, 130, 4, 0, TP_MLP_ACT_GELU};     /* F % t != 0 */
  CHECK(tp_mlp_workspace_bytes(&bad, 0) == 0);

  void* p = (void*)(uintptr_t)0x7f0000000000ull;              /* never dereferenced */
  CHECK(tp_mlp_fwd_shard(&bad, p, p, NULL, p, p, p, NULL, NULL, NULL, 0, NULL) == TP_MLP_ERR_INVALID_ARG);
  CHECK(tp_mlp_fwd_shard(&dec, p, p, p, p, p, p, NULL, NULL, NULL, 0, NULL) != TP_MLP_OK);
  const void* parts[2] = {p, p};
  CHECK(tp_mlp_reduce_partials_local(2, parts, 4, 12, NULL, p, NULL) == TP_MLP_ERR_INVALID_ARG);

  tp_attn_shape as = {8, 8192, 64, 8, 128, 4, 0};
  CHECK(tp_attn_workspace_bytes(&as) > 0);
  CHECK(tp_sp_layernorm_bwd_workspace_bytes(256, 12288) > 0);
  CHECK(tp_sp_layernorm_bwd_workspace_bytes(4, 12) == 0);
  CHECK(tp_sp_layernorm_fwd(4, 16, 0.0f, p, p, NULL, p, NULL, NULL, NULL) == TP_MLP_ERR_INVALID_ARG);
  puts("c abi ok");
  return 0;
}
