/* A plain C99 client of include/kd_topk_kl.h, built and run by
 * tests/test_c_client.py: the header compiles as C, the library links and
 * its host-side entry points answer without touching a GPU (sizes, the
 * head-gradient grouping, status strings, argument errors). */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kd_topk_kl.h"

int main(void) {
  /* the 32K workload: T = 32768, d = 2880, V = 201088, K = 100, chunk = 2048 */
  const size_t ws = kd_topk_kl_workspace_bytes(32768, 2880, 201088, 100, 2048, KD_BF16);
  const size_t ws_f = kd_topk_kl_fwd_workspace_bytes(32768, 2880, 201088, 100, 2048, KD_BF16);
  const size_t ws_b = kd_topk_kl_bwd_workspace_bytes(32768, 2880, 201088, 100, 2048, KD_BF16);
  const size_t ws_c = kd_topk_cache_workspace_bytes(32768, 2880, 201088, 100, 2048, KD_BF16);
  const int32_t group = kd_topk_kl_dw_chunks(32768, 2880, 201088, 100, 2048, KD_BF16);
  /* the workspace does not grow with T beyond the chunk */
  const size_t ws_long = kd_topk_kl_workspace_bytes(262144, 2880, 201088, 100, 2048, KD_BF16);
  printf("workspace %zu fwd %zu bwd %zu cache %zu group %d same_for_256k %d\n", ws, ws_f, ws_b, ws_c, (int)group,
         ws_long == ws);
  /* invalid shapes size to 0 */
  printf("bad_shape_size %zu\n", kd_topk_kl_workspace_bytes(0, 2880, 201088, 100, 2048, KD_BF16));
  /* argument errors come back before any launch */
  float loss = 0.f;
  const int32_t e_null = kd_topk_kl_fwd_bwd(NULL, NULL, KD_BF16, NULL, NULL, NULL, 16, 64, 128, 4, 1.0f, 8, &loss,
                                            NULL, NULL, NULL, NULL, NULL, 0, NULL, NULL);
  printf("null_args %d %s\n", (int)e_null, kd_status_str(e_null));
  printf("status_ok %s\n", kd_status_str(KD_OK));
  return (ws > 0 && ws_f > 0 && ws_b > 0 && ws_c > 0 && group >= 1 && ws_long == ws && e_null == KD_ERR_NULL_ARG &&
          strcmp(kd_status_str(KD_OK), "ok") == 0)
             ? 0
             : 1;
}
