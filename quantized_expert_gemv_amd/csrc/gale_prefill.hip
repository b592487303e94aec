// Grouped prefill path (token-sorted, MFMA on signs unpacked in LDS).
#include "gale_internal.h"

namespace gale {

size_t prefill_workspace_bytes(int n_tok, int n_exp, int k, int hidden, int inter) {
  (void)n_tok; (void)n_exp; (void)k; (void)hidden; (void)inter;
  return 256;
}

int run_prefill(int hidden, int inter, const gale_expert* experts, int n_exp, const float* logits, int k,
                const void* x, int n_tok, void* y, int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                hipStream_t s) {
  (void)hidden; (void)inter; (void)experts; (void)n_exp; (void)logits; (void)k; (void)x; (void)n_tok; (void)y;
  (void)topk_idx; (void)topk_w; (void)ws; (void)ws_bytes; (void)s;
  set_error("gale_moe_layer_fwd: grouped prefill path not built yet");
  return GALE_ERR_UNSUPPORTED;
}

}  // namespace gale
