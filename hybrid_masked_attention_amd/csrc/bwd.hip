// Backward of the full- and target-attention layers (in progress).
#include "api_internal.h"

int64_t bwd_ws_bytes(const MetaPlan& p, const mtfm_dims* d, int op) {
  (void)p; (void)d; (void)op;
  return 0;
}

mtfm_status run_full_bwd(const Ctx&, const mtfm_dims*, const mtfm_full_w*, const void*, const void*, void*,
                         const mtfm_full_grad*, char*) {
  return MTFM_E_UNSUPPORTED;
}

mtfm_status run_target_bwd(const Ctx&, const mtfm_dims*, const mtfm_target_w*, const void*, const void*, void*,
                           const mtfm_target_grad*, char*) {
  return MTFM_E_UNSUPPORTED;
}
