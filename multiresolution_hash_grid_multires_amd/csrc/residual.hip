// Fused PINN residual step (SIREN decoder on the Hermite encoding).
#include "hashenc.h"
#include "hashenc_internal.h"

extern "C" {

int hashenc_residual_workspace_size(const hashenc* h, const hashenc_mlp* mlp, int64_t n,
                                    size_t* bytes) {
  (void)h; (void)mlp; (void)n;
  if (bytes) *bytes = 0;
  return HASHENC_EUNSUPPORTED;
}

int hashenc_residual(const hashenc* h, const hashenc_mlp* mlp, int64_t n, const float* x,
                     const float* params, const float* mlp_params, float* residual, float* loss,
                     float* grad_params, float* grad_mlp, void* workspace, size_t workspace_bytes,
                     hashenc_stream_t stream) {
  (void)h; (void)mlp; (void)n; (void)x; (void)params; (void)mlp_params; (void)residual;
  (void)loss; (void)grad_params; (void)grad_mlp; (void)workspace; (void)workspace_bytes;
  (void)stream;
  return HASHENC_EUNSUPPORTED;
}

}  // extern "C"
