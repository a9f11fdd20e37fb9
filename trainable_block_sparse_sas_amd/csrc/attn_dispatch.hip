// Dispatch of the gated attention calls to the matrix-core (bf16) or vector
// (fp32) kernels, and the workspace each needs.
#include "common.h"
#include "internal.h"

namespace sas {

hipError_t launch_fwd_simt(const void* q, const void* k, const void* v, const float* scores,
                           const int32_t* idx, void* o, float* lse, float* lse_s, const Dims& d,
                           int topk, float scale, bool bf16, hipStream_t s);
hipError_t launch_bwd_simt(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* scores, const int32_t* idx,
                           const float* lse, const float* lse_s, void* dq, void* dk, void* dv,
                           float* ds, const Dims& d, int topk, float scale, bool bf16,
                           float* delta, hipStream_t s);

bool fwd_mfma_supported(const Dims& d, int topk, bool sparse);
size_t fwd_mfma_workspace(const Dims& d, int topk, bool sparse);
hipError_t launch_fwd_mfma(const void* q, const void* k, const void* v, const float* scores,
                           const int32_t* idx, void* o, float* lse, float* lse_s, const Dims& d,
                           int topk, float scale, void* ws, hipStream_t s);

bool bwd_mfma_supported(const Dims& d, int topk, bool sparse);
size_t bwd_mfma_workspace(const Dims& d, int topk, bool sparse);
hipError_t launch_bwd_mfma(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* scores, const int32_t* idx,
                           const float* lse, const float* lse_s, void* dq, void* dk, void* dv,
                           float* ds, const Dims& d, int topk, float scale, void* ws,
                           hipStream_t s);

size_t fwd_workspace(const Dims& d, int topk, bool bf16) {
  const bool sparse = topk >= 0;
  if (bf16 && fwd_mfma_supported(d, sparse ? topk : 0, sparse))
    return fwd_mfma_workspace(d, sparse ? topk : 0, sparse);
  return 0;
}

size_t bwd_workspace(const Dims& d, int topk, bool bf16) {
  const bool sparse = topk >= 0;
  if (bf16 && bwd_mfma_supported(d, sparse ? topk : 0, sparse))
    return bwd_mfma_workspace(d, topk, sparse);
  return align_up(size_t(d.B) * d.Hq * d.N * sizeof(float));  // Delta per row
}

hipError_t launch_fwd(const void* q, const void* k, const void* v, const float* scores,
                      const int32_t* idx, void* o, float* lse, float* lse_s, const Dims& d,
                      int topk, float scale, bool bf16, void* ws, hipStream_t s) {
  if (bf16 && fwd_mfma_supported(d, topk, idx != nullptr))
    return launch_fwd_mfma(q, k, v, scores, idx, o, lse, lse_s, d, topk, scale, ws, s);
  return launch_fwd_simt(q, k, v, scores, idx, o, lse, lse_s, d, topk, scale, bf16, s);
}

hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* scores, const int32_t* idx,
                      const float* lse, const float* lse_s, void* dq, void* dk, void* dv,
                      float* ds, const Dims& d, int topk, float scale, bool bf16, void* ws,
                      hipStream_t s) {
  if (bf16 && bwd_mfma_supported(d, topk, idx != nullptr))
    return launch_bwd_mfma(q, k, v, o, dout, scores, idx, lse, lse_s, dq, dk, dv, ds, d, topk, scale,
                           ws, s);
  float* delta = static_cast<float*>(ws);
  return launch_bwd_simt(q, k, v, o, dout, scores, idx, lse, lse_s, dq, dk, dv, ds, d, topk,
                         scale, bf16, delta, s);
}

}  // namespace sas
