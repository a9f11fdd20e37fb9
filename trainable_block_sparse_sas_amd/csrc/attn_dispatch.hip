// Dispatch of the gated attention calls to the matrix-core (bf16) or vector
// (fp32) kernels, the workspace each needs, and the gate activations.
//
// Gate activations (blog 方法核心, the ablation table's gate-activation row;
// jaehun.me review "Why the Four Design Choices Matter", gate activation).  The
// kernels add bias = s - LSE_s to a gated block's logits.  The sigmoid gate's
// bias log sigmoid(s) is that bias for the scores s' = log sigmoid(s) and
// LSE_s = 0, the raw logit's bias s for the scores s and LSE_s = 0, so these
// gates run the same kernels on rewritten scores; only the ds epilogues take
// the gate (ds = dbeta (1 - g) with g = e^{s'} = sigmoid(s), or ds = dbeta,
// instead of dbeta - g sum(dbeta)).
#include "common.h"
#include "internal.h"

namespace sas {

hipError_t launch_fwd_simt(const void* q, const void* k, const void* v, const float* scores,
                           const int32_t* idx, void* o, float* lse, float* lse_s, const Dims& d,
                           int topk, float scale, bool bf16, bool norm, hipStream_t s);
hipError_t launch_bwd_simt(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* scores, const int32_t* idx,
                           const float* lse, const float* lse_s, void* dq, void* dk, void* dv,
                           float* ds, const Dims& d, int topk, float scale, bool bf16, int gate,
                           float* delta, hipStream_t s);

bool fwd_mfma_supported(const Dims& d, int topk, bool sparse);
size_t fwd_mfma_workspace(const Dims& d, int topk, bool sparse);
hipError_t launch_fwd_mfma(const void* q, const void* k, const void* v, const float* scores,
                           const int32_t* idx, void* o, float* lse, float* lse_s, const Dims& d,
                           int topk, float scale, bool norm, void* ws, hipStream_t s);

bool bwd_mfma_supported(const Dims& d, int topk, bool sparse);
size_t bwd_mfma_workspace(const Dims& d, int topk, bool sparse);
hipError_t launch_bwd_mfma(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* scores, const int32_t* idx,
                           const float* lse, const float* lse_s, void* dq, void* dk, void* dv,
                           float* ds, const Dims& d, int topk, float scale, int gate, void* ws,
                           hipStream_t s);

namespace {

// log sigmoid(x) = -log(1 + e^-x), without overflow for either sign.
__device__ __forceinline__ float log_sigmoid(float x) {
  return x >= 0.f ? -log1pf(expf(-x)) : x - log1pf(expf(x));
}

// zero: [rows] <- 0 (LSE_s of a gate without normaliser); sp (sigmoid gate
// only): [rows * C] <- log sigmoid(scores).
__global__ __launch_bounds__(256) void gate_prep_kernel(const float* __restrict__ scores, float* __restrict__ sp,
                                                        float* __restrict__ zero, size_t rows, size_t n) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    if (sp) sp[i] = log_sigmoid(scores[i]);
    if (i < rows) zero[i] = 0.f;
  }
}

hipError_t launch_gate_prep(const float* scores, float* sp, float* zero, const Dims& d, hipStream_t s) {
  const size_t rows = size_t(d.B) * d.Hq * d.N;
  const size_t n = sp ? rows * size_t(d.C) : rows;
  if (n == 0) return hipSuccess;
  const size_t want = (n + 255) / 256;
  const unsigned grid = unsigned(want < 65536 ? want : 65536);
  SAS_LAUNCH("gate_prep", gate_prep_kernel, dim3(grid), dim3(256), 0, s, scores, sp, zero, rows, n);
  return hipGetLastError();
}

size_t rows_of(const Dims& d) { return size_t(d.B) * d.Hq * d.N; }

}  // namespace

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

// After the kernels' own workspace: log sigmoid(s) (sigmoid gate), then (the
// backward) a zero LSE_s per row.
size_t fwd_gate_workspace(const Dims& d, int topk, bool bf16, int gate) {
  const size_t base = fwd_workspace(d, topk, bf16);
  if (gate == kGateSoftmax) return base;
  return align_up(base) + (gate == kGateSigmoid ? align_up(rows_of(d) * d.C * sizeof(float)) : 0);
}

size_t bwd_gate_workspace(const Dims& d, int topk, bool bf16, int gate) {
  const size_t base = bwd_workspace(d, topk, bf16);
  if (gate == kGateSoftmax) return base;
  return align_up(base) + (gate == kGateSigmoid ? align_up(rows_of(d) * d.C * sizeof(float)) : 0) +
         align_up(rows_of(d) * sizeof(float));
}

hipError_t launch_fwd(const void* q, const void* k, const void* v, const float* scores,
                      const int32_t* idx, void* o, float* lse, float* lse_s, const Dims& d,
                      int topk, float scale, bool bf16, int gate, void* ws, hipStream_t s) {
  const bool norm = gate == kGateSoftmax;
  if (!norm) {
    // lse_s <- 0, and the sigmoid gate's scores log sigmoid(s)
    char* extra = static_cast<char*>(ws) + align_up(fwd_workspace(d, idx ? topk : -1, bf16));
    float* sp = gate == kGateSigmoid ? reinterpret_cast<float*>(extra) : nullptr;
    const hipError_t e = launch_gate_prep(scores, sp, lse_s, d, s);
    if (e != hipSuccess) return e;
    if (sp) scores = sp;
  }
  if (bf16 && fwd_mfma_supported(d, topk, idx != nullptr))
    return launch_fwd_mfma(q, k, v, scores, idx, o, lse, lse_s, d, topk, scale, norm, ws, s);
  return launch_fwd_simt(q, k, v, scores, idx, o, lse, lse_s, d, topk, scale, bf16, norm, s);
}

hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* scores, const int32_t* idx,
                      const float* lse, const float* lse_s, void* dq, void* dk, void* dv,
                      float* ds, const Dims& d, int topk, float scale, bool bf16, int gate, void* ws,
                      hipStream_t s) {
  if (gate != kGateSoftmax) {
    char* extra = static_cast<char*>(ws) + align_up(bwd_workspace(d, idx ? topk : -1, bf16));
    float* sp = nullptr;
    if (gate == kGateSigmoid) {
      sp = reinterpret_cast<float*>(extra);
      extra += align_up(rows_of(d) * d.C * sizeof(float));
    }
    float* zero = reinterpret_cast<float*>(extra);
    const hipError_t e = launch_gate_prep(scores, sp, zero, d, s);
    if (e != hipSuccess) return e;
    if (sp) scores = sp;
    lse_s = zero;
  }
  if (bf16 && bwd_mfma_supported(d, topk, idx != nullptr))
    return launch_bwd_mfma(q, k, v, o, dout, scores, idx, lse, lse_s, dq, dk, dv, ds, d, topk, scale,
                           gate, ws, s);
  float* delta = static_cast<float*>(ws);
  return launch_bwd_simt(q, k, v, o, dout, scores, idx, lse, lse_s, dq, dk, dv, ds, d, topk,
                         scale, bf16, gate, delta, s);
}

}  // namespace sas
