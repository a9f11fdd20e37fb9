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
// instead of dbeta - g sum(dbeta)).  The outer gate (gate placement of the
// same pages) keeps LSE_s and the scores; its kernels take it as a template
// argument: no bias on gated blocks, g scales P in P V, in dV and in dZ, and
// the dK/dV kernels record g dg in dbeta's place, so the softmax gate's ds
// epilogue applies.  The hard gate with a straight-through estimator (ranking
// preservation, same section) is composed from the raw gate on zero scores:
// its forward is plain block-sparse attention; its backward takes dq, dk, dv
// from the sparse pass and, from a full-scope pass with the hard LSE_S, the
// gate gradient dh of every history block, which ste_ds_kernel turns into
// ds = g (dh - sum g dh) with g = softmax(s).
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace sas {

hipError_t launch_fwd_simt(const void* q, const void* k, const void* v, const float* scores,
                           const int32_t* idx, void* o, float* lse, float* lse_s, const Dims& d,
                           int topk, float scale, bool bf16, int norm, bool outer, hipStream_t s);
hipError_t launch_bwd_simt(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* scores, const int32_t* idx,
                           const float* lse, const float* lse_s, void* dq, void* dk, void* dv,
                           float* ds, const Dims& d, int topk, float scale, bool bf16, int gate,
                           float* delta, hipStream_t s);

bool fwd_mfma_supported(const Dims& d, int topk, bool sparse);
size_t fwd_mfma_workspace(const Dims& d, int topk, bool sparse);
hipError_t launch_fwd_mfma(const void* q, const void* k, const void* v, const float* scores,
                           const int32_t* idx, void* o, float* lse, float* lse_s, const Dims& d,
                           int topk, float scale, int norm, bool outer, void* ws, hipStream_t s,
                           void* ctx = nullptr, const float* gates = nullptr);

hipError_t launch_fwd_mfma_shared_row(const void* q, const void* k, const void* v, const float* score_row,
                                      const float* lse_s, void* o, float* lse, const Dims& d, float scale,
                                      void* ws, hipStream_t s);

bool bwd_mfma_supported(const Dims& d, int topk, bool sparse);
size_t bwd_mfma_workspace(const Dims& d, int topk, bool sparse);
hipError_t launch_bwd_mfma(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* scores, const int32_t* idx,
                           const float* lse, const float* lse_s, void* dq, void* dk, void* dv,
                           float* ds, const Dims& d, int topk, float scale, int gate, void* ws,
                           hipStream_t s, const void* ctx = nullptr);

namespace {

// log sigmoid(x) = min(x, 0) - log(1 + e^-|x|): no overflow for either sign,
// -inf at -inf, 0 at +inf.  On the hardware exp2 / log2 the result is off by
// about 1e-7 absolute, which is what a logit bias can absorb.
__device__ __forceinline__ float log_sigmoid(float x) {
  return fminf(x, 0.f) - log_hw(1.f + exp_hw(-fabsf(x)));
}

// zero: [rows] <- 0 (LSE_s of a gate without normaliser); sp (sigmoid gate
// only): [n] <- log sigmoid(scores), 16 bytes per access when n % 4 == 0 and
// both arrays are 16-byte aligned.
__global__ __launch_bounds__(256) void gate_prep_kernel(const float* __restrict__ scores, float* __restrict__ sp,
                                                        float* __restrict__ zero, size_t rows, size_t n) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  const size_t tid = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  for (size_t i = tid; i < rows; i += stride) zero[i] = 0.f;
  if (!sp) return;
  if ((n & 3) == 0 && ((reinterpret_cast<uintptr_t>(scores) | reinterpret_cast<uintptr_t>(sp)) & 15) == 0) {
    const float4* s4 = reinterpret_cast<const float4*>(scores);
    float4* o4 = reinterpret_cast<float4*>(sp);
    for (size_t i = tid; i < n / 4; i += stride) {
      const float4 x = s4[i];
      o4[i] = make_float4(log_sigmoid(x.x), log_sigmoid(x.y), log_sigmoid(x.z), log_sigmoid(x.w));
    }
  } else {
    for (size_t i = tid; i < n; i += stride) sp[i] = log_sigmoid(scores[i]);
  }
}

hipError_t launch_gate_prep(const float* scores, float* sp, float* zero, const Dims& d, hipStream_t s) {
  const size_t rows = size_t(d.B) * d.Hq * d.N;
  const size_t n = sp ? rows * size_t(d.C) : 0;
  const size_t work = std::max(rows, (n & 3) == 0 ? n / 4 : n);
  if (work == 0) return hipSuccess;
  const size_t want = (work + 255) / 256;
  const unsigned grid = unsigned(want < 8192 ? want : 8192);
  SAS_LAUNCH("gate_prep", gate_prep_kernel, dim3(grid), dim3(256), 0, s, scores, sp, zero, rows, n);
  return hipGetLastError();
}

size_t rows_of(const Dims& d) { return size_t(d.B) * d.Hq * d.N; }

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, size_t n) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0.f;
}

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const size_t want = (n + 255) / 256;
  SAS_LAUNCH("fill_zero", fill_zero_kernel, dim3(unsigned(want < 8192 ? want : 8192)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

// STE gate, last step: ds holds dh_m (every history block m < c) and becomes
// g (dh - sum_m' g dh) with g = exp(s - LSE_s): the soft gate's Jacobian.
// One wave per row.
__global__ __launch_bounds__(256) void ste_ds_kernel(const float* __restrict__ scores,
                                                     const float* __restrict__ lse_s, float* __restrict__ ds,
                                                     int N, int C, int block, size_t rows) {
  const size_t row = size_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int t = int(row % N);
  const int c = min(t / block, C);
  const float ls = lse_s[row];
  const float* srow = scores + row * C;
  float* drow = ds + row * C;
  float tot = 0.f;
  for (int m = lane; m < c; m += 64) tot += exp_hw(srow[m] - ls) * drow[m];
  for (int off = 32; off >= 1; off >>= 1) tot += shfl_xor(tot, off);
  for (int m = lane; m < C; m += 64) drow[m] = m < c ? exp_hw(srow[m] - ls) * (drow[m] - tot) : 0.f;
}

// STE scratch: zero scores, then (backward) dq, dk, dv of the full-scope pass.
size_t ste_zero_bytes(const Dims& d) { return align_up(rows_of(d) * d.C * sizeof(float)); }
size_t ste_grad_bytes(const Dims& d, bool bf16) {
  const size_t esz = bf16 ? 2 : 4;
  return align_up(rows_of(d) * d.D * esz) + 2 * align_up(size_t(d.B) * d.Hkv * d.N * d.D * esz);
}

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
  if (gate == kGateSoftmax || gate == kGateOuter) return base;
  if (gate == kGateSte) return ste_zero_bytes(d) + fwd_gate_workspace(d, topk, bf16, kGateRaw);
  return align_up(base) + (gate == kGateSigmoid ? align_up(rows_of(d) * d.C * sizeof(float)) : 0);
}

size_t bwd_gate_workspace(const Dims& d, int topk, bool bf16, int gate) {
  const size_t base = bwd_workspace(d, topk, bf16);
  if (gate == kGateSoftmax || gate == kGateOuter) return base;
  if (gate == kGateSte)
    return ste_zero_bytes(d) + ste_grad_bytes(d, bf16) +
           std::max(bwd_gate_workspace(d, topk, bf16, kGateRaw), bwd_gate_workspace(d, -1, bf16, kGateRaw));
  return align_up(base) + (gate == kGateSigmoid ? align_up(rows_of(d) * d.C * sizeof(float)) : 0) +
         align_up(rows_of(d) * sizeof(float));
}

size_t train_ctx_bytes(const Dims& d, int topk, bool bf16) {
  if (topk < 0 || !bf16 || !fwd_mfma_supported(d, topk, true) || !bwd_mfma_supported(d, topk, true)) return 0;
  size_t n = 0;
  sparse_ctx_layout(d, topk, nullptr, &n);
  return n;
}

hipError_t launch_fwd(const void* q, const void* k, const void* v, const float* scores,
                      const int32_t* idx, void* o, float* lse, float* lse_s, const Dims& d,
                      int topk, float scale, bool bf16, int gate, void* ws, hipStream_t s, bool lse_given,
                      void* ctx, const float* gates) {
  if (gate == kGateSte) {
    // the hard gate: plain block-sparse attention (the raw gate on zero
    // scores), then the real LSE_s for the backward's soft gate
    float* zs = static_cast<float*>(ws);
    hipError_t e = launch_fill_zero(zs, rows_of(d) * d.C, s);
    if (e != hipSuccess) return e;
    e = launch_fwd(q, k, v, zs, idx, o, lse, lse_s, d, topk, scale, bf16, kGateRaw,
                   static_cast<char*>(ws) + ste_zero_bytes(d), s);
    if (e != hipSuccess) return e;
    return launch_lse_rows(scores, lse_s, d, s);
  }
  const bool norm = gate == kGateSoftmax || gate == kGateOuter;
  const bool outer = gate == kGateOuter;
  if (!norm) {
    // lse_s <- 0, and the sigmoid gate's scores log sigmoid(s)
    char* extra = static_cast<char*>(ws) + align_up(fwd_workspace(d, idx ? topk : -1, bf16));
    float* sp = gate == kGateSigmoid ? reinterpret_cast<float*>(extra) : nullptr;
    const hipError_t e = launch_gate_prep(scores, sp, lse_s, d, s);
    if (e != hipSuccess) return e;
    if (sp) scores = sp;
  }
  // gate normaliser: 0 none (lse_s holds 0), 1 computed here, 2 given in lse_s
  const int nm = !norm ? 0 : lse_given ? 2 : 1;
  if (bf16 && fwd_mfma_supported(d, topk, idx != nullptr))
    return launch_fwd_mfma(q, k, v, scores, idx, o, lse, lse_s, d, topk, scale, nm, outer, ws, s, ctx, gates);
  return launch_fwd_simt(q, k, v, scores, idx, o, lse, lse_s, d, topk, scale, bf16, nm, outer, s);
}

hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* scores, const int32_t* idx,
                      const float* lse, const float* lse_s, void* dq, void* dk, void* dv,
                      float* ds, const Dims& d, int topk, float scale, bool bf16, int gate, void* ws,
                      hipStream_t s, const void* ctx) {
  if (gate == kGateSte) {
    // dq, dk, dv of the hard gate's attention; then one full-scope pass on
    // zero scores with the hard LSE_S, whose raw-gate ds is dh of every
    // history block; then the soft gate's Jacobian
    char* w = static_cast<char*>(ws);
    float* zs = reinterpret_cast<float*>(w);
    w += ste_zero_bytes(d);
    const size_t esz = bf16 ? 2 : 4;
    void* dq2 = w;
    void* dk2 = w + align_up(rows_of(d) * d.D * esz);
    void* dv2 = static_cast<char*>(dk2) + align_up(size_t(d.B) * d.Hkv * d.N * d.D * esz);
    w += ste_grad_bytes(d, bf16);
    hipError_t e = launch_fill_zero(zs, rows_of(d) * d.C, s);
    if (e == hipSuccess)
      e = launch_bwd(q, k, v, o, dout, zs, idx, lse, nullptr, dq, dk, dv, ds, d, topk, scale, bf16, kGateRaw, w,
                     s);
    if (e == hipSuccess)
      e = launch_bwd(q, k, v, o, dout, zs, nullptr, lse, nullptr, dq2, dk2, dv2, ds, d, 0, scale, bf16, kGateRaw,
                     w, s);
    if (e != hipSuccess) return e;
    const size_t rows = rows_of(d);
    SAS_LAUNCH("ste_ds", ste_ds_kernel, dim3(unsigned((rows + 3) / 4)), dim3(256), 0, s, scores, lse_s, ds, d.N,
               d.C, d.block, rows);
    return hipGetLastError();
  }
  if (gate == kGateSigmoid || gate == kGateRaw) {
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
                           gate, ws, s, gate == kGateSoftmax ? ctx : nullptr);
  float* delta = static_cast<float*>(ws);
  return launch_bwd_simt(q, k, v, o, dout, scores, idx, lse, lse_s, dq, dk, dv, ds, d, topk,
                         scale, bf16, gate, delta, s);
}

// Plain causal attention over N tokens (prefill: no gate; every key at or
// before the row with bias 0): the full-scope raw-gate forward with zero
// scores and a zero LSE_s.  On the matrix cores (bf16, block 64, G in {1, 2,
// 4, 8}, at least one block) every row reads one shared row of C zero scores;
// otherwise the SIMT forward reads a zero [B, Hq, N, C] score tensor.
// Workspace: the forward's own workspace, the zero scores, the zero LSE_s.
size_t fwd_dense_workspace(const Dims& d, bool bf16) {
  const bool mfma = bf16 && fwd_mfma_supported(d, 0, false);
  const size_t own = mfma ? align_up(fwd_mfma_workspace(d, 0, false)) : 0;
  const size_t zs = mfma ? size_t(d.C > 0 ? d.C : 1) : rows_of(d) * size_t(d.C > 0 ? d.C : 1);
  return own + align_up(zs * sizeof(float)) + align_up(rows_of(d) * sizeof(float));
}

hipError_t launch_fwd_dense(const void* q, const void* k, const void* v, void* o, float* lse, const Dims& d,
                            float scale, bool bf16, void* ws, hipStream_t s) {
  if (d.B == 0 || d.Hq == 0 || d.N == 0) return hipSuccess;
  const bool mfma = bf16 && fwd_mfma_supported(d, 0, false);
  char* w = static_cast<char*>(ws);
  const size_t own = mfma ? align_up(fwd_mfma_workspace(d, 0, false)) : 0;
  const size_t nzs = mfma ? size_t(d.C > 0 ? d.C : 1) : rows_of(d) * size_t(d.C > 0 ? d.C : 1);
  float* zs = reinterpret_cast<float*>(w + own);
  float* zl = reinterpret_cast<float*>(w + own + align_up(nzs * sizeof(float)));
  hipError_t e = launch_fill_zero(zs, nzs, s);
  if (e == hipSuccess) e = launch_fill_zero(zl, rows_of(d), s);
  if (e != hipSuccess) return e;
  if (mfma) return launch_fwd_mfma_shared_row(q, k, v, zs, zl, o, lse, d, scale, ws, s);
  return launch_fwd_simt(q, k, v, zs, nullptr, o, lse, zl, d, 0, scale, bf16, 0, false, s);
}

}  // namespace sas
