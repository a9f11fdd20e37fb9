// C ABI of libsas: argument validation on the host, then dispatch to the
// kernel launchers.  Nothing here touches the GPU before every check passed.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/sas.h"
#include "internal.h"

namespace {

thread_local std::string g_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SAS_EHIP, "%s: HIP error %d (%s)", what, int(e), hipGetErrorString(e));
  g_error.clear();
  return SAS_OK;
}

constexpr int kMaxTopk = 256;
constexpr int kMaxBlocks = 16384;
constexpr int kMaxGroupDecode = 16;

int check_common(int B, int Hq, int Hkv, int n, int D, int block, int dtype, const char* what) {
  if (B < 0 || Hq < 0 || Hkv < 1 || n < 0)
    return fail(SAS_EINVAL, "%s: sizes must be non-negative and Hkv >= 1 (B=%d Hq=%d Hkv=%d N=%d)",
                what, B, Hq, Hkv, n);
  if (Hq % Hkv != 0) return fail(SAS_EINVAL, "%s: Hq (%d) must be a multiple of Hkv (%d)", what, Hq, Hkv);
  if (block < 1) return fail(SAS_EINVAL, "%s: block must be >= 1 (got %d)", what, block);
  if (dtype != SAS_F32 && dtype != SAS_BF16) return fail(SAS_EINVAL, "%s: unknown dtype %d", what, dtype);
  if (D != 64 && D != 128) return fail(SAS_EUNSUPPORTED, "%s: head dim %d not supported (64 or 128)", what, D);
  return SAS_OK;
}

bool empty(int B, int Hq, int n) { return B == 0 || Hq == 0 || n == 0; }

// Paged decode workspace: group-summed scores, the selected blocks, the
// attention partials.
struct PagedWs {
  size_t scores, idx, part, total;
};
PagedWs paged_ws(int B, int Hq, int Hkv, int L_max, int D, int block, int topk) {
  PagedWs w{};
  const size_t C = size_t(L_max / block);
  w.scores = 0;
  w.idx = sas::align_up(size_t(B) * Hkv * C * sizeof(float));
  w.part = w.idx + sas::align_up(size_t(B) * Hkv * size_t(topk > 0 ? topk : 1) * sizeof(int32_t));
  w.total = w.part + sas::decode_workspace(B, Hq, Hkv, L_max, D, block, topk);
  return w;
}

// The logit scale must be a positive finite number (the kernels take the row
// maximum of the raw scores, which is the maximum of the scaled ones only for
// a positive scale).
int check_scale(float scale, const char* what) {
  if (!(scale > 0.f) || !(scale < __builtin_huge_valf()))
    return fail(SAS_EINVAL, "%s: scale must be positive and finite (got %g)", what, double(scale));
  return SAS_OK;
}

// One decode step (scores, Top-K, attention, merge) over contiguous caches
// (table == NULL) or pages: the group-summed scores land at the start of the
// workspace, lengths are clamped to L_max before Top-K.
hipError_t decode_chain(const void* q, const void* kbar, const void* kc, const void* vc, const int32_t* cache_len,
                        const int32_t* table, int topk, void* o, float* lse, int32_t* idx_out, int B, int Hq,
                        int Hkv, int L_max, int D, int block, float scale, bool bf16, void* workspace,
                        hipStream_t s) {
  const PagedWs W = paged_ws(B, Hq, Hkv, L_max, D, block, topk);
  const int C = L_max / block;
  char* w = static_cast<char*>(workspace);
  float* scores = reinterpret_cast<float*>(w + W.scores);
  int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(w + W.idx);
  hipError_t e = sas::launch_score_decode(q, kbar, scores, cache_len, B, Hq, Hkv, L_max, D, block, C, scale, true,
                                          bf16, s, table);
  if (e == hipSuccess && topk > 0) e = sas::launch_topk(scores, idx, cache_len, B, Hkv, 1, 1, C, block, topk, s, L_max);
  if (e == hipSuccess)
    e = sas::launch_decode(q, kc, vc, cache_len, idx, o, lse, B, Hq, Hkv, L_max, D, block, topk, scale, bf16,
                           w + W.part, s, table);
  return e;
}

}  // namespace

extern "C" {

const char* sas_last_error(void) { return g_error.c_str(); }

int sas_abi_version(void) { return 106; }

size_t sas_workspace_bytes(int op, int B, int Hq, int Hkv, int n, int D, int block, int topk,
                           int dtype) {
  if (B < 0 || Hq < 0 || Hkv < 1 || n < 0 || block < 1 || (Hq % Hkv) != 0) return size_t(-1);
  sas::Dims d{B, Hq, Hkv, n, D, block, n / block};
  const bool bf16 = dtype == SAS_BF16;
  switch (op) {
    case SAS_OP_SCORE:
    case SAS_OP_TOPK:
      return 0;
    case SAS_OP_FWD:
      return sas::fwd_workspace(d, topk, bf16);
    case SAS_OP_BWD:
      return sas::bwd_workspace(d, topk, bf16);
    case SAS_OP_DECODE:
      return sas::decode_workspace(B, Hq, Hkv, n, D, block, topk);
    case SAS_OP_SELECTOR_BWD:
      if (D != 64 && D != 128) return size_t(-1);
      return sas::selector_bwd_workspace(d, bf16);
    case SAS_OP_PREFILL:
      if (D != 64 && D != 128) return size_t(-1);
      return sas::fwd_dense_workspace(d, bf16) + sas::align_up(size_t(B) * Hq * n * sizeof(float));
    case SAS_OP_PAGED_DECODE:
    case SAS_OP_DECODE_STEP:
      if (topk < 0) return size_t(-1);
      return paged_ws(B, Hq, Hkv, n, D, block, topk).total;
    case SAS_OP_FWD_GATE:
      return std::max(sas::fwd_gate_workspace(d, topk, bf16, SAS_GATE_SIGMOID),
                      sas::fwd_gate_workspace(d, topk, bf16, SAS_GATE_STE));
    case SAS_OP_BWD_GATE:
      return std::max(sas::bwd_gate_workspace(d, topk, bf16, SAS_GATE_SIGMOID),
                      sas::bwd_gate_workspace(d, topk, bf16, SAS_GATE_STE));
    case SAS_OP_CTX:
      return sas::train_ctx_bytes(d, topk, bf16);
    default:
      return size_t(-1);
  }
}

int sas_score_blocks(const void* q, const void* k, void* kbar, float* scores,
                     const int32_t* cache_len, int B, int Hq, int Hkv, int Nq, int L, int D,
                     int block, float scale, int group_sum, int dtype, void* stream) {
  int st = check_common(B, Hq, Hkv, L, D, block, dtype, "sas_score_blocks");
  if (!st) st = check_scale(scale, "sas_score_blocks");
  if (st) return st;
  if (Nq < 0) return fail(SAS_EINVAL, "sas_score_blocks: Nq must be >= 0");
  const int C = L / block;
  if (cache_len) {
    if (Nq != 1 && !(B == 0 || Hq == 0)) return fail(SAS_EINVAL, "sas_score_blocks: decode mode needs Nq == 1 (got %d)", Nq);
    if (Hq / Hkv > kMaxGroupDecode)
      return fail(SAS_EUNSUPPORTED, "sas_score_blocks: at most %d query heads per KV head in decode mode", kMaxGroupDecode);
  } else if (Nq != L) {
    return fail(SAS_EINVAL, "sas_score_blocks: training mode needs Nq == L (got Nq=%d L=%d)", Nq, L);
  }
  if (empty(B, Hq, Nq) && !(k && B > 0 && C > 0)) {
    g_error.clear();
    return SAS_OK;
  }
  if (!q || !kbar || !scores) return fail(SAS_EINVAL, "sas_score_blocks: q, kbar and scores must be non-NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = dtype == SAS_BF16;
  if (k) {
    hipError_t e = sas::launch_pool(k, kbar, B, Hkv, L, D, block, C, bf16, s);
    if (e != hipSuccess) return hip_status(e, "sas_score_blocks (pool)");
  }
  if (empty(B, Hq, Nq)) return hip_status(hipSuccess, "");
  hipError_t e;
  if (cache_len) {
    e = sas::launch_score_decode(q, kbar, scores, cache_len, B, Hq, Hkv, L, D, block, C, scale,
                                 group_sum != 0, bf16, s);
  } else {
    sas::Dims d{B, Hq, Hkv, L, D, block, C};
    e = sas::launch_score_train(q, kbar, scores, d, scale, group_sum != 0, bf16, s);
  }
  return hip_status(e, "sas_score_blocks");
}

int sas_score_blocks_lse(const void* q, const void* k, void* kbar, float* scores, float* lse_s, int B,
                         int Hq, int Hkv, int N, int D, int block, float scale, int dtype, void* stream) {
  const char* what = "sas_score_blocks_lse";
  int st = check_common(B, Hq, Hkv, N, D, block, dtype, what);
  if (!st) st = check_scale(scale, what);
  if (st) return st;
  const int C = N / block;
  if (empty(B, Hq, N) && !(k && B > 0 && C > 0)) {
    g_error.clear();
    return SAS_OK;
  }
  if (!q || !kbar || !scores || !lse_s) return fail(SAS_EINVAL, "%s: q, kbar, scores and lse_s must be non-NULL", what);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = dtype == SAS_BF16;
  if (k) {
    hipError_t e = sas::launch_pool(k, kbar, B, Hkv, N, D, block, C, bf16, s);
    if (e != hipSuccess) return hip_status(e, "sas_score_blocks_lse (pool)");
  }
  if (empty(B, Hq, N)) return hip_status(hipSuccess, "");
  sas::Dims d{B, Hq, Hkv, N, D, block, C};
  return hip_status(sas::launch_score_train(q, kbar, scores, d, scale, false, bf16, s, lse_s, true), what);
}

int sas_topk_select(const float* scores, int32_t* idx, const int32_t* cache_len, int B, int Hkv,
                    int heads_per_row, int Nq, int C, int block, int topk, void* workspace,
                    size_t workspace_bytes, void* stream) {
  (void)workspace;  // Top-K needs no scratch; the arguments are kept for ABI stability
  (void)workspace_bytes;
  if (B < 0 || Hkv < 1 || Nq < 0 || C < 0)
    return fail(SAS_EINVAL, "sas_topk_select: invalid sizes (B=%d Hkv=%d Nq=%d C=%d)", B, Hkv, Nq, C);
  if (heads_per_row < 1) return fail(SAS_EINVAL, "sas_topk_select: heads_per_row must be >= 1");
  if (block < 1) return fail(SAS_EINVAL, "sas_topk_select: block must be >= 1");
  if (topk < 0) return fail(SAS_EINVAL, "sas_topk_select: topk must be >= 0");
  if (topk > kMaxTopk) return fail(SAS_EUNSUPPORTED, "sas_topk_select: topk %d > %d", topk, kMaxTopk);
  if (C > kMaxBlocks) return fail(SAS_EUNSUPPORTED, "sas_topk_select: C %d > %d", C, kMaxBlocks);
  if (cache_len && Nq != 1 && B > 0) return fail(SAS_EINVAL, "sas_topk_select: decode rows need Nq == 1");
  if (B == 0 || Nq == 0 || topk == 0) {
    g_error.clear();
    return SAS_OK;
  }
  if (!scores || !idx) return fail(SAS_EINVAL, "sas_topk_select: scores and idx must be non-NULL");
  hipError_t e = sas::launch_topk(scores, idx, cache_len, B, Hkv, heads_per_row, Nq, C, block, topk,
                                  static_cast<hipStream_t>(stream));
  return hip_status(e, "sas_topk_select");
}

int sas_topk_select_gated(const float* scores, const float* lse_s, int32_t* idx, float* gates, int B,
                          int Hkv, int heads_per_row, int Nq, int C, int block, int topk, void* stream) {
  if (B < 0 || Hkv < 1 || Nq < 0 || C < 0)
    return fail(SAS_EINVAL, "sas_topk_select_gated: invalid sizes (B=%d Hkv=%d Nq=%d C=%d)", B, Hkv, Nq, C);
  if (heads_per_row < 1) return fail(SAS_EINVAL, "sas_topk_select_gated: heads_per_row must be >= 1");
  if (block < 1) return fail(SAS_EINVAL, "sas_topk_select_gated: block must be >= 1");
  if (topk < 0) return fail(SAS_EINVAL, "sas_topk_select_gated: topk must be >= 0");
  const int h = heads_per_row;
  if (C > 1024 || topk > 64 || (h != 1 && h != 2 && h != 4 && h != 8))
    return fail(SAS_EUNSUPPORTED, "sas_topk_select_gated: needs C <= 1024, topk <= 64, heads_per_row 1, 2, 4 or 8 "
                "(C=%d topk=%d heads_per_row=%d)", C, topk, heads_per_row);
  if (B == 0 || Nq == 0 || topk == 0) {
    g_error.clear();
    return SAS_OK;
  }
  if (!scores || !lse_s || !idx || !gates)
    return fail(SAS_EINVAL, "sas_topk_select_gated: scores, lse_s, idx and gates must be non-NULL");
  hipError_t e = sas::launch_topk_gated(scores, lse_s, idx, gates, B, Hkv, heads_per_row, Nq, C, block, topk,
                                        static_cast<hipStream_t>(stream));
  return hip_status(e, "sas_topk_select_gated");
}

static int check_attn(const char* what, int B, int Hq, int Hkv, int N, int D, int block,
                      const int32_t* idx, int topk, int dtype) {
  int st = check_common(B, Hq, Hkv, N, D, block, dtype, what);
  if (st) return st;
  if (idx) {
    if (topk < 0) return fail(SAS_EINVAL, "%s: topk must be >= 0 with idx", what);
    if (topk > kMaxTopk) return fail(SAS_EUNSUPPORTED, "%s: topk %d > %d", what, topk, kMaxTopk);
    if (N / block > kMaxBlocks) return fail(SAS_EUNSUPPORTED, "%s: sparse scope with more than %d blocks", what, kMaxBlocks);
  }
  return SAS_OK;
}

constexpr size_t kNoCtx = size_t(-1);  // ctx_bytes of the calls without a saved context

static int attn_fwd(const char* what, const void* q, const void* k, const void* v, const float* scores,
                    const int32_t* idx, void* o, float* lse, float* lse_s, int B, int Hq, int Hkv, int N,
                    int D, int block, int topk, float scale, int dtype, int gate, void* workspace,
                    size_t workspace_bytes, void* stream, bool lse_given = false, void* ctx = nullptr,
                    size_t ctx_bytes = kNoCtx, const float* gates = nullptr) {
  int st = check_attn(what, B, Hq, Hkv, N, D, block, idx, topk, dtype);
  if (!st) st = check_scale(scale, what);
  if (st) return st;
  if (gate < SAS_GATE_SOFTMAX || gate > SAS_GATE_STE) return fail(SAS_EINVAL, "%s: unknown gate %d", what, gate);
  if (empty(B, Hq, N)) {
    g_error.clear();
    return SAS_OK;
  }
  if (!q || !k || !v || !scores || !o || !lse || !lse_s)
    return fail(SAS_EINVAL, "%s: q, k, v, scores, o, lse, lse_s must be non-NULL", what);
  sas::Dims d{B, Hq, Hkv, N, D, block, N / block};
  const bool bf16 = dtype == SAS_BF16;
  const size_t need = sas::fwd_gate_workspace(d, idx ? topk : -1, bf16, gate);
  if (need && (!workspace || workspace_bytes < need))
    return fail(SAS_EWORKSPACE, "%s: workspace of %zu bytes required (got %zu)", what, need, workspace_bytes);
  if (ctx_bytes != kNoCtx) {  // a call with a saved context
    const size_t cneed = sas::train_ctx_bytes(d, idx ? topk : -1, bf16);
    if (cneed && (!ctx || ctx_bytes < cneed))
      return fail(SAS_EWORKSPACE, "%s: saved context of %zu bytes required (got %zu)", what, cneed, ctx_bytes);
    if (!cneed) ctx = nullptr;
  }
  if (gates && !idx) return fail(SAS_EINVAL, "%s: gates are the log gates of a selection (idx required)", what);
  hipError_t e = sas::launch_fwd(q, k, v, scores, idx, o, lse, lse_s, d, idx ? topk : 0, scale,
                                 bf16, gate, workspace, static_cast<hipStream_t>(stream), lse_given, ctx, gates);
  return hip_status(e, what);
}

static int attn_bwd(const char* what, const void* q, const void* k, const void* v, const void* o,
                    const void* dout, const float* scores, const int32_t* idx, const float* lse,
                    const float* lse_s, void* dq, void* dk, void* dv, float* ds, int B, int Hq, int Hkv,
                    int N, int D, int block, int topk, float scale, int dtype, int gate, void* workspace,
                    size_t workspace_bytes, void* stream, const void* ctx = nullptr,
                    size_t ctx_bytes = kNoCtx) {
  int st = check_attn(what, B, Hq, Hkv, N, D, block, idx, topk, dtype);
  if (!st) st = check_scale(scale, what);
  if (st) return st;
  if (gate < SAS_GATE_SOFTMAX || gate > SAS_GATE_STE) return fail(SAS_EINVAL, "%s: unknown gate %d", what, gate);
  if (empty(B, Hq, N)) {
    g_error.clear();
    return SAS_OK;
  }
  const bool needs_lse_s = gate == SAS_GATE_SOFTMAX || gate == SAS_GATE_OUTER || gate == SAS_GATE_STE;
  if (!q || !k || !v || !o || !dout || !scores || !lse || (!lse_s && needs_lse_s) || !dq ||
      !dk || !dv || !ds)
    return fail(SAS_EINVAL, "%s: every tensor pointer except idx (and lse_s for the sigmoid and raw gates) must be non-NULL",
                what);
  sas::Dims d{B, Hq, Hkv, N, D, block, N / block};
  const bool bf16 = dtype == SAS_BF16;
  const size_t need = sas::bwd_gate_workspace(d, idx ? topk : -1, bf16, gate);
  if (need && (!workspace || workspace_bytes < need))
    return fail(SAS_EWORKSPACE, "%s: workspace of %zu bytes required (got %zu)", what, need, workspace_bytes);
  if (ctx_bytes != kNoCtx) {  // a call with a saved context
    const size_t cneed = sas::train_ctx_bytes(d, idx ? topk : -1, bf16);
    if (cneed && (!ctx || ctx_bytes < cneed))
      return fail(SAS_EWORKSPACE, "%s: saved context of %zu bytes required (got %zu)", what, cneed, ctx_bytes);
    if (!cneed) ctx = nullptr;
  }
  hipError_t e = sas::launch_bwd(q, k, v, o, dout, scores, idx, lse, lse_s, dq, dk, dv, ds, d,
                                 idx ? topk : 0, scale, bf16, gate, workspace,
                                 static_cast<hipStream_t>(stream), ctx);
  return hip_status(e, what);
}

int sas_gated_attn_fwd(const void* q, const void* k, const void* v, const float* scores,
                       const int32_t* idx, void* o, float* lse, float* lse_s, int B, int Hq,
                       int Hkv, int N, int D, int block, int topk, float scale, int dtype,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return attn_fwd("sas_gated_attn_fwd", q, k, v, scores, idx, o, lse, lse_s, B, Hq, Hkv, N, D, block, topk,
                  scale, dtype, SAS_GATE_SOFTMAX, workspace, workspace_bytes, stream);
}

int sas_gated_attn_fwd_lse(const void* q, const void* k, const void* v, const float* scores,
                           const int32_t* idx, const float* lse_s, void* o, float* lse, int B, int Hq,
                           int Hkv, int N, int D, int block, int topk, float scale, int dtype,
                           void* workspace, size_t workspace_bytes, void* stream) {
  // lse_s is only read (the kernels take it through the same pointer they
  // would otherwise write it through)
  return attn_fwd("sas_gated_attn_fwd_lse", q, k, v, scores, idx, o, lse, const_cast<float*>(lse_s), B, Hq,
                  Hkv, N, D, block, topk, scale, dtype, SAS_GATE_SOFTMAX, workspace, workspace_bytes, stream,
                  true);
}

int sas_gated_attn_fwd_ctx(const void* q, const void* k, const void* v, const float* scores,
                           const int32_t* idx, const float* lse_s, const float* gates, void* o, float* lse,
                           int B, int Hq, int Hkv, int N, int D, int block, int topk, float scale, int dtype,
                           void* ctx, size_t ctx_bytes, void* workspace, size_t workspace_bytes, void* stream) {
  return attn_fwd("sas_gated_attn_fwd_ctx", q, k, v, scores, idx, o, lse, const_cast<float*>(lse_s), B, Hq,
                  Hkv, N, D, block, topk, scale, dtype, SAS_GATE_SOFTMAX, workspace, workspace_bytes, stream,
                  true, ctx, ctx_bytes, gates);
}

int sas_gated_attn_fwd_gate(const void* q, const void* k, const void* v, const float* scores,
                            const int32_t* idx, void* o, float* lse, float* lse_s, int B, int Hq,
                            int Hkv, int N, int D, int block, int topk, float scale, int dtype, int gate,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return attn_fwd("sas_gated_attn_fwd_gate", q, k, v, scores, idx, o, lse, lse_s, B, Hq, Hkv, N, D, block,
                  topk, scale, dtype, gate, workspace, workspace_bytes, stream);
}

int sas_gated_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* scores, const int32_t* idx,
                       const float* lse, const float* lse_s, void* dq, void* dk, void* dv,
                       float* ds, int B, int Hq, int Hkv, int N, int D, int block, int topk,
                       float scale, int dtype, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return attn_bwd("sas_gated_attn_bwd", q, k, v, o, dout, scores, idx, lse, lse_s, dq, dk, dv, ds, B, Hq,
                  Hkv, N, D, block, topk, scale, dtype, SAS_GATE_SOFTMAX, workspace, workspace_bytes, stream);
}

int sas_gated_attn_bwd_ctx(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* scores, const int32_t* idx,
                           const float* lse, const float* lse_s, const void* ctx, size_t ctx_bytes,
                           void* dq, void* dk, void* dv, float* ds, int B, int Hq, int Hkv, int N, int D,
                           int block, int topk, float scale, int dtype, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return attn_bwd("sas_gated_attn_bwd_ctx", q, k, v, o, dout, scores, idx, lse, lse_s, dq, dk, dv, ds, B, Hq,
                  Hkv, N, D, block, topk, scale, dtype, SAS_GATE_SOFTMAX, workspace, workspace_bytes, stream,
                  ctx, ctx_bytes);
}

int sas_gated_attn_bwd_gate(const void* q, const void* k, const void* v, const void* o,
                            const void* dout, const float* scores, const int32_t* idx,
                            const float* lse, const float* lse_s, void* dq, void* dk, void* dv,
                            float* ds, int B, int Hq, int Hkv, int N, int D, int block, int topk,
                            float scale, int dtype, int gate, void* workspace, size_t workspace_bytes,
                            void* stream) {
  return attn_bwd("sas_gated_attn_bwd_gate", q, k, v, o, dout, scores, idx, lse, lse_s, dq, dk, dv, ds, B,
                  Hq, Hkv, N, D, block, topk, scale, dtype, gate, workspace, workspace_bytes, stream);
}

// Checks shared by the two sparse-decode calls.  Returns SAS_OK with *noop set
// when there is nothing to do.
static int check_decode(const char* what, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* cache_len, const int32_t* idx, const void* o, int B, int Hq,
                        int Hkv, int L_max, int D, int block, int topk, float scale, int dtype, bool* noop) {
  *noop = false;
  int st = check_common(B, Hq, Hkv, L_max, D, block, dtype, what);
  if (!st) st = check_scale(scale, what);
  if (st) return st;
  if (Hkv > 0 && Hq / Hkv > kMaxGroupDecode)
    return fail(SAS_EUNSUPPORTED, "%s: at most %d query heads per KV head", what, kMaxGroupDecode);
  if (idx && topk < 0) return fail(SAS_EINVAL, "%s: topk must be >= 0 with idx", what);
  if (idx && topk > kMaxTopk) return fail(SAS_EUNSUPPORTED, "%s: topk %d > %d", what, topk, kMaxTopk);
  if (B == 0 || Hq == 0) {
    g_error.clear();
    *noop = true;
    return SAS_OK;
  }
  if (!q || !k_cache || !v_cache || !cache_len || !o)
    return fail(SAS_EINVAL, "%s: q, caches, cache_len and o must be non-NULL", what);
  return SAS_OK;
}

int sas_sparse_decode(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* cache_len, const int32_t* idx, void* o, float* lse, int B,
                      int Hq, int Hkv, int L_max, int D, int block, int topk, float scale,
                      int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  bool noop = false;
  int st = check_decode("sas_sparse_decode", q, k_cache, v_cache, cache_len, idx, o, B, Hq, Hkv, L_max, D,
                        block, topk, scale, dtype, &noop);
  if (st || noop) return st;
  const size_t need = sas::decode_workspace(B, Hq, Hkv, L_max, D, block, idx ? topk : -1);
  if (!workspace || workspace_bytes < need)
    return fail(SAS_EWORKSPACE, "sas_sparse_decode: workspace of %zu bytes required (got %zu)", need, workspace_bytes);
  hipError_t e = sas::launch_decode(q, k_cache, v_cache, cache_len, idx, o, lse, B, Hq, Hkv, L_max,
                                    D, block, idx ? topk : -1, scale, dtype == SAS_BF16, workspace,
                                    static_cast<hipStream_t>(stream));
  return hip_status(e, "sas_sparse_decode");
}

int sas_sparse_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* cache_len, const int32_t* idx, void* o, float* lse,
                              int B, int Hq, int Hkv, int L_max, int D, int block, int topk,
                              float scale, int dtype, void* stream) {
  bool noop = false;
  int st = check_decode("sas_sparse_decode_noalloc", q, k_cache, v_cache, cache_len, idx, o, B, Hq, Hkv,
                        L_max, D, block, topk, scale, dtype, &noop);
  if (st || noop) return st;
  const size_t need = sas::decode_workspace(B, Hq, Hkv, L_max, D, block, idx ? topk : -1);
  if (need > sas::kNoAllocScratchBytes)
    return fail(SAS_EUNSUPPORTED,
                "sas_sparse_decode_noalloc: these sizes need %zu bytes of scratch, more than the %zu bytes "
                "the allocation-free call holds per GPU (use sas_sparse_decode with a workspace)",
                need, sas::kNoAllocScratchBytes);
  void* scratch_ptr = nullptr;
  hipError_t e = sas::noalloc_scratch(&scratch_ptr);
  if (e != hipSuccess) return hip_status(e, "sas_sparse_decode_noalloc (scratch address)");
  e = sas::launch_decode(q, k_cache, v_cache, cache_len, idx, o, lse, B, Hq, Hkv, L_max, D, block,
                         idx ? topk : -1, scale, dtype == SAS_BF16, scratch_ptr, static_cast<hipStream_t>(stream));
  return hip_status(e, "sas_sparse_decode_noalloc");
}

int sas_pool_pages(const void* k_pages, void* kbar_pages, const int32_t* pages, int n_pages, int Hkv,
                   int D, int block, int dtype, void* stream) {
  int st = check_common(1, Hkv, Hkv, 0, D, block, dtype, "sas_pool_pages");
  if (st) return st;
  if (n_pages < 0) return fail(SAS_EINVAL, "sas_pool_pages: n_pages must be >= 0");
  if (n_pages == 0) {
    g_error.clear();
    return SAS_OK;
  }
  if (!k_pages || !kbar_pages || !pages)
    return fail(SAS_EINVAL, "sas_pool_pages: k_pages, kbar_pages and pages must be non-NULL");
  hipError_t e = sas::launch_pool_pages(k_pages, kbar_pages, pages, n_pages, Hkv, D, block, dtype == SAS_BF16,
                                        static_cast<hipStream_t>(stream));
  return hip_status(e, "sas_pool_pages");
}

int sas_paged_decode(const void* q, const void* k_pages, const void* v_pages, const void* kbar_pages,
                     const int32_t* block_table, int max_blocks, const int32_t* cache_len, int topk,
                     void* o, float* lse, int32_t* idx_out, int B, int Hq, int Hkv, int D, int block,
                     float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (max_blocks < 0 || block < 1) return fail(SAS_EINVAL, "sas_paged_decode: max_blocks >= 0 and block >= 1 required");
  if (max_blocks > kMaxBlocks) return fail(SAS_EUNSUPPORTED, "sas_paged_decode: max_blocks %d > %d", max_blocks, kMaxBlocks);
  if (size_t(max_blocks) * size_t(block) > size_t(0x7fffffff))
    return fail(SAS_EINVAL, "sas_paged_decode: max_blocks * block too large");
  const int L_max = max_blocks * block;
  int st = check_common(B, Hq, Hkv, L_max, D, block, dtype, "sas_paged_decode");
  if (!st) st = check_scale(scale, "sas_paged_decode");
  if (st) return st;
  if (dtype != SAS_BF16) return fail(SAS_EUNSUPPORTED, "sas_paged_decode: bf16 only");
  if (Hq / Hkv > kMaxGroupDecode)
    return fail(SAS_EUNSUPPORTED, "sas_paged_decode: at most %d query heads per KV head", kMaxGroupDecode);
  if (topk < 0) return fail(SAS_EINVAL, "sas_paged_decode: topk must be >= 0");
  if (topk > kMaxTopk) return fail(SAS_EUNSUPPORTED, "sas_paged_decode: topk %d > %d", topk, kMaxTopk);
  if (B == 0 || Hq == 0 || max_blocks == 0) {
    g_error.clear();
    return SAS_OK;
  }
  if (!q || !k_pages || !v_pages || !kbar_pages || !block_table || !cache_len || !o)
    return fail(SAS_EINVAL, "sas_paged_decode: q, pages, pooled keys, block_table, cache_len and o must be non-NULL");
  const PagedWs W = paged_ws(B, Hq, Hkv, L_max, D, block, topk);
  if (!workspace || workspace_bytes < W.total)
    return fail(SAS_EWORKSPACE, "sas_paged_decode: workspace of %zu bytes required (got %zu)", W.total, workspace_bytes);
  hipError_t e = decode_chain(q, kbar_pages, k_pages, v_pages, cache_len, block_table, topk, o, lse, idx_out, B, Hq,
                              Hkv, L_max, D, block, scale, true, workspace, static_cast<hipStream_t>(stream));
  return hip_status(e, "sas_paged_decode");
}

int sas_decode_step(const void* q, const void* kbar, const void* k_cache, const void* v_cache,
                    const int32_t* cache_len, int topk, void* o, float* lse, int32_t* idx_out, int B, int Hq,
                    int Hkv, int L_max, int D, int block, float scale, int dtype, void* workspace,
                    size_t workspace_bytes, void* stream) {
  int st = check_common(B, Hq, Hkv, L_max, D, block, dtype, "sas_decode_step");
  if (!st) st = check_scale(scale, "sas_decode_step");
  if (st) return st;
  if (Hq / Hkv > kMaxGroupDecode)
    return fail(SAS_EUNSUPPORTED, "sas_decode_step: at most %d query heads per KV head", kMaxGroupDecode);
  if (topk < 0) return fail(SAS_EINVAL, "sas_decode_step: topk must be >= 0");
  if (topk > kMaxTopk) return fail(SAS_EUNSUPPORTED, "sas_decode_step: topk %d > %d", topk, kMaxTopk);
  if (L_max / block > kMaxBlocks)
    return fail(SAS_EUNSUPPORTED, "sas_decode_step: %d blocks > %d", L_max / block, kMaxBlocks);
  if (B == 0 || Hq == 0) {
    g_error.clear();
    return SAS_OK;
  }
  if (!q || !kbar || !k_cache || !v_cache || !cache_len || !o)
    return fail(SAS_EINVAL, "sas_decode_step: q, kbar, caches, cache_len and o must be non-NULL");
  const PagedWs W = paged_ws(B, Hq, Hkv, L_max, D, block, topk);
  if (!workspace || workspace_bytes < W.total)
    return fail(SAS_EWORKSPACE, "sas_decode_step: workspace of %zu bytes required (got %zu)", W.total, workspace_bytes);
  hipError_t e = decode_chain(q, kbar, k_cache, v_cache, cache_len, nullptr, topk, o, lse, idx_out, B, Hq, Hkv,
                              L_max, D, block, scale, dtype == SAS_BF16, workspace, static_cast<hipStream_t>(stream));
  return hip_status(e, "sas_decode_step");
}

int sas_prefill_paged(const void* q, const void* k, const void* v, const int32_t* seq_len, void* o, float* lse,
                      void* k_pages, void* v_pages, void* kbar_pages, const int32_t* block_table, int max_blocks,
                      int B, int Hq, int Hkv, int N, int D, int block, float scale, int dtype, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int st = check_common(B, Hq, Hkv, N, D, block, dtype, "sas_prefill_paged");
  if (!st) st = check_scale(scale, "sas_prefill_paged");
  if (st) return st;
  if (max_blocks < 0) return fail(SAS_EINVAL, "sas_prefill_paged: max_blocks must be >= 0");
  if (size_t(N) > size_t(max_blocks) * size_t(block))
    return fail(SAS_EINVAL, "sas_prefill_paged: N (%d) exceeds the table's capacity max_blocks * block (%d * %d)", N,
                max_blocks, block);
  if (empty(B, Hq, N)) {
    g_error.clear();
    return SAS_OK;
  }
  if (!q || !k || !v || !seq_len || !o || !k_pages || !v_pages || !kbar_pages || !block_table)
    return fail(SAS_EINVAL, "sas_prefill_paged: every pointer except lse must be non-NULL");
  sas::Dims d{B, Hq, Hkv, N, D, block, N / block};
  const bool bf16 = dtype == SAS_BF16;
  const size_t fws = sas::fwd_dense_workspace(d, bf16);
  const size_t need = fws + (lse ? 0 : sas::align_up(size_t(B) * Hq * N * sizeof(float)));
  if (!workspace || workspace_bytes < need)
    return fail(SAS_EWORKSPACE, "sas_prefill_paged: workspace of %zu bytes required (got %zu)", need, workspace_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* lse_out = lse ? lse : reinterpret_cast<float*>(static_cast<char*>(workspace) + fws);
  hipError_t e = sas::launch_prefill_pages(k, v, seq_len, block_table, k_pages, v_pages, kbar_pages, B, Hkv, N, D,
                                           block, max_blocks, bf16, s);
  if (e == hipSuccess) e = sas::launch_fwd_dense(q, k, v, o, lse_out, d, scale, bf16, workspace, s);
  return hip_status(e, "sas_prefill_paged");
}

int sas_selector_bwd(const void* q, const void* kbar, const float* ds, void* dq, void* dk,
                     float* dkbar, int B, int Hq, int Hkv, int N, int D, int block, float scale,
                     int accumulate, int dtype, void* workspace, size_t workspace_bytes,
                     void* stream) {
  int st = check_common(B, Hq, Hkv, N, D, block, dtype, "sas_selector_bwd");
  if (!st) st = check_scale(scale, "sas_selector_bwd");
  if (st) return st;
  if (accumulate != 0 && accumulate != 1)
    return fail(SAS_EINVAL, "sas_selector_bwd: accumulate must be 0 or 1 (got %d)", accumulate);
  if (empty(B, Hq, N)) {
    g_error.clear();
    return SAS_OK;
  }
  if (!q || !kbar || !ds || !dq || !dk)
    return fail(SAS_EINVAL, "sas_selector_bwd: q, kbar, ds, dq and dk must be non-NULL");
  sas::Dims d{B, Hq, Hkv, N, D, block, N / block};
  const bool bf16 = dtype == SAS_BF16;
  const size_t need = sas::selector_bwd_workspace(d, bf16);
  if (need && (!workspace || workspace_bytes < need))
    return fail(SAS_EWORKSPACE, "sas_selector_bwd: workspace of %zu bytes required (got %zu)", need, workspace_bytes);
  hipError_t e = sas::launch_selector_bwd(q, kbar, ds, dq, dk, dkbar, d, scale, accumulate != 0, bf16, workspace,
                                          static_cast<hipStream_t>(stream));
  return hip_status(e, "sas_selector_bwd");
}

}  // extern "C"
