// Host-side launchers behind the C ABI.  Each takes already validated
// arguments and enqueues its kernels on `stream`; it returns hipSuccess or the
// launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sas {

// Kernel timing for diagnostics (sas_profile_enable): while on, every launch
// is bracketed by a pair of HIP events recorded on its stream.
class ProfScope {
 public:
  ProfScope(const char* name, hipStream_t s);
  ~ProfScope();

 private:
  const char* name_;
  hipStream_t s_;
  hipEvent_t a_ = nullptr;
};

#define SAS_LAUNCH(NAME, K, GRID, BLOCK, SHMEM, STREAM, ...)      \
  do {                                                              \
    ::sas::ProfScope sas_prof_scope_(NAME, STREAM);                 \
    hipLaunchKernelGGL(K, GRID, BLOCK, SHMEM, STREAM, __VA_ARGS__); \
  } while (0)

struct Dims {
  int B, Hq, Hkv, N, D, block, C;
  int G() const { return Hq / Hkv; }
};

// Compute units of the current device (persistent-grid sizing).
inline int num_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

// Device workspace carving: 256-byte aligned slices.
inline size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// ---- selector: pooling and scores -------------------------------------------
hipError_t launch_pool(const void* k, void* kbar, int B, int Hkv, int L, int D, int block,
                       int C, bool bf16, hipStream_t s);
// lse_s (optional, not with group_sum): also the softmax gate's LSE_s per row.
// hist_only: the columns m >= c(t) of each row (no history block) are not
// written.
hipError_t launch_score_train(const void* q, const void* kbar, float* scores, const Dims& d,
                              float scale, bool group_sum, bool bf16, hipStream_t s,
                              float* lse_s = nullptr, bool hist_only = false);
// LSE_s of every row over its history scores (any dtype: reads the fp32 scores).
hipError_t launch_lse_rows(const float* scores, float* lse_s, const Dims& d, hipStream_t s);
// table (bf16 only): pooled key m of sequence b is row table[b * C + m] of
// kbar [num_pages, Hkv, D].
hipError_t launch_score_decode(const void* q, const void* kbar, float* scores,
                               const int32_t* cache_len, int B, int Hq, int Hkv, int L, int D,
                               int block, int C, float scale, bool group_sum, bool bf16,
                               hipStream_t s, const int32_t* table = nullptr);
hipError_t launch_pool_pages(const void* k_pages, void* kbar_pages, const int32_t* pages, int n_pages,
                             int Hkv, int D, int block, bool bf16, hipStream_t s);

// ---- Top-K ------------------------------------------------------------------------
// Decode rows clamp cache_len to len_cap (the cache capacity, when known).
// Training Top-K that also writes the selection's base-2 log gates
// (s - LSE_s) log2 e, [rows][topk][hpr] by slot (ascending block order);
// hipErrorNotSupported outside C <= 1024, topk <= 64, hpr in {1, 2, 4, 8}.
hipError_t launch_topk_gated(const float* scores, const float* lse_s, int32_t* idx, float* gates, int B,
                             int Hkv, int hpr, int Nq, int C, int block, int topk, hipStream_t s);
hipError_t launch_topk(const float* scores, int32_t* idx, const int32_t* cache_len, int B,
                       int Hkv, int hpr, int Nq, int C, int block, int topk, hipStream_t s,
                       int len_cap = 0x7fffffff);

// ---- selection lists (key-major sparse kernels) ---------------------------------
// Per KV head, the tokens selecting each history block, ascending; built from
// the Top-K indices by launch_sel_lists into a workspace slice.
struct SelLists {
  uint32_t* bits;    // [pairs * N][MWB] selected-block bitmask per token
  uint16_t* pre;     // [pairs * N][MWB + 1] set bits before each word; [MWB] = count
  uint32_t* cnt;     // [pairs][NB][nseg] tokens of a segment selecting a block
  uint32_t* segoff;  // [pairs][NB][nseg] list offset of (block, segment)
  uint32_t* blkoff;  // [pairs][NB + 1] list offset of each block; [NB] = total
  uint32_t* nitems;  // [pairs] work items
  uint32_t* items;   // [pairs][maxitems][4] {block | own << 31, first entry, end entry, 0}
  uint32_t* ents;    // [pairs][ents_per_pair] token | (slot << 23)
  uint32_t* pos;     // [pairs * N][topk] list position of each (token, slot) entry
  int MWB, NB, nseg, chunk, maxitems, topk;
  size_t ents_per_pair;
};
// base == NULL: sizes only (*bytes).  chunk = tokens per work item.
SelLists sel_lists_layout(int B, int Hkv, int N, int C, int topk, int block, int chunk, char* base,
                          size_t* bytes);
// Optional output of the list build: per (token, slot) and query head of the
// group the base-2 log gate (s - LSE_s) log2 e of the slot's block, read from
// scores [B, Hkv G, N, C] and lse_s [B, Hkv G, N] row by row.
struct SelGates {
  const float* scores;
  const float* lse_s;
  float* out;  // [pairs * N][topk][G]
  int Hkv, G, C;
};
hipError_t launch_sel_lists(const int32_t* idx, const SelLists& L, int B, int Hkv, int N, int C,
                            int topk, int block, hipStream_t s, const SelGates* gates = nullptr);
constexpr int kListChunk = 256;  // list entries per work item of the key-major kernels

// Saved context of a sparse-scope training forward, read by its backward:
// the selection lists of idx, then per (KV head, list entry, query head of the
// group) the base-2 log gate (s - LSE_s) log2 e of that history entry.
struct SparseCtx {
  SelLists L;
  float* lg2;  // [pairs][ents_per_pair][G]
};
// base == NULL: sizes only (*bytes).
SparseCtx sparse_ctx_layout(const Dims& d, int topk, char* base, size_t* bytes);
// Bytes of the saved context a training forward writes for these sizes: the
// layout above where the sparse scope runs on the matrix cores, else 0 (the
// context is not used).
size_t train_ctx_bytes(const Dims& d, int topk, bool bf16);

// ---- gated attention ----------------------------------------------------------
size_t fwd_sel_workspace(const Dims& d, int topk);
hipError_t launch_fwd_sel(const void* q, const void* k, const void* v, const float* scores,
                          const int32_t* idx, void* o, float* lse, const float* lse_s, const Dims& d,
                          int topk, float scale, bool outer, void* ws, hipStream_t s, void* ctx = nullptr,
                          const float* gates = nullptr);
size_t fwd_workspace(const Dims& d, int topk, bool bf16);
size_t bwd_workspace(const Dims& d, int topk, bool bf16);
size_t fwd_gate_workspace(const Dims& d, int topk, bool bf16, int gate);
size_t bwd_gate_workspace(const Dims& d, int topk, bool bf16, int gate);
// lse_given (softmax gate only): lse_s already holds LSE_s; it is read, not
// computed.  ctx (sparse scope on the matrix cores; else unused): the saved
// context for the backward (sparse_ctx_layout) is written.  gates (same
// scope): the selection's log gates from launch_topk_gated, read instead of
// the scores' selected entries.
hipError_t launch_fwd(const void* q, const void* k, const void* v, const float* scores,
                      const int32_t* idx, void* o, float* lse, float* lse_s, const Dims& d,
                      int topk, float scale, bool bf16, int gate, void* ws, hipStream_t s,
                      bool lse_given = false, void* ctx = nullptr, const float* gates = nullptr);
// ctx (softmax gate, sparse scope on the matrix cores; else unused): the
// saved context the forward wrote; the selection lists are not rebuilt.
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* scores, const int32_t* idx,
                      const float* lse, const float* lse_s, void* dq, void* dk, void* dv,
                      float* ds, const Dims& d, int topk, float scale, bool bf16, int gate, void* ws,
                      hipStream_t s, const void* ctx = nullptr);

// ---- decode --------------------------------------------------------------------
size_t selector_bwd_workspace(const Dims& d, bool bf16);
hipError_t launch_selector_bwd(const void* q, const void* kbar, const float* ds, void* dq, void* dk,
                               float* dkbar, const Dims& d, float scale, bool accumulate, bool bf16,
                               void* ws, hipStream_t s);
size_t decode_workspace(int B, int Hq, int Hkv, int L_max, int D, int block, int topk);
// table (bf16 only): block m of sequence b is page table[b * (L_max / block) + m]
// of kc, vc [num_pages, Hkv, block, D].
hipError_t launch_decode(const void* q, const void* kc, const void* vc, const int32_t* cache_len,
                         const int32_t* idx, void* o, float* lse, int B, int Hq, int Hkv,
                         int L_max, int D, int block, int topk, float scale, bool bf16, void* ws,
                         hipStream_t s, const int32_t* table = nullptr);

// ---- prefill into a paged cache ----------------------------------------------------
// Plain causal attention (no gate) over N tokens: the full-scope forward on
// zero scores (see attn_dispatch.hip).
size_t fwd_dense_workspace(const Dims& d, bool bf16);
hipError_t launch_fwd_dense(const void* q, const void* k, const void* v, void* o, float* lse, const Dims& d,
                            float scale, bool bf16, void* ws, hipStream_t s);
// Rows t < seq_len[b] of k, v [B, Hkv, N, D] into the pages of their blocks
// (table [B, max_blocks]); complete blocks' pooled keys into kbar_pages.
hipError_t launch_prefill_pages(const void* k, const void* v, const int32_t* seq_len, const int32_t* table,
                                void* k_pages, void* v_pages, void* kbar_pages, int B, int Hkv, int N, int D,
                                int block, int max_blocks, bool bf16, hipStream_t s);

// ---- allocation-free decode ----------------------------------------------------
// Size of the per-GPU scratch array behind sas_sparse_decode_noalloc.
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
// Device address of the current device's scratch array (looked up once per
// device with hipGetSymbolAddress, then cached).
hipError_t noalloc_scratch(void** ptr);

}  // namespace sas
