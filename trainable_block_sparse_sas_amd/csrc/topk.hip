// Hard Top-K block selection (jaehun.me review, "Background", paper Eq. 3;
// "A Concrete Walkthrough", Step 3 and Step 6).
//
// Per row (one query token and one KV head) the candidates are the history
// blocks m < c.  The group score is the fp32 sum of the row's head scores in
// head-index order.  Exactly min(K, c) blocks are kept, ordered by score
// descending with ties to the lower block index (-0.0 == +0.0, NaN == -inf).
//
// Rows of up to 1024 candidates (and long rows with K > 64) use an MSB-first
// radix select over the order-preserving uint32 key: it finds the K-th largest
// key T in four 8-bit passes (LDS histogram), every key > T is kept and the
// keys equal to T are taken in index order; only the K survivors are then
// ranked, by counting.  Long rows with K <= 64 (decode) merge sorted runs in
// registers instead, with no histogram passes and no atomics.
#include "common.h"
#include "internal.h"
#include "runs.h"

namespace sas {
namespace {

constexpr int kMaxTopk = 256;

// Candidates of a row: the history blocks m < c.  Training rows: c = t / block.
// Decode rows: the query sits at len - 1 with len clamped to len_cap (the
// cache capacity when the caller knows it), c = (len - 1) / block, none for an
// idle sequence.  Never more than C.
__device__ __forceinline__ int row_candidates(const int32_t* __restrict__ cache_len, int b, long t,
                                              int block, int C, int len_cap) {
  int c;
  if (cache_len) {
    int len = cache_len[b];
    len = len < len_cap ? len : len_cap;
    c = len > 0 ? (len - 1) / block : 0;
  } else {
    c = int(t / block);
  }
  return c < C ? c : C;
}

// Group score of each of the lane's PER candidates m[i] (where ok[i]): the sum
// of the row's hpr head scores, hstride floats apart, added in head order.
// Every load of a chunk of HC heads is issued before the first add, so a row
// costs one memory round trip per chunk rather than one per head.  From 8
// candidates a lane on, a chunk is one head: the registers the loads would
// hold cost more occupancy than the round trips (rows of 512 candidates and
// 4 heads: 0.38 ms at one head per chunk, 0.41 ms at four).
template <int PER>
__device__ __forceinline__ void group_sum(const float* __restrict__ row0, size_t hstride, int hpr,
                                          const int (&m)[PER], const bool (&ok)[PER], float (&u)[PER]) {
  constexpr int HC = PER <= 4 ? 4 : 1;
#pragma unroll
  for (int i = 0; i < PER; ++i) u[i] = 0.f;
  for (int h0 = 0; h0 < hpr; h0 += HC) {
    float v[HC][PER];
#pragma unroll
    for (int j = 0; j < HC; ++j)
#pragma unroll
      for (int i = 0; i < PER; ++i)
        v[j][i] = (h0 + j < hpr && ok[i]) ? row0[size_t(h0 + j) * hstride + m[i]] : 0.f;
#pragma unroll
    for (int j = 0; j < HC; ++j)
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (h0 + j < hpr) u[i] = h0 + j == 0 ? v[j][i] : u[i] + v[j][i];
  }
}

// WPR waves cooperate on one row; PER lanes-slots per lane (c <= 64*WPR*PER).
template <int WPR, int PER>
__global__ __launch_bounds__(256 * (WPR > 4 ? 4 : 1)) void topk_kernel(
    const float* __restrict__ scores, int32_t* __restrict__ idx,
    const int32_t* __restrict__ cache_len, int Hkv, int hpr, int Nq, int C, int block, int topk,
    int len_cap, long total_rows) {
  constexpr int WAVES = (WPR > 4 ? 16 : 4);
  constexpr int ROWS = WAVES / WPR;  // rows per workgroup
  __shared__ uint32_t hist[ROWS][256];
  __shared__ uint32_t sel_key[ROWS][kMaxTopk];
  __shared__ int32_t sel_m[ROWS][kMaxTopk];
  __shared__ uint32_t cnt[ROWS][PER][WPR];
  __shared__ uint32_t bcast[ROWS][2];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rw = wave / WPR;        // row slot in the workgroup
  const int wr = wave % WPR;        // wave index within the row
  const long row = long(blockIdx.x) * ROWS + rw;
  const bool active = row < total_rows;

  int c = 0, K = 0;
  long t = 0, bg = 0;
  if (active) {
    t = row % Nq;
    bg = row / Nq;
    const int b = int(bg / Hkv);
    c = row_candidates(cache_len, b, t, block, C, len_cap);
    K = topk < c ? topk : c;
  }
  // Load the group-summed scores as order-preserving keys.
  uint32_t key[PER];
  bool valid[PER];
  {
    const int g = int(bg % Hkv);
    const int b = int(bg / Hkv);
    int m[PER];
    float u[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      m[i] = (i * WPR + wr) * 64 + lane;
      valid[i] = active && m[i] < c;
    }
    group_sum<PER>(scores + ((size_t(b) * Hkv + g) * hpr * size_t(Nq) + t) * C, size_t(Nq) * C, hpr, m,
                   valid, u);
#pragma unroll
    for (int i = 0; i < PER; ++i) key[i] = valid[i] ? score_key(u[i]) : 0u;
  }
  // Radix select of the K-th largest key.
  uint32_t prefix = 0;
  int need = K;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = threadIdx.x % (64 * WPR); i < 256; i += 64 * WPR) hist[rw][i] = 0;
    __syncthreads();
    if (need > 0) {
      for (int i = 0; i < PER; ++i) {
        const bool match = valid[i] && (pass == 0 || (key[i] >> (shift + 8)) == (prefix >> (shift + 8)));
        if (match) atomicAdd(&hist[rw][(key[i] >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    if (wr == 0 && need > 0) {
      // lane l owns buckets 4l .. 4l+3; suffix sums from the top bucket down.
      uint32_t h4[4];
      for (int j = 0; j < 4; ++j) h4[j] = hist[rw][4 * lane + j];
      uint32_t local = h4[0] + h4[1] + h4[2] + h4[3];
      uint32_t suffix = local;  // inclusive suffix over lanes >= l
      for (int off = 1; off < 64; off <<= 1) {
        uint32_t o = __shfl_down(suffix, off, 64);
        if (lane + off < 64) suffix += o;
      }
      const unsigned long long ball = __ballot(suffix >= uint32_t(need));
      const int L = 63 - __builtin_clzll(ball);  // highest lane whose suffix reaches need
      if (lane == L) {
        uint32_t above = suffix - local;  // keys in lanes > L
        int digit = 4 * L;
        for (int j = 3; j >= 0; --j) {
          if (above + h4[j] >= uint32_t(need)) {
            digit = 4 * L + j;
            break;
          }
          above += h4[j];
        }
        bcast[rw][0] = prefix | (uint32_t(digit) << shift);
        bcast[rw][1] = uint32_t(need) - above;
      }
    }
    __syncthreads();
    if (need > 0) {
      prefix = bcast[rw][0];
      need = int(bcast[rw][1]);
    }
  }
  const uint32_t T = prefix;  // K-th largest key; `need` keys equal to T are taken
  // Select: keys > T, and the first `need` keys == T in block order.
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  bool take[PER];
  for (int i = 0; i < PER; ++i) {
    const bool eq = K > 0 && valid[i] && key[i] == T;
    const unsigned long long be = __ballot(eq);
    if (lane == 0) cnt[rw][i][wr] = __popcll(be);
    take[i] = eq;  // provisional, refined below
  }
  __syncthreads();
  {
    uint32_t before = 0;
    for (int i = 0; i < PER; ++i) {
      const unsigned long long be = __ballot(take[i]);
      uint32_t preceding_waves = 0;
      for (int w = 0; w < wr; ++w) preceding_waves += cnt[rw][i][w];
      const uint32_t rank = before + preceding_waves + __popcll(be & lt);
      take[i] = (K > 0 && valid[i] && key[i] > T) || (take[i] && rank < uint32_t(need));
      for (int w = 0; w < WPR; ++w) before += cnt[rw][i][w];
    }
  }
  __syncthreads();
  // Compact the survivors into LDS (block order), reusing cnt for the counts.
  for (int i = 0; i < PER; ++i) {
    const unsigned long long bt = __ballot(take[i]);
    if (lane == 0) cnt[rw][i][wr] = __popcll(bt);
  }
  __syncthreads();
  {
    uint32_t before = 0;
    for (int i = 0; i < PER; ++i) {
      const unsigned long long bt = __ballot(take[i]);
      uint32_t pw = 0;
      for (int w = 0; w < wr; ++w) pw += cnt[rw][i][w];
      if (take[i]) {
        const uint32_t pos = before + pw + __popcll(bt & lt);
        sel_key[rw][pos] = key[i];
        sel_m[rw][pos] = (i * WPR + wr) * 64 + lane;
      }
      for (int w = 0; w < WPR; ++w) before += cnt[rw][i][w];
    }
  }
  __syncthreads();
  // Rank the K survivors (score descending, block ascending) and write the row.
  if (active) {
    int32_t* out = idx + size_t(row) * topk;
    for (int e = threadIdx.x % (64 * WPR); e < topk; e += 64 * WPR) {
      if (e >= K) {
        out[e] = -1;
        continue;
      }
      const uint32_t ke = sel_key[rw][e];
      const int me = sel_m[rw][e];
      int slot = 0;
      for (int f = 0; f < K; ++f) {
        const uint32_t kf = sel_key[rw][f];
        slot += (kf > ke) || (kf == ke && sel_m[rw][f] < me);
      }
      out[slot] = me;
    }
  }
}

// ---- long rows (decode: thousands of candidates per row) ----------------------
// Composite key (hi, lo) = (order-preserving score key, ~block index): all
// distinct, and larger means "score higher, or equal score and lower index".

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Marks in `take` the K largest composite keys among the wave's valid
// candidates (PER per lane; fewer valid than K: all of them).  MSB-first radix
// select over 8-bit digits of hi then lo with a histogram private to the wave
// (256 LDS counters); stops as soon as the tied candidates are exactly the
// number still needed.
template <int PER>
__device__ void wave_select(const uint32_t (&hi)[PER], const uint32_t (&lo)[PER],
                            const bool (&valid)[PER], int K, uint32_t* hist, bool (&take)[PER]) {
  const int lane = threadIdx.x & 63;
  bool tied[PER];
  int nvalid = 0;
  for (int i = 0; i < PER; ++i) {
    take[i] = false;
    tied[i] = valid[i];
    nvalid += __popcll(__ballot(valid[i]));
  }
  int need = K < nvalid ? K : nvalid;
  if (need == nvalid) {  // everything valid is taken
    for (int i = 0; i < PER; ++i) take[i] = valid[i];
    return;
  }
  for (int pass = 0; pass < 8 && need > 0; ++pass) {
    const int shift = 24 - 8 * (pass & 3);
    for (int j = lane; j < 256; j += 64) hist[j] = 0;
    wave_sync();
    uint32_t dig[PER];
    for (int i = 0; i < PER; ++i) {
      dig[i] = (((pass < 4) ? hi[i] : lo[i]) >> shift) & 255u;
      if (tied[i]) atomicAdd(&hist[dig[i]], 1u);
    }
    wave_sync();
    uint32_t h4[4];
    for (int j = 0; j < 4; ++j) h4[j] = hist[4 * lane + j];
    const uint32_t local = h4[0] + h4[1] + h4[2] + h4[3];
    uint32_t suffix = local;
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_down(suffix, off, 64);
      if (lane + off < 64) suffix += o;
    }
    const unsigned long long ball = __ballot(suffix >= uint32_t(need));
    const int L = 63 - __builtin_clzll(ball);
    uint32_t digit = 0, above = 0, cnt = 0;
    if (lane == L) {
      above = suffix - local;
      for (int j = 3; j >= 0; --j) {
        if (above + h4[j] >= uint32_t(need)) {
          digit = 4 * L + j;
          cnt = h4[j];
          break;
        }
        above += h4[j];
      }
    }
    digit = __shfl(digit, L, 64);
    above = __shfl(above, L, 64);
    cnt = __shfl(cnt, L, 64);
    wave_sync();
    for (int i = 0; i < PER; ++i) {
      if (!tied[i]) continue;
      if (dig[i] > digit) {
        take[i] = true;
        tied[i] = false;
      } else if (dig[i] < digit) {
        tied[i] = false;
      }
    }
    need -= int(above);
    if (int(cnt) == need) {
      for (int i = 0; i < PER; ++i)
        if (tied[i]) take[i] = true;
      need = 0;
    }
  }
}

// One row per workgroup of 16 waves.  Stage 1: wave w selects the top K of its
// candidates m = (i*16 + w)*64 + lane.  Stage 2: wave 0 selects the top K of
// the 16 survivor lists.  The K winners are then ranked by counting.
template <int PER, int PER2>
__global__ __launch_bounds__(1024) void topk_long_kernel(const float* __restrict__ scores,
                                                         int32_t* __restrict__ idx,
                                                         const int32_t* __restrict__ cache_len,
                                                         int Hkv, int hpr, int Nq, int C, int block,
                                                         int topk, int len_cap) {
  __shared__ uint32_t hist[16][256];
  __shared__ uint32_t cand_hi[16][kMaxTopk];
  __shared__ uint32_t cand_lo[16][kMaxTopk];
  __shared__ int cand_n[16];
  __shared__ uint32_t fin_hi[kMaxTopk], fin_lo[kMaxTopk];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const long row = blockIdx.x;
  const long t = row % Nq, bg = row / Nq;
  const int b = int(bg / Hkv), g = int(bg % Hkv);
  const int c = row_candidates(cache_len, b, t, block, C, len_cap);
  const int K = topk < c ? topk : c;
  const unsigned long long lt = lane ? (~0ull >> (64 - lane)) : 0ull;

  uint32_t hi[PER], lo[PER];
  bool valid[PER], take[PER];
  {
    int m[PER];
    float u[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      m[i] = (i * 16 + w) * 64 + lane;
      valid[i] = m[i] < c;
      lo[i] = ~uint32_t(m[i]);
    }
    group_sum<PER>(scores + ((size_t(b) * Hkv + g) * hpr * size_t(Nq) + t) * C, size_t(Nq) * C, hpr, m,
                   valid, u);
#pragma unroll
    for (int i = 0; i < PER; ++i) hi[i] = valid[i] ? score_key(u[i]) : 0u;
  }
  if (K > 0) wave_select<PER>(hi, lo, valid, K, hist[w], take);
  else
    for (int i = 0; i < PER; ++i) take[i] = false;
  int n = 0;
  for (int i = 0; i < PER; ++i) {
    const unsigned long long bt = __ballot(take[i]);
    if (take[i]) {
      const int pos = n + __popcll(bt & lt);
      cand_hi[w][pos] = hi[i];
      cand_lo[w][pos] = lo[i];
    }
    n += __popcll(bt);
  }
  if (lane == 0) cand_n[w] = n;
  __syncthreads();
  if (w == 0 && K > 0) {
    int off[16];
    int tot = 0;
    for (int v = 0; v < 16; ++v) {
      off[v] = tot;
      tot += cand_n[v];
    }
    uint32_t h2[PER2], l2[PER2];
    bool v2[PER2], t2[PER2];
    for (int i = 0; i < PER2; ++i) {
      const int e = i * 64 + lane;
      v2[i] = e < tot;
      h2[i] = 0;
      l2[i] = 0;
      if (v2[i]) {
        int src = 0;
        while (src < 15 && e >= off[src + 1]) ++src;
        h2[i] = cand_hi[src][e - off[src]];
        l2[i] = cand_lo[src][e - off[src]];
      }
    }
    wave_select<PER2>(h2, l2, v2, K, hist[0], t2);
    int nn = 0;
    for (int i = 0; i < PER2; ++i) {
      const unsigned long long bt = __ballot(t2[i]);
      if (t2[i]) {
        const int pos = nn + __popcll(bt & lt);
        fin_hi[pos] = h2[i];
        fin_lo[pos] = l2[i];
      }
      nn += __popcll(bt);
    }
  }
  __syncthreads();
  int32_t* out = idx + size_t(row) * topk;
  for (int e = threadIdx.x; e < topk; e += 1024) {
    if (e >= K) {
      out[e] = -1;
      continue;
    }
    const uint32_t he = fin_hi[e], le = fin_lo[e];
    int slot = 0;
    for (int f = 0; f < K; ++f) slot += (fin_hi[f] > he) || (fin_hi[f] == he && fin_lo[f] > le);
    out[slot] = int(~le);
  }
}

// ---- long rows, K <= 64: sorted runs merged in registers --------------------
// One row per workgroup of W waves.  Each lane sorts its PER composite keys
// (score key << 32 | ~block: all distinct, larger = higher score, ties to the
// lower block; an invalid candidate is 0) descending with a bitonic network,
// keeps its best E = min(PER, KP) and groups of R = KP / E lanes build sorted
// runs of KP keys (element q E + r of a run: lane q of the group, register r).
// Two sorted runs A and B reduce to the KP largest keys of their union by
// max(A[j], B[KP - 1 - j]), a bitonic sequence that the half-cleaners sort
// again; both partner groups compute it (one sees the sequence reversed,
// which sorts to the same run), so after log2(64 / R) rounds every group of
// the wave holds the wave's best KP keys.  The W wave runs are merged the
// same way through LDS.  The final run is the answer in rank order.

// A filter runs first.  Take each lane's largest score key (32-bit, the score
// alone): if tau is the K-th largest of these lane maxima, K lanes hold a key
// whose score key is >= tau, so the K-th largest key and everything above it
// has a score key >= tau, and every key below is out.  With random scores the
// survivors are barely more than K; when they fit one wave (at most 64) each
// survivor's rank is counted directly.  Otherwise (many equal scores) the
// whole row goes through the run merge above.
template <int PER, int KP, int W>
__global__ __launch_bounds__(64 * W) void topk_runs_kernel(const float* __restrict__ scores,
                                                         int32_t* __restrict__ idx,
                                                         const int32_t* __restrict__ cache_len,
                                                         int Hkv, int hpr, int Nq, int C, int block,
                                                         int topk, int len_cap) {
  constexpr int E = PER < KP ? PER : KP;  // keys per lane in a run
  constexpr int R = KP / E;               // lanes per run
  constexpr int E1 = KP <= 8 ? 1 : KP / 8;  // filter: 32-bit runs of KP as E1 x R1
  constexpr int R1 = KP / E1;
  static_assert(R <= 32 && (KP & (KP - 1)) == 0 && (PER & (PER - 1)) == 0, "run shape");
  __shared__ uint64_t runs[2][W][KP];
  __shared__ uint32_t fruns[2][W][KP];
  __shared__ uint64_t surv[64];
  __shared__ uint32_t rank[64];
  __shared__ int wcnt[W];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const long row = blockIdx.x;
  const long t = row % Nq, bg = row / Nq;
  const int b = int(bg / Hkv), g = int(bg % Hkv);
  // score loads first: their addresses do not depend on cache_len
  float u[PER];
  {
    int m[PER];
    bool in[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      m[i] = (i * W + w) * 64 + lane;
      in[i] = m[i] < C;
    }
    group_sum<PER>(scores + ((size_t(b) * Hkv + g) * hpr * size_t(Nq) + t) * C, size_t(Nq) * C, hpr, m, in,
                   u);
  }
  if (threadIdx.x < 64) rank[threadIdx.x] = 0;
  const int c = row_candidates(cache_len, b, t, block, C, len_cap);
  const int K = topk < c ? topk : c;
  int32_t* out = idx + size_t(row) * topk;
  if (K == 0) {
    for (int e = threadIdx.x; e < topk; e += 64 * W) out[e] = -1;
    return;
  }
  uint64_t key[PER];
  uint32_t fmax = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int m = (i * W + w) * 64 + lane;
    const uint32_t hk = m < c ? score_key(u[i]) : 0u;  // valid score keys are > 0
    key[i] = m < c ? (uint64_t(hk) << 32) | uint32_t(~uint32_t(m)) : 0ull;
    fmax = fmax > hk ? fmax : hk;
  }
  // ---- filter (candidate m < 64 W sits alone on thread m, so at least K
  // lanes hold a valid key): the wave's KP largest lane maxima, then the row's
  uint32_t f[1] = {fmax};
  build_runs<1, 2, KP, uint32_t>(f, lane);
  if constexpr (KP < 64) merge_wave_runs<1, KP, uint32_t>(f, lane);
  if (lane < KP) fruns[0][w][lane] = f[0];
  int buf = merge_block_runs<E1, R1, KP, W, uint32_t>(fruns, w, lane);
  const uint32_t tau = fruns[buf][0][K - 1];
  const unsigned long long lt = lane ? (~0ull >> (64 - lane)) : 0ull;
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) cnt += __popcll(__ballot(uint32_t(key[i] >> 32) >= tau));
  if (lane == 0) wcnt[w] = cnt;
  __syncthreads();
  int S = 0, before = 0;
#pragma unroll
  for (int v = 0; v < W; ++v) {
    before += v < w ? wcnt[v] : 0;
    S += wcnt[v];
  }
  if (S <= 64) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const bool in = uint32_t(key[i] >> 32) >= tau;
      const unsigned long long bt = __ballot(in);
      if (in) surv[before + __popcll(bt & lt)] = key[i];
      before += __popcll(bt);
    }
    __syncthreads();
    // rank of survivor `lane`: wave w counts the larger ones among its
    // 64 / W survivors (64 w / W ...)
    if (lane < S) {
      const uint64_t me = surv[lane];
      uint32_t larger = 0;
#pragma unroll
      for (int j = 0; j < 64 / W; ++j) {
        const int o = (64 / W) * w + j;
        larger += (o < S && surv[o] > me) ? 1u : 0u;
      }
      if (larger) atomicAdd(&rank[lane], larger);
    }
    __syncthreads();
    if (w == 0) {
      if (lane < S && rank[lane] < uint32_t(K)) out[rank[lane]] = int(~uint32_t(surv[lane]));
      if (lane >= K && lane < topk) out[lane] = -1;
    }
    return;
  }

  // ---- full run merge
  // the lane's keys, descending
#pragma unroll
  for (int k = 2; k <= PER; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int l = i ^ j;
        if (l > i) {
          const bool desc = (i & k) == 0;
          const uint64_t a = key[i], bb = key[l];
          const bool sw = desc ? a < bb : a > bb;
          key[i] = sw ? bb : a;
          key[l] = sw ? a : bb;
        }
      }
  uint64_t v[E];
#pragma unroll
  for (int r = 0; r < E; ++r) v[r] = key[r];
  build_runs<E, 2, R, uint64_t>(v, lane);
  merge_wave_runs<E, R, uint64_t>(v, lane);
  if (lane < R)
#pragma unroll
    for (int r = 0; r < E; ++r) runs[0][w][lane * E + r] = v[r];
  buf = merge_block_runs<E, R, KP, W, uint64_t>(runs, w, lane);
  for (int e = threadIdx.x; e < topk; e += 64 * W)
    out[e] = e < K ? int(~uint32_t(runs[buf][0][e])) : -1;
}

// Rows of up to 1024 candidates with K <= 64 (training): one wave per row and
// no workgroup barrier.  The K-th largest of the lanes' maximum score keys
// bounds the K-th key from below (candidate m < 64 sits alone on lane m, and
// c >= K), so only keys at or above it survive; with many equal scores (more
// than 64 survivors) the wave radix select picks exactly K instead.  The
// survivors are sorted in one 64-lane bitonic network, lane e holding the
// e-th largest.  GH > 0 (training rows, GH = hpr): lane e also writes the
// softmax gate's base-2 log gates (s - LSE_s) log2 e of its block for every
// head of the row, at the block's slot, its rank in ascending block order
// among the selected (the slot the key-major attention kernels give it), so
// that the forward need not gather them from the score tensor again.
struct TopkGates {
  const float* lse_s;  // [B, Hkv hpr, Nq] gate normaliser of each query row
  float* out;          // [rows][topk][hpr]
};

template <int PER, int GH>
__global__ __launch_bounds__(256) void topk_wave_kernel(const float* __restrict__ scores,
                                                        int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ cache_len, int Hkv,
                                                        int hpr, int Nq, int C, int block, int topk,
                                                        int len_cap, long total_rows, TopkGates tg) {
  __shared__ uint32_t hist[4][256];
  __shared__ uint64_t surv[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const long row = long(blockIdx.x) * 4 + w;
  if (row >= total_rows) return;  // waves are independent: no workgroup barrier below
  const long t = row % Nq, bg = row / Nq;
  const int b = int(bg / Hkv), g = int(bg % Hkv);
  const int c = row_candidates(cache_len, b, t, block, C, len_cap);
  const int K = topk < c ? topk : c;
  int32_t* out = idx + size_t(row) * topk;
  if (K == 0) {
    if (lane < topk) out[lane] = -1;
    return;
  }
  uint32_t hk[PER];
  uint32_t fmax = 0;
  {
    int m[PER];
    bool in[PER];
    float u[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      m[i] = i * 64 + lane;
      in[i] = m[i] < c;
    }
    group_sum<PER>(scores + ((size_t(b) * Hkv + g) * hpr * size_t(Nq) + t) * C, size_t(Nq) * C, hpr, m, in,
                   u);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      hk[i] = in[i] ? score_key(u[i]) : 0u;  // valid score keys are > 0
      fmax = fmax > hk[i] ? fmax : hk[i];
    }
  }
  uint32_t f[1] = {fmax};
  build_runs<1, 2, 64, uint32_t>(f, lane);  // lane e: the e-th largest lane maximum
  const uint32_t tau = uint32_t(__builtin_amdgcn_readlane(int(f[0]), K - 1));
  int S = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) S += __popcll(__ballot(hk[i] >= tau));
  bool take[PER];
  if (S <= 64) {
#pragma unroll
    for (int i = 0; i < PER; ++i) take[i] = hk[i] >= tau;
  } else {
    uint32_t lo[PER];
    bool valid[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      lo[i] = ~uint32_t(i * 64 + lane);
      valid[i] = i * 64 + lane < c;
    }
    wave_select<PER>(hk, lo, valid, K, hist[w], take);
  }
  const unsigned long long lt = lane ? (~0ull >> (64 - lane)) : 0ull;
  int n = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const unsigned long long bt = __ballot(take[i]);
    if (take[i]) surv[w][n + __popcll(bt & lt)] = (uint64_t(hk[i]) << 32) | uint32_t(~uint32_t(i * 64 + lane));
    n += __popcll(bt);
  }
  wave_sync();
  uint64_t x[1] = {lane < n ? surv[w][lane] : 0ull};
  build_runs<1, 2, 64, uint64_t>(x, lane);
  const int me = int(~uint32_t(x[0]));  // lane e < K: the e-th best block
  if (lane < topk) out[lane] = lane < K ? me : -1;
  if constexpr (GH > 0) {
    // the block's scores were read above (cache hits); all loads go out
    // first (lanes past K read column 0), then the slot, the block's rank in
    // ascending block order among the K selected, is counted while they are
    // in flight
    const size_t r0 = (size_t(b) * Hkv + g) * GH * size_t(Nq) + t;  // query row of head 0
    const int mc = lane < K ? me : 0;
    float sv[GH], lv[GH];
#pragma unroll
    for (int h = 0; h < GH; ++h) {
      const size_t r = r0 + size_t(h) * Nq;
      sv[h] = scores[r * C + mc];
      lv[h] = tg.lse_s[r];
    }
    int slot = 0;
    for (int j = 0; j < K; ++j) slot += __builtin_amdgcn_readlane(me, j) < me ? 1 : 0;
    if (lane < K) {
      float* op = tg.out + (size_t(row) * topk + slot) * GH;
      if constexpr (GH == 4) {
        *reinterpret_cast<float4*>(op) = make_float4((sv[0] - lv[0]) * kLog2e, (sv[1] - lv[1]) * kLog2e,
                                                     (sv[2] - lv[2]) * kLog2e, (sv[3] - lv[3]) * kLog2e);
      } else {
#pragma unroll
        for (int h = 0; h < GH; ++h) op[h] = (sv[h] - lv[h]) * kLog2e;
      }
    }
  }
}

}  // namespace

hipError_t launch_topk(const float* scores, int32_t* idx, const int32_t* cache_len, int B, int Hkv,
                       int hpr, int Nq, int C, int block, int topk, hipStream_t s, int len_cap) {
  const long rows = long(B) * Hkv * Nq;
  if (rows == 0 || topk == 0) return hipSuccess;
  if (C <= 1024 && topk <= 64) {
    const dim3 grid((rows + 3) / 4);
    const TopkGates tg{};
    if (C <= 256)
      SAS_LAUNCH("topk", (topk_wave_kernel<4, 0>), grid, dim3(256), 0, s, scores, idx, cache_len, Hkv, hpr,
                 Nq, C, block, topk, len_cap, rows, tg);
    else if (C <= 512)
      SAS_LAUNCH("topk", (topk_wave_kernel<8, 0>), grid, dim3(256), 0, s, scores, idx, cache_len, Hkv, hpr,
                 Nq, C, block, topk, len_cap, rows, tg);
    else
      SAS_LAUNCH("topk", (topk_wave_kernel<16, 0>), grid, dim3(256), 0, s, scores, idx, cache_len, Hkv, hpr,
                 Nq, C, block, topk, len_cap, rows, tg);
  } else if (C <= 256) {
    SAS_LAUNCH("topk", (topk_kernel<1, 4>), dim3((rows + 3) / 4), dim3(256), 0, s, scores, idx,
                       cache_len, Hkv, hpr, Nq, C, block, topk, len_cap, rows);
  } else if (C <= 1024) {
    SAS_LAUNCH("topk", (topk_kernel<1, 16>), dim3((rows + 3) / 4), dim3(256), 0, s, scores, idx,
                       cache_len, Hkv, hpr, Nq, C, block, topk, len_cap, rows);
  } else if (topk <= 64 && C <= 16384) {
    // 8 waves, PER candidates per lane: just enough for C; run length: the
    // power of two at or above K (at least 8)
#define SAS_TOPK_RUNS(PER, KP, W)                                                                     \
  SAS_LAUNCH("topk_runs", (topk_runs_kernel<PER, KP, W>), dim3(rows), dim3(64 * W), 0, s, scores, idx, \
             cache_len, Hkv, hpr, Nq, C, block, topk, len_cap)
#define SAS_TOPK_RUNS_KP(PER, W)                        \
  if (topk <= 8) SAS_TOPK_RUNS(PER, 8, W);               \
  else if (topk <= 16) SAS_TOPK_RUNS(PER, 16, W);        \
  else if (topk <= 32) SAS_TOPK_RUNS(PER, 32, W);        \
  else SAS_TOPK_RUNS(PER, 64, W);
    if (C <= 2048) { SAS_TOPK_RUNS_KP(4, 8) }
    else if (C <= 4096) { SAS_TOPK_RUNS_KP(8, 8) }
    else if (C <= 8192) { SAS_TOPK_RUNS_KP(16, 8) }
    else { SAS_TOPK_RUNS_KP(32, 8) }  // 8 waves: 16 would cap a lane at 128 registers and spill
#undef SAS_TOPK_RUNS_KP
#undef SAS_TOPK_RUNS
  } else {
    // candidates per lane: just enough for C (16 waves x 64 lanes x PER);
    // survivors per lane in the second stage: 16 K / 64
#define SAS_TOPK_LONG(PER, PER2)                                                                          \
  SAS_LAUNCH("topk_long", (topk_long_kernel<PER, PER2>), dim3(rows), dim3(1024), 0, s, scores, idx, cache_len, \
             Hkv, hpr, Nq, C, block, topk, len_cap)
    const int per = C <= 2048 ? 2 : C <= 4096 ? 4 : C <= 8192 ? 8 : 16;
    const int per2 = topk <= 16 ? 4 : topk <= 32 ? 8 : 64;
    if (per == 2 && per2 == 4) SAS_TOPK_LONG(2, 4);
    else if (per == 2 && per2 == 8) SAS_TOPK_LONG(2, 8);
    else if (per == 2) SAS_TOPK_LONG(2, 64);
    else if (per == 4 && per2 == 4) SAS_TOPK_LONG(4, 4);
    else if (per == 4 && per2 == 8) SAS_TOPK_LONG(4, 8);
    else if (per == 4) SAS_TOPK_LONG(4, 64);
    else if (per == 8 && per2 == 4) SAS_TOPK_LONG(8, 4);
    else if (per == 8 && per2 == 8) SAS_TOPK_LONG(8, 8);
    else if (per == 8) SAS_TOPK_LONG(8, 64);
    else if (per2 == 4) SAS_TOPK_LONG(16, 4);
    else if (per2 == 8) SAS_TOPK_LONG(16, 8);
    else SAS_TOPK_LONG(16, 64);
#undef SAS_TOPK_LONG
  }
  return hipGetLastError();
}

// Training rows (c = t / block), with the selection's log gates; the wave
// kernel's range only (C <= 1024, topk <= 64, hpr one of 1, 2, 4, 8).
hipError_t launch_topk_gated(const float* scores, const float* lse_s, int32_t* idx, float* gates, int B,
                             int Hkv, int hpr, int Nq, int C, int block, int topk, hipStream_t s) {
  const long rows = long(B) * Hkv * Nq;
  if (rows == 0 || topk == 0) return hipSuccess;
  if (C > 1024 || topk > 64) return hipErrorNotSupported;
  const dim3 grid((rows + 3) / 4);
  const TopkGates tg{lse_s, gates};
  const int cap = 0x7fffffff;
#define SAS_TOPK_GATED(PER, GH)                                                                              \
  SAS_LAUNCH("topk", (topk_wave_kernel<PER, GH>), grid, dim3(256), 0, s, scores, idx, nullptr, Hkv, hpr, Nq, C, \
             block, topk, cap, rows, tg)
#define SAS_TOPK_GATED_PER(GH)                \
  if (C <= 256) SAS_TOPK_GATED(4, GH);         \
  else if (C <= 512) SAS_TOPK_GATED(8, GH);    \
  else SAS_TOPK_GATED(16, GH);
  if (hpr == 1) { SAS_TOPK_GATED_PER(1) }
  else if (hpr == 2) { SAS_TOPK_GATED_PER(2) }
  else if (hpr == 4) { SAS_TOPK_GATED_PER(4) }
  else if (hpr == 8) { SAS_TOPK_GATED_PER(8) }
  else return hipErrorNotSupported;
#undef SAS_TOPK_GATED_PER
#undef SAS_TOPK_GATED
  return hipGetLastError();
}

}  // namespace sas
