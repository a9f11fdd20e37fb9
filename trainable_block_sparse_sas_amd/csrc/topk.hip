// Hard Top-K block selection (jaehun.me review, "Background", paper Eq. 3;
// "A Concrete Walkthrough", Step 3 and Step 6).
//
// Per row (one query token and one KV head) the candidates are the history
// blocks m < c.  The group score is the fp32 sum of the row's head scores in
// head-index order.  Exactly min(K, c) blocks are kept, ordered by score
// descending with ties to the lower block index (-0.0 == +0.0, NaN == -inf).
//
// Selection is sort-free: an MSB-first radix select over the order-preserving
// uint32 key finds the K-th largest key T in four 8-bit passes (LDS histogram),
// every key > T is kept and the keys equal to T are taken in index order.
// Only the K survivors are then ranked, by counting.
#include "common.h"
#include "internal.h"

namespace sas {
namespace {

constexpr int kMaxTopk = 256;

// WPR waves cooperate on one row; PER lanes-slots per lane (c <= 64*WPR*PER).
template <int WPR, int PER>
__global__ __launch_bounds__(256 * (WPR > 4 ? 4 : 1)) void topk_kernel(
    const float* __restrict__ scores, int32_t* __restrict__ idx,
    const int32_t* __restrict__ cache_len, int Hkv, int hpr, int Nq, int C, int block, int topk,
    long total_rows) {
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
    if (cache_len) {
      int len = cache_len[b];
      c = len > 0 ? (len - 1) / block : 0;
    } else {
      c = int(t / block);
    }
    c = c < C ? c : C;
    K = topk < c ? topk : c;
  }
  // Load the group-summed scores as order-preserving keys.
  uint32_t key[PER];
  bool valid[PER];
  {
    const int g = int(bg % Hkv);
    const int b = int(bg / Hkv);
    for (int i = 0; i < PER; ++i) {
      const int m = (i * WPR + wr) * 64 + lane;
      valid[i] = active && m < c;
      key[i] = 0;
      if (valid[i]) {
        const float* base = scores + ((size_t(b) * Hkv + g) * hpr * size_t(Nq) + t) * C + m;
        float u = base[0];
        for (int h = 1; h < hpr; ++h) u = u + base[size_t(h) * Nq * C];
        key[i] = score_key(u);
      }
    }
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

}  // namespace

hipError_t launch_topk(const float* scores, int32_t* idx, const int32_t* cache_len, int B, int Hkv,
                       int hpr, int Nq, int C, int block, int topk, hipStream_t s) {
  const long rows = long(B) * Hkv * Nq;
  if (rows == 0 || topk == 0) return hipSuccess;
  if (C <= 256) {
    hipLaunchKernelGGL((topk_kernel<1, 4>), dim3((rows + 3) / 4), dim3(256), 0, s, scores, idx,
                       cache_len, Hkv, hpr, Nq, C, block, topk, rows);
  } else if (C <= 1024) {
    hipLaunchKernelGGL((topk_kernel<1, 16>), dim3((rows + 3) / 4), dim3(256), 0, s, scores, idx,
                       cache_len, Hkv, hpr, Nq, C, block, topk, rows);
  } else {
    hipLaunchKernelGGL((topk_kernel<16, 16>), dim3(rows), dim3(1024), 0, s, scores, idx,
                       cache_len, Hkv, hpr, Nq, C, block, topk, rows);
  }
  return hipGetLastError();
}

}  // namespace sas
