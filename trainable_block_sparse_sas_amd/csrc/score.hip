// Selector stage: block mean-pooling of keys and block scores.
//
// Pooled block summaries (jaehun.me review, "Our Perspective", Limitations)
// K̄_m = mean of the keys of block m; the selector score of history block m for
// a query is s_m = scale * q . K̄_m (one score per block: review "Background",
// paper Eq. 3).  Columns that are not history blocks of the query hold -inf.
#include "common.h"
#include "internal.h"
#include "mfma.h"

namespace sas {
namespace {

// One workgroup per (block m, KV head g, batch b); thread d sums the b tokens of
// column d in fp32 and writes the mean in the storage type.
template <typename T>
__global__ void pool_kernel(const T* __restrict__ k, T* __restrict__ kbar, int Hkv, int L, int D,
                            int block, int C) {
  const int m = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const T* src = k + ((size_t(b) * Hkv + g) * L + size_t(m) * block) * D;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float acc = 0.f;
    for (int j = 0; j < block; ++j) acc += to_f32(src[size_t(j) * D + d]);
    kbar[((size_t(b) * Hkv + g) * C + m) * D + d] = from_f32<T>(acc / float(block));
  }
}

// Pooled keys of cache pages: kbar_pages[p, g] = mean of the `block` keys of
// page p, head g ([num_pages, Hkv, block, D] -> [num_pages, Hkv, D]); one
// workgroup per (listed page, KV head).
template <typename T>
__global__ void pool_pages_kernel(const T* __restrict__ kp, T* __restrict__ kbar,
                                  const int32_t* __restrict__ pages, int Hkv, int D, int block) {
  const int p = pages[blockIdx.x], g = blockIdx.y;
  const T* src = kp + (size_t(p) * Hkv + g) * size_t(block) * D;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float acc = 0.f;
    for (int j = 0; j < block; ++j) acc += to_f32(src[size_t(j) * D + d]);
    kbar[(size_t(p) * Hkv + g) * D + d] = from_f32<T>(acc / float(block));
  }
}

// Training scores: a workgroup owns 64 query rows of one KV head and loops over
// that head's G query heads and over 64-wide tiles of blocks.  Tiles are staged
// in LDS as fp32; each thread produces 4 rows x 4 blocks per tile.
// hist_only: the columns m >= c(t) (no history block) are not written.
template <typename T, int D>
__global__ __launch_bounds__(256) void score_train_kernel(const T* __restrict__ q,
                                                          const T* __restrict__ kbar,
                                                          float* __restrict__ out, int Hq, int Hkv,
                                                          int N, int C, int block, float scale,
                                                          int group_sum, int hist_only) {
  constexpr int TR = 64, TM = 64, PAD = 1;
  __shared__ float qs[TR][D + PAD];
  __shared__ float ks[TM][D + PAD];
  const int tile = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x;
  const int r0 = (tid / 16) * 4;  // 16 x 16 thread grid, 4 x 4 outputs each
  const int c0 = (tid % 16) * 4;
  const int t0 = tile * TR;
  for (int mt = 0; mt < C; mt += TM) {
    float usum[4][4];
    for (int h = g * G; h < (g + 1) * G; ++h) {
      __syncthreads();
      for (int i = tid; i < TR * D; i += 256) {
        int r = i / D, d = i % D;
        int t = t0 + r;
        qs[r][d] = t < N ? to_f32(q[((size_t(b) * Hq + h) * N + t) * D + d]) : 0.f;
      }
      if (h == g * G) {
        for (int i = tid; i < TM * D; i += 256) {
          int r = i / D, d = i % D;
          int m = mt + r;
          ks[r][d] = m < C ? to_f32(kbar[((size_t(b) * Hkv + g) * C + m) * D + d]) : 0.f;
        }
      }
      __syncthreads();
      float acc[4][4] = {};
      for (int d = 0; d < D; ++d) {
        float a[4], w[4];
        for (int i = 0; i < 4; ++i) a[i] = qs[r0 + i][d];
        for (int j = 0; j < 4; ++j) w[j] = ks[c0 + j][d];
        for (int i = 0; i < 4; ++i)
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], w[j], acc[i][j]);
      }
      for (int i = 0; i < 4; ++i) {
        int t = t0 + r0 + i;
        if (t >= N) continue;
        int c = t / block;
        for (int j = 0; j < 4; ++j) {
          int m = mt + c0 + j;
          if (m >= C || (hist_only && m >= c)) continue;
          float sv = m < c ? acc[i][j] * scale : kNegInf;
          if (group_sum) {
            usum[i][j] = (h == g * G) ? sv : usum[i][j] + sv;
          } else {
            out[((size_t(b) * Hq + h) * N + t) * C + m] = sv;
          }
        }
      }
    }
    if (group_sum) {
      for (int i = 0; i < 4; ++i) {
        int t = t0 + r0 + i;
        if (t >= N) continue;
        for (int j = 0; j < 4; ++j) {
          int m = mt + c0 + j;
          if (m < C) out[((size_t(b) * Hkv + g) * N + t) * C + m] = usum[i][j];
        }
      }
    }
  }
}

// Training scores on the matrix cores (bf16 q and pooled keys, fp32 out):
// S = Q K̄^T on v_mfma_f32_16x16x32_bf16.  A workgroup owns 64 query rows of
// one head (16 per wave; the rows of a wave share one block when block % 16 == 0)
// and walks the blocks in chunks of 64 staged in LDS.  Chunks at or beyond a
// wave's own block are not computed, only filled with -inf.
// lse_s (optional): the softmax gate's normaliser LSE_s(t) = log sum over the
// history blocks m < c(t) of exp(s[t,m]) (jaehun.me review, "Why the Four
// Design Choices Matter": log g = s - LSE(s)), -inf without history.  Each
// lane keeps a running (max, sum of exp) of its columns for its four rows;
// the 16 lanes of a row group merge theirs at the end.
// hist_only: the columns m >= c(t) (no history block) are not written.
template <int D>
__global__ __launch_bounds__(256) void score_train_mfma_kernel(const bf16_t* __restrict__ q,
                                                               const bf16_t* __restrict__ kbar,
                                                               float* __restrict__ out,
                                                               float* __restrict__ lse_s, int Hq,
                                                               int Hkv, int N, int C, int block,
                                                               float scale, int hist_only) {
  constexpr int KS = D / 32, CH = D / 8;
  __shared__ __attribute__((aligned(16))) uint16_t ks[64][D + 8];
  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / (Hq / Hkv);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int t0 = tile * 64 + wave * 16;
  const int c = t0 < N ? t0 / block : 0;  // shared by the wave's 16 rows
  int c_max = min(N - 1, tile * 64 + 63) / block;
  const bf16_t* kb = kbar + (size_t(b) * Hkv + g) * size_t(C) * D;
  uint4 qa[KS];
  {
    const int t = t0 + lr;
    const bf16_t* qr = q + ((size_t(b) * Hq + h) * N + (t < N ? t : 0)) * D;
    for (int k2 = 0; k2 < KS; ++k2)
      qa[k2] = t < N ? *reinterpret_cast<const uint4*>(qr + k2 * 32 + lq * 8) : make_uint4(0, 0, 0, 0);
  }
  float* orow[4];
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 4 * lq + i;
    orow[i] = t < N ? out + ((size_t(b) * Hq + h) * N + t) * C : nullptr;
  }
  float lmx[4], lsm[4];
  for (int i = 0; i < 4; ++i) {
    lmx[i] = kNegInf;
    lsm[i] = 0.f;
  }
  for (int m0 = 0; m0 < C; m0 += 64) {
    const bool load = m0 < c_max;  // uniform: some wave of the group computes here
    if (load) {
      __syncthreads();
      for (int i = tid; i < 64 * CH; i += 256) {
        const int r = i / CH, c8 = i % CH;
        const int m = m0 + r;
        *reinterpret_cast<uint4*>(&ks[r][c8 * 8]) =
            m < C ? *reinterpret_cast<const uint4*>(kb + size_t(m) * D + c8 * 8) : make_uint4(0, 0, 0, 0);
      }
      __syncthreads();
    }
    for (int nt = 0; nt < 4; ++nt) {
      const int mb = m0 + 16 * nt;
      if (mb >= C) break;
      const int m = mb + lr;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      if (mb < c) {
        for (int k2 = 0; k2 < KS; ++k2) {
          const uint4 bf = *reinterpret_cast<const uint4*>(&ks[16 * nt + lr][k2 * 32 + lq * 8]);
          acc = mfma16(qa[k2], bf, acc);
        }
        if (lse_s != nullptr && m < c)
          for (int i = 0; i < 4; ++i) {
            const float x = acc[i] * scale;
            const float nm = fmaxf(lmx[i], x);
            lsm[i] = lsm[i] * exp2_hw((lmx[i] - nm) * kLog2e) + exp2_hw((x - nm) * kLog2e);
            lmx[i] = nm;
          }
      }
      if (m < (hist_only ? c : C))
        for (int i = 0; i < 4; ++i)
          if (orow[i]) orow[i][m] = m < c ? acc[i] * scale : kNegInf;
    }
  }
  if (lse_s != nullptr) {
    for (int i = 0; i < 4; ++i) {
      for (int off = 1; off < 16; off <<= 1) {
        const float om = shfl_xor(lmx[i], off), os = shfl_xor(lsm[i], off);
        const float nm = fmaxf(lmx[i], om);
        if (nm != kNegInf) lsm[i] = lsm[i] * exp2_hw((lmx[i] - nm) * kLog2e) + os * exp2_hw((om - nm) * kLog2e);
        lmx[i] = nm;
      }
      const int t = t0 + 4 * lq + i;
      if (lr == 0 && t < N) lse_s[(size_t(b) * Hq + h) * N + t] = c > 0 ? lmx[i] + log_hw(lsm[i]) : kNegInf;
    }
  }
}

// Decode scores (fp32): one query token per sequence scans the pooled keys of its KV
// head.  A K̄ row (D values) is read by LPR lanes with 16-byte loads, so a wave
// covers 64/LPR rows per load; partial dots are reduced across those lanes.
// The G query heads of the group are handled together; with group_sum the fp32
// scores are added in head-index order.
template <typename T, int D, int G>
__global__ __launch_bounds__(256) void score_decode_kernel(
    const T* __restrict__ q, const T* __restrict__ kbar, float* __restrict__ out,
    const int32_t* __restrict__ cache_len, int Hq, int Hkv, int L, int C, int block, float scale,
    int group_sum) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int LPR = D / VEC;        // lanes per K̄ row
  constexpr int RPW = 64 / LPR;       // rows per wave per load
  constexpr int MAXG = G;
  const int g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPR, rsub = lane / LPR;
  int len = cache_len[b];
  len = len > L ? L : len;
  const int c = len > 0 ? (len - 1) / block : 0;
  const int c_eff = c < C ? c : C;
  float qv[MAXG][VEC];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i = 0; i < VEC; ++i)
      qv[h][i] = to_f32(q[(size_t(b) * Hq + g * G + h) * D + sub * VEC + i]);
  const int rows_per_wg = RPW * 4 * 4;  // 4 waves, 4 loads per wave
  const int m_base = blockIdx.x * rows_per_wg;
  // All four row loads first (their addresses do not depend on cache_len, so
  // they overlap its load); rows past the history are masked below.
  uint4 raw[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int m = m_base + (it * 4 + wave) * RPW + rsub;
    raw[it] = m < C ? *reinterpret_cast<const uint4*>(kbar + ((size_t(b) * Hkv + g) * C + m) * D + sub * VEC)
                    : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int m = m_base + (it * 4 + wave) * RPW + rsub;
    float dots[MAXG];
    const bool in = m < C;
    T kv[VEC];
    {
      const T* p = reinterpret_cast<const T*>(&raw[it]);
      for (int i = 0; i < VEC; ++i) kv[i] = m < c_eff ? p[i] : T(0);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < VEC; ++i) a = fmaf(qv[h][i], to_f32(kv[i]), a);
      for (int off = LPR / 2; off >= 1; off >>= 1) a += shfl_xor(a, off);
      dots[h] = a;
    }
    if (in && sub == 0) {
      if (group_sum) {
        float u = kNegInf;
        if (m < c_eff) {
          u = dots[0] * scale;
#pragma unroll
          for (int h = 1; h < G; ++h) u = u + dots[h] * scale;
        }
        out[(size_t(b) * Hkv + g) * C + m] = u;
      } else {
#pragma unroll
        for (int h = 0; h < G; ++h)
          out[(size_t(b) * Hq + g * G + h) * C + m] = m < c_eff ? dots[h] * scale : kNegInf;
      }
    }
  }
}

// Decode scores on the matrix cores (bf16): the G query heads of a KV head
// form the A operand (rows 0..G-1 of a 16-row tile, the rest zero) and 16
// pooled keys the B operand, so one v_mfma_f32_16x16x32_bf16 per 32 columns
// scores 16 blocks for all heads.  Lane (lq, lr) loads row lr of the tile at
// the KS consecutive 16-byte chunks lq KS .. lq KS + KS - 1 (the head rows
// use the same column order), i.e. 64 contiguous bytes per lane.  Each wave
// scores TPW tiles with all loads issued first (they do not depend on
// cache_len).  The heads' scores of block lr come out in lanes lr, lr + 16,
// lr + 32, lr + 48 (4 heads each) and are added in head-index order.  With a
// page table, pooled key m of sequence b is row table[b, m] of kbar
// [num_pages, Hkv, D] (pages past the sequence's history are not read).
template <int D, int G, int TPW>
__global__ __launch_bounds__(256) void score_decode_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ kbar, float* __restrict__ out,
    const int32_t* __restrict__ cache_len, int Hq, int Hkv, int L, int C, int block, float scale,
    int group_sum, const int32_t* __restrict__ table) {
  constexpr int KS = D / 32;
  static_assert(G <= 16, "one 16-row tile of heads");
  const int g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int m0 = (blockIdx.x * 4 + wave) * TPW * 16;  // first block of the wave
  const bf16_t* kb = kbar + (size_t(b) * Hkv + g) * size_t(C) * D;
  int hist = C;  // blocks that may be read: all of them, or the history when paged
  if (table) {
    int len0 = cache_len[b];
    len0 = len0 > L ? L : len0;
    hist = len0 > 0 ? min((len0 - 1) / block, C) : 0;
  }
  uint4 kf[TPW][KS];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int m = m0 + tt * 16 + lr;
    const bf16_t* row = nullptr;
    if (m < hist)
      row = table ? kbar + (size_t(table[size_t(b) * C + m]) * Hkv + g) * D : kb + size_t(m) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kf[tt][ks] = row ? *reinterpret_cast<const uint4*>(row + (lq * KS + ks) * 8) : make_uint4(0, 0, 0, 0);
  }
  uint4 qa[KS];
  {
    const bf16_t* qr = q + (size_t(b) * Hq + g * G + (lr < G ? lr : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qa[ks] = lr < G ? *reinterpret_cast<const uint4*>(qr + (lq * KS + ks) * 8) : make_uint4(0, 0, 0, 0);
  }
  int len = cache_len[b];
  len = len > L ? L : len;
  const int c = len > 0 ? (len - 1) / block : 0;
  const int c_eff = c < C ? c : C;
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc = mfma16(qa[ks], kf[tt][ks], acc);
    const int m = m0 + tt * 16 + lr;
    if (group_sum) {
      // heads 4 lq .. 4 lq + 3 of block lr sit in lane (lq, lr)
      float hv[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = acc[j];
        hv[j] = x;
        if constexpr (G > 4) hv[4 + j] = __shfl_xor(x, 16, 64);
        if constexpr (G > 8) hv[8 + j] = __shfl_xor(x, 32, 64);
        if constexpr (G > 12) hv[12 + j] = __shfl_xor(x, 48, 64);
      }
      if (lq == 0 && m < C) {
        float u = kNegInf;
        if (m < c_eff) {
          u = hv[0] * scale;
#pragma unroll
          for (int h = 1; h < G; ++h) u = u + hv[h] * scale;
        }
        out[(size_t(b) * Hkv + g) * C + m] = u;
      }
    } else if (m < C) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int h = 4 * lq + j;
        if (h < G) out[(size_t(b) * Hq + g * G + h) * C + m] = m < c_eff ? acc[j] * scale : kNegInf;
      }
    }
  }
}

}  // namespace

hipError_t launch_pool(const void* k, void* kbar, int B, int Hkv, int L, int D, int block, int C,
                       bool bf16, hipStream_t s) {
  if (C == 0 || B == 0) return hipSuccess;
  dim3 grid(C, Hkv, B);
  if (bf16)
    SAS_LAUNCH("pool", pool_kernel<bf16_t>, grid, dim3(D), 0, s, (const bf16_t*)k, (bf16_t*)kbar,
                       Hkv, L, D, block, C);
  else
    SAS_LAUNCH("pool", pool_kernel<float>, grid, dim3(D), 0, s, (const float*)k, (float*)kbar, Hkv,
                       L, D, block, C);
  return hipGetLastError();
}

template <typename T, int D>
static void score_train_t(const void* q, const void* kbar, float* scores, const Dims& d,
                          float scale, bool group_sum, bool hist_only, hipStream_t s) {
  dim3 grid((d.N + 63) / 64, d.Hkv, d.B);
  SAS_LAUNCH("score_train", (score_train_kernel<T, D>), grid, dim3(256), 0, s, (const T*)q,
                     (const T*)kbar, scores, d.Hq, d.Hkv, d.N, d.C, d.block, scale,
                     group_sum ? 1 : 0, hist_only ? 1 : 0);
}

hipError_t launch_score_train(const void* q, const void* kbar, float* scores, const Dims& d,
                              float scale, bool group_sum, bool bf16, hipStream_t s, float* lse_s,
                              bool hist_only) {
  if (d.N == 0 || d.B == 0) return hipSuccess;
  if (d.C == 0) return lse_s ? launch_lse_rows(scores, lse_s, d, s) : hipSuccess;  // rows without history
  if (bf16 && !group_sum && d.block % 16 == 0) {
    dim3 grid((d.N + 63) / 64, d.Hq, d.B);
    if (d.D == 64)
      SAS_LAUNCH("score_train_mfma", score_train_mfma_kernel<64>, grid, dim3(256), 0, s, (const bf16_t*)q,
                         (const bf16_t*)kbar, scores, lse_s, d.Hq, d.Hkv, d.N, d.C, d.block, scale,
                         int(hist_only));
    else
      SAS_LAUNCH("score_train_mfma", score_train_mfma_kernel<128>, grid, dim3(256), 0, s, (const bf16_t*)q,
                         (const bf16_t*)kbar, scores, lse_s, d.Hq, d.Hkv, d.N, d.C, d.block, scale,
                         int(hist_only));
    return hipGetLastError();
  }
  if (bf16) {
    if (d.D == 64) score_train_t<bf16_t, 64>(q, kbar, scores, d, scale, group_sum, hist_only, s);
    else score_train_t<bf16_t, 128>(q, kbar, scores, d, scale, group_sum, hist_only, s);
  } else {
    if (d.D == 64) score_train_t<float, 64>(q, kbar, scores, d, scale, group_sum, hist_only, s);
    else score_train_t<float, 128>(q, kbar, scores, d, scale, group_sum, hist_only, s);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || !lse_s) return e;
  return launch_lse_rows(scores, lse_s, d, s);  // a pass over the scores just written
}

template <int D>
static void score_decode_mfma_t(const void* q, const void* kbar, float* scores, const int32_t* cl,
                                int B, int Hq, int Hkv, int L, int block, int C, float scale,
                                bool group_sum, const int32_t* table, hipStream_t s) {
  constexpr int TPW = 2;
  const int rows_per_wg = 4 * TPW * 16;
  dim3 grid((C + rows_per_wg - 1) / rows_per_wg, Hkv, B);
  switch (Hq / Hkv) {
#define SAS_SCDM_G(GG)                                                                              \
  case GG:                                                                                         \
    SAS_LAUNCH("score_decode", (score_decode_mfma_kernel<D, GG, TPW>), grid, dim3(256), 0, s,       \
               (const bf16_t*)q, (const bf16_t*)kbar, scores, cl, Hq, Hkv, L, C, block, scale,      \
               group_sum ? 1 : 0, table);                                                          \
    break;
    SAS_SCDM_G(1) SAS_SCDM_G(2) SAS_SCDM_G(3) SAS_SCDM_G(4) SAS_SCDM_G(5) SAS_SCDM_G(6) SAS_SCDM_G(7)
    SAS_SCDM_G(8) SAS_SCDM_G(9) SAS_SCDM_G(10) SAS_SCDM_G(11) SAS_SCDM_G(12) SAS_SCDM_G(13)
    SAS_SCDM_G(14) SAS_SCDM_G(15) SAS_SCDM_G(16)
#undef SAS_SCDM_G
    default: break;
  }
}

template <typename T, int D>
static void score_decode_t(const void* q, const void* kbar, float* scores, const int32_t* cl,
                           int B, int Hq, int Hkv, int L, int block, int C, float scale,
                           bool group_sum, hipStream_t s) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int RPW = 64 / (D / VEC);
  const int rows_per_wg = RPW * 16;
  dim3 grid((C + rows_per_wg - 1) / rows_per_wg, Hkv, B);
  switch (Hq / Hkv) {
#define SAS_SCD_G(GG)                                                                        \
  case GG:                                                                                  \
    SAS_LAUNCH("score_decode", (score_decode_kernel<T, D, GG>), grid, dim3(256), 0, s, (const T*)q, \
                       (const T*)kbar, scores, cl, Hq, Hkv, L, C, block, scale, group_sum ? 1 : 0); \
    break;
    SAS_SCD_G(1) SAS_SCD_G(2) SAS_SCD_G(3) SAS_SCD_G(4) SAS_SCD_G(5) SAS_SCD_G(6) SAS_SCD_G(7)
    SAS_SCD_G(8) SAS_SCD_G(9) SAS_SCD_G(10) SAS_SCD_G(11) SAS_SCD_G(12) SAS_SCD_G(13)
    SAS_SCD_G(14) SAS_SCD_G(15) SAS_SCD_G(16)
#undef SAS_SCD_G
    default: break;
  }
}

hipError_t launch_pool_pages(const void* k_pages, void* kbar_pages, const int32_t* pages, int n_pages,
                             int Hkv, int D, int block, bool bf16, hipStream_t s) {
  if (n_pages == 0 || Hkv == 0) return hipSuccess;
  dim3 grid(n_pages, Hkv);
  if (bf16)
    SAS_LAUNCH("pool_pages", pool_pages_kernel<bf16_t>, grid, dim3(D), 0, s, (const bf16_t*)k_pages,
               (bf16_t*)kbar_pages, pages, Hkv, D, block);
  else
    SAS_LAUNCH("pool_pages", pool_pages_kernel<float>, grid, dim3(D), 0, s, (const float*)k_pages,
               (float*)kbar_pages, pages, Hkv, D, block);
  return hipGetLastError();
}

hipError_t launch_score_decode(const void* q, const void* kbar, float* scores,
                               const int32_t* cache_len, int B, int Hq, int Hkv, int L, int D,
                               int block, int C, float scale, bool group_sum, bool bf16,
                               hipStream_t s, const int32_t* table) {
  if (B == 0 || C == 0) return hipSuccess;
  if (bf16) {
    if (D == 64) score_decode_mfma_t<64>(q, kbar, scores, cache_len, B, Hq, Hkv, L, block, C, scale, group_sum, table, s);
    else score_decode_mfma_t<128>(q, kbar, scores, cache_len, B, Hq, Hkv, L, block, C, scale, group_sum, table, s);
  } else {
    if (D == 64) score_decode_t<float, 64>(q, kbar, scores, cache_len, B, Hq, Hkv, L, block, C, scale, group_sum, s);
    else score_decode_t<float, 128>(q, kbar, scores, cache_len, B, Hq, Hkv, L, block, C, scale, group_sum, s);
  }
  return hipGetLastError();
}

}  // namespace sas
