// SAS gated attention, forward and backward, on the vector ALUs (fp32 math).
//
// This is the path for fp32 tensors (and for bf16 shapes the matrix-core
// kernels do not cover).  Four lanes share one query row (or one key in the
// dK/dV kernel), each owning D/4 of the head dimension; dot products are
// reduced across the four lanes.  Keys are streamed through LDS 32 at a time.
//
// Logit of query t and key j (blog 方法核心 SAS formula; jaehun.me review,
// "New Approach", paper Eq. 9):
//   z = scale * q_t . k_j + bias(t, j),
//   bias = 0                      key in the own block c(t) = t / b, j <= t
//        = s[t,m] - LSE_s(t)      key in history block m < c(t) that is gated
//                                 (full scope: all of them; sparse: selected)
//        = -inf                   otherwise.
// log g = s - LSE(s): review "Why the Four Design Choices Matter".
#include "common.h"
#include "internal.h"

namespace sas {
namespace {

constexpr int KT = 32;  // keys per LDS tile

// Selection bitmask of one row: bit m set when history block m is selected.
__device__ __forceinline__ bool mask_bit(const uint32_t* mask, int m) {
  return (mask[m >> 5] >> (m & 31)) & 1u;
}

__device__ __forceinline__ float quad_sum(float x) {
  x += shfl_xor(x, 1);
  x += shfl_xor(x, 2);
  return x;
}

// Builds the row's selection mask from idx (entries outside [0, c) ignored).
__device__ void build_row_mask(uint32_t* mask, int MW, const int32_t* idx_row, int topk, int c,
                               bool rv, int p) {
  for (int w = p; w < MW; w += 4) mask[w] = 0u;
  __syncthreads();
  if (rv) {
    for (int e = p; e < topk; e += 4) {
      const int m = idx_row[e];
      if (m >= 0 && m < c) atomicOr(&mask[m >> 5], 1u << (m & 31));
    }
  }
  __syncthreads();
}

// Is any key of [j0, j0+KT) attended by row t?
__device__ __forceinline__ bool row_attends_tile(int t, int c, int j0, int block, bool full,
                                                 const uint32_t* mask) {
  if (j0 > t) return false;
  const int jl = min(j0 + KT - 1, t);
  for (int m = j0 / block; m <= jl / block; ++m)
    if (m == c || full || mask_bit(mask, m)) return true;
  return false;
}

template <typename T, int D>
__device__ __forceinline__ void load_tile(float (*dst)[D + 1], const T* src, int j0, int N) {
  for (int i = threadIdx.x; i < KT * D; i += blockDim.x) {
    const int jj = i / D, d = i % D;
    dst[jj][d] = (j0 + jj < N) ? to_f32(src[size_t(j0 + jj) * D + d]) : 0.f;
  }
}

// ---------------------------------------------------------------- forward ---
template <typename T, int D>
__global__ __launch_bounds__(256) void fwd_simt_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ scores, const int32_t* __restrict__ idx, T* __restrict__ o,
    float* __restrict__ lse, float* __restrict__ lse_s, int Hq, int Hkv, int N, int C, int block,
    int topk, float scale, int norm, int outer) {
  constexpr int DS = D / 4;
  extern __shared__ uint32_t dyn_mask[];
  __shared__ float ks[KT][D + 1];
  __shared__ float vs[KT][D + 1];
  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv, g = h / G;
  const int r = threadIdx.x >> 2, p = threadIdx.x & 3;
  const int t = tile * 64 + r;
  const bool rv = t < N;
  const int c = rv ? t / block : 0;
  const size_t row = (size_t(b) * Hq + h) * N + (rv ? t : 0);
  const float* srow = scores + row * C;
  const bool full = (idx == nullptr);

  // LSE of the row's history scores (the softmax gate's normaliser; norm 2:
  // given in lse_s; the other gates have none: 0, already in lse_s).
  float mx = kNegInf, sm = 0.f;
  for (int m = p; norm == 1 && m < c; m += 4) {
    const float x = srow[m];
    const float nm = fmaxf(mx, x);
    sm = sm * exp_hw(mx - nm) + exp_hw(x - nm);
    mx = nm;
  }
  for (int off = 1; off <= 2; off <<= 1) {
    const float om = shfl_xor(mx, off), os = shfl_xor(sm, off);
    const float nm = fmaxf(mx, om);
    if (nm != kNegInf) {
      sm = sm * exp_hw(mx - nm) + os * exp_hw(om - nm);
      mx = nm;
    }
  }
  const float lses = norm == 2 ? (rv ? lse_s[row] : 0.f) : !norm ? 0.f : c > 0 ? mx + log_hw(sm) : kNegInf;
  if (norm == 1 && rv && p == 0) lse_s[row] = lses;

  const int MW = (C + 31) / 32;
  uint32_t* mask = dyn_mask + r * MW;
  if (!full)
    build_row_mask(mask, MW, idx + ((size_t(b) * Hkv + g) * N + (rv ? t : 0)) * topk, topk, c, rv, p);

  float qv[DS], acc[DS];
  for (int i = 0; i < DS; ++i) {
    qv[i] = rv ? to_f32(q[row * D + p * DS + i]) : 0.f;
    acc[i] = 0.f;
  }
  float mi = kNegInf, li = 0.f;
  int cur_m = -1;
  float cur_bias = kNegInf, cur_g = 1.f;  // outer gate: no bias, g scales the value
  const T* kh = k + (size_t(b) * Hkv + g) * N * D;
  const T* vh = v + (size_t(b) * Hkv + g) * N * D;
  const int t_last = min(N, tile * 64 + 64) - 1;
  for (int j0 = 0; j0 <= t_last; j0 += KT) {
    const bool any = rv && row_attends_tile(t, c, j0, block, full, mask);
    if (!__syncthreads_or(any)) continue;
    load_tile<T, D>(ks, kh, j0, N);
    load_tile<T, D>(vs, vh, j0, N);
    __syncthreads();
    if (any) {
      for (int jj = 0; jj < KT; ++jj) {
        const int j = j0 + jj;
        if (j > t) break;
        const int m = j / block;
        if (m != cur_m) {
          cur_m = m;
          cur_bias = (m == c) ? 0.f : ((full || mask_bit(mask, m)) ? srow[m] - lses : kNegInf);
          cur_g = 1.f;
          if (outer && m != c && cur_bias != kNegInf) {
            cur_g = exp_hw(cur_bias);
            cur_bias = 0.f;
          }
        }
        if (cur_bias == kNegInf) continue;
        float dot = 0.f;
        for (int i = 0; i < DS; ++i) dot = fmaf(qv[i], ks[jj][p * DS + i], dot);
        const float z = quad_sum(dot) * scale + cur_bias;
        const float nm = fmaxf(mi, z);
        const float alpha = exp_hw(mi - nm);
        const float pe = exp_hw(z - nm);
        li = li * alpha + pe;
        const float pv = pe * cur_g;
        for (int i = 0; i < DS; ++i) acc[i] = acc[i] * alpha + pv * vs[jj][p * DS + i];
        mi = nm;
      }
    }
    __syncthreads();
  }
  if (rv) {
    const float inv = 1.f / li;
    for (int i = 0; i < DS; ++i) o[row * D + p * DS + i] = from_f32<T>(acc[i] * inv);
    if (p == 0) lse[row] = mi + log_hw(li);
  }
}

// --------------------------------------------------------------- backward ---
// Delta[row] = sum_d dO[row,d] * o[row,d].
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const T* __restrict__ o,
                                                        const T* __restrict__ dout,
                                                        float* __restrict__ delta, size_t rows) {
  constexpr int DS = D / 4;
  const size_t row = size_t(blockIdx.x) * 64 + (threadIdx.x >> 2);
  const int p = threadIdx.x & 3;
  float a = 0.f;
  if (row < rows)
    for (int i = 0; i < DS; ++i)
      a = fmaf(to_f32(o[row * D + p * DS + i]), to_f32(dout[row * D + p * DS + i]), a);
  a = quad_sum(a);
  if (row < rows && p == 0) delta[row] = a;
}

// dq and ds, query-major.  dbeta of a gated history block is the sum of dz over
// its keys (inner-gate gradient of blog 方法核心 / review paper Eq. 5, times g);
// ds = dbeta - g * sum(dbeta) is the chain rule through log g = s - LSE(s)
// (gate_ds: the other gate activations' rules).
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_dq_simt_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const float* __restrict__ scores, const int32_t* __restrict__ idx,
    const float* __restrict__ lse, const float* __restrict__ lse_s,
    const float* __restrict__ delta, T* __restrict__ dq, float* __restrict__ ds, int Hq, int Hkv,
    int N, int C, int block, int topk, float scale, int gate) {
  constexpr int DS = D / 4;
  extern __shared__ uint32_t dyn_mask[];
  __shared__ float ks[KT][D + 1];
  __shared__ float vs[KT][D + 1];
  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv, g = h / G;
  const int r = threadIdx.x >> 2, p = threadIdx.x & 3;
  const int t = tile * 64 + r;
  const bool rv = t < N;
  const int c = rv ? t / block : 0;
  const size_t row = (size_t(b) * Hq + h) * N + (rv ? t : 0);
  const float* srow = scores + row * C;
  float* dsrow = ds + row * C;
  const bool full = (idx == nullptr);
  const float lrow = rv ? lse[row] : 0.f;
  const float lses = rv ? lse_s[row] : 0.f;
  const float drow = rv ? delta[row] : 0.f;

  const int MW = (C + 31) / 32;
  uint32_t* mask = dyn_mask + r * MW;
  if (!full)
    build_row_mask(mask, MW, idx + ((size_t(b) * Hkv + g) * N + (rv ? t : 0)) * topk, topk, c, rv, p);

  float qv[DS], dov[DS], dqa[DS];
  for (int i = 0; i < DS; ++i) {
    qv[i] = rv ? to_f32(q[row * D + p * DS + i]) : 0.f;
    dov[i] = rv ? to_f32(dout[row * D + p * DS + i]) : 0.f;
    dqa[i] = 0.f;
  }
  int cur_m = -1;
  float cur_bias = kNegInf, cur_g = 1.f, db_cur = 0.f, db_total = 0.f;
  const bool outer = gate == kGateOuter;
  const T* kh = k + (size_t(b) * Hkv + g) * N * D;
  const T* vh = v + (size_t(b) * Hkv + g) * N * D;
  const int t_last = min(N, tile * 64 + 64) - 1;
  for (int j0 = 0; j0 <= t_last; j0 += KT) {
    const bool any = rv && row_attends_tile(t, c, j0, block, full, mask);
    if (!__syncthreads_or(any)) continue;
    load_tile<T, D>(ks, kh, j0, N);
    load_tile<T, D>(vs, vh, j0, N);
    __syncthreads();
    if (any) {
      for (int jj = 0; jj < KT; ++jj) {
        const int j = j0 + jj;
        if (j > t) break;
        const int m = j / block;
        if (m != cur_m) {
          if (cur_m >= 0 && cur_m < c && cur_bias != kNegInf) {
            db_total += db_cur;
            if ((cur_m & 3) == p) dsrow[cur_m] = db_cur;
          }
          db_cur = 0.f;
          cur_m = m;
          cur_bias = (m == c) ? 0.f : ((full || mask_bit(mask, m)) ? srow[m] - lses : kNegInf);
          cur_g = 1.f;
          if (outer && m != c && cur_bias != kNegInf) {
            cur_g = exp_hw(cur_bias);
            cur_bias = 0.f;
          }
        }
        if (cur_bias == kNegInf) continue;
        float dot = 0.f, dpp = 0.f;
        for (int i = 0; i < DS; ++i) {
          dot = fmaf(qv[i], ks[jj][p * DS + i], dot);
          dpp = fmaf(dov[i], vs[jj][p * DS + i], dpp);
        }
        const float z = quad_sum(dot) * scale + cur_bias;
        const float pr = exp_hw(z - lrow);
        const float gdp = cur_g * quad_sum(dpp);
        const float dz = pr * (gdp - drow);
        for (int i = 0; i < DS; ++i) dqa[i] = fmaf(scale * dz, ks[jj][p * DS + i], dqa[i]);
        db_cur += outer ? pr * gdp : dz;  // outer gate: g dg in dbeta's place
      }
    }
    __syncthreads();
  }
  if (rv) {
    if (cur_m >= 0 && cur_m < c && cur_bias != kNegInf) {
      db_total += db_cur;
      if ((cur_m & 3) == p) dsrow[cur_m] = db_cur;
    }
    for (int i = 0; i < DS; ++i) dq[row * D + p * DS + i] = from_f32<T>(dqa[i]);
  }
  __threadfence();
  if (rv) {
    for (int m = p; m < C; m += 4) {
      float out = 0.f;
      if (m < c) {
        const float db = (full || mask_bit(mask, m)) ? dsrow[m] : 0.f;
        out = gate_ds(gate, db, srow[m] - lses, db_total);
      }
      dsrow[m] = out;
    }
  }
}

// dk and dv, key-major: four lanes per key, every query row of the G heads of
// the KV head that can attend the key (rows t >= j).
template <typename T, int D>
__global__ __launch_bounds__(128) void bwd_dkdv_simt_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const float* __restrict__ scores, const int32_t* __restrict__ idx,
    const float* __restrict__ lse, const float* __restrict__ lse_s,
    const float* __restrict__ delta, T* __restrict__ dk, T* __restrict__ dv, int Hq, int Hkv,
    int N, int C, int block, int topk, float scale, int outer) {
  constexpr int DS = D / 4;
  constexpr int RT = 32;  // query rows per LDS tile
  __shared__ float qs[RT][D + 1];
  __shared__ float dos[RT][D + 1];
  __shared__ float rlse[RT], rdelta[RT];
  __shared__ float rbias[RT][KT];
  __shared__ float rgate[RT][KT];  // outer gate: g of (row, block), else 1
  const int tile = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv;
  const int kk = threadIdx.x >> 2, p = threadIdx.x & 3;
  const int j = tile * KT + kk;
  const bool kv = j < N;
  const size_t krow = (size_t(b) * Hkv + g) * N + (kv ? j : 0);
  float kvv[DS], vvv[DS], dka[DS], dva[DS];
  for (int i = 0; i < DS; ++i) {
    kvv[i] = kv ? to_f32(k[krow * D + p * DS + i]) : 0.f;
    vvv[i] = kv ? to_f32(v[krow * D + p * DS + i]) : 0.f;
    dka[i] = 0.f;
    dva[i] = 0.f;
  }
  const int j0 = tile * KT;
  const int m_first = j0 / block;
  const int m_last = (min(N, j0 + KT) - 1) / block;
  const int nb = m_last - m_first + 1;
  for (int h = g * G; h < (g + 1) * G; ++h) {
    for (int r0 = j0; r0 < N; r0 += RT) {
      __syncthreads();
      for (int i = threadIdx.x; i < RT * D; i += blockDim.x) {
        const int rr = i / D, d = i % D;
        const int t = r0 + rr;
        const size_t row = (size_t(b) * Hq + h) * N + t;
        qs[rr][d] = t < N ? to_f32(q[row * D + d]) : 0.f;
        dos[rr][d] = t < N ? to_f32(dout[row * D + d]) : 0.f;
      }
      for (int i = threadIdx.x; i < RT; i += blockDim.x) {
        const int t = r0 + i;
        const size_t row = (size_t(b) * Hq + h) * N + t;
        rlse[i] = t < N ? lse[row] : 0.f;
        rdelta[i] = t < N ? delta[row] : 0.f;
      }
      for (int i = threadIdx.x; i < RT * nb; i += blockDim.x) {
        const int rr = i / nb, mb = i % nb;
        const int t = r0 + rr, m = m_first + mb;
        float bias = kNegInf, gt = 1.f;
        if (t < N) {
          const int c = t / block;
          const size_t row = (size_t(b) * Hq + h) * N + t;
          if (m == c) {
            bias = 0.f;
          } else if (m < c) {
            bool sel = (idx == nullptr);
            if (!sel) {
              const int32_t* ir = idx + ((size_t(b) * Hkv + g) * N + t) * topk;
              for (int e = 0; e < topk && !sel; ++e) sel = (ir[e] == m);
            }
            if (sel) bias = scores[row * C + m] - lse_s[row];
            if (sel && outer) {
              gt = exp_hw(bias);
              bias = 0.f;
            }
          }
        }
        rbias[rr][mb] = bias;
        rgate[rr][mb] = gt;
      }
      __syncthreads();
      if (kv) {
        for (int rr = 0; rr < RT; ++rr) {
          const int t = r0 + rr;
          if (t >= N) break;
          if (t < j) continue;
          const float bias = rbias[rr][j / block - m_first];
          const float gt = rgate[rr][j / block - m_first];
          if (bias == kNegInf) continue;
          float dot = 0.f, dpp = 0.f;
          for (int i = 0; i < DS; ++i) {
            dot = fmaf(qs[rr][p * DS + i], kvv[i], dot);
            dpp = fmaf(dos[rr][p * DS + i], vvv[i], dpp);
          }
          const float z = quad_sum(dot) * scale + bias;
          const float pr = exp_hw(z - rlse[rr]);
          const float dz = pr * (gt * quad_sum(dpp) - rdelta[rr]);
          const float pg = pr * gt;
          for (int i = 0; i < DS; ++i) {
            dva[i] = fmaf(pg, dos[rr][p * DS + i], dva[i]);
            dka[i] = fmaf(scale * dz, qs[rr][p * DS + i], dka[i]);
          }
        }
      }
    }
  }
  if (kv) {
    for (int i = 0; i < DS; ++i) {
      dk[krow * D + p * DS + i] = from_f32<T>(dka[i]);
      dv[krow * D + p * DS + i] = from_f32<T>(dva[i]);
    }
  }
}

template <typename T, int D>
hipError_t fwd_simt(const void* q, const void* k, const void* v, const float* scores,
                    const int32_t* idx, void* o, float* lse, float* lse_s, const Dims& d, int topk,
                    float scale, int norm, bool outer, hipStream_t s) {
  const size_t mask_bytes = idx ? size_t(64) * ((d.C + 31) / 32) * 4 : 0;
  dim3 grid((d.N + 63) / 64, d.Hq, d.B);
  SAS_LAUNCH("fwd_simt", (fwd_simt_kernel<T, D>), grid, dim3(256), mask_bytes, s, (const T*)q,
                     (const T*)k, (const T*)v, scores, idx, (T*)o, lse, lse_s, d.Hq, d.Hkv, d.N,
                     d.C, d.block, topk, scale, norm, int(outer));
  return hipGetLastError();
}

template <typename T, int D>
hipError_t bwd_simt(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* scores, const int32_t* idx, const float* lse, const float* lse_s,
                    void* dq, void* dk, void* dv, float* ds, const Dims& d, int topk, float scale,
                    int gate, float* delta, hipStream_t s) {
  const size_t rows = size_t(d.B) * d.Hq * d.N;
  SAS_LAUNCH("bwd_delta", (bwd_delta_kernel<T, D>), dim3((rows + 63) / 64), dim3(256), 0, s,
                     (const T*)o, (const T*)dout, delta, rows);
  const size_t mask_bytes = idx ? size_t(64) * ((d.C + 31) / 32) * 4 : 0;
  SAS_LAUNCH("bwd_dq_simt", (bwd_dq_simt_kernel<T, D>), dim3((d.N + 63) / 64, d.Hq, d.B), dim3(256),
                     mask_bytes, s, (const T*)q, (const T*)k, (const T*)v, (const T*)dout, scores,
                     idx, lse, lse_s, delta, (T*)dq, ds, d.Hq, d.Hkv, d.N, d.C, d.block, topk,
                     scale, gate);
  SAS_LAUNCH("bwd_dkdv_simt", (bwd_dkdv_simt_kernel<T, D>), dim3((d.N + KT - 1) / KT, d.Hkv, d.B),
                     dim3(128), 0, s, (const T*)q, (const T*)k, (const T*)v, (const T*)dout,
                     scores, idx, lse, lse_s, delta, (T*)dk, (T*)dv, d.Hq, d.Hkv, d.N, d.C,
                     d.block, topk, scale, int(gate == kGateOuter));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_simt(const void* q, const void* k, const void* v, const float* scores,
                           const int32_t* idx, void* o, float* lse, float* lse_s, const Dims& d,
                           int topk, float scale, bool bf16, int norm, bool outer, hipStream_t s) {
  if (bf16) {
    if (d.D == 64) return fwd_simt<bf16_t, 64>(q, k, v, scores, idx, o, lse, lse_s, d, topk, scale, norm, outer, s);
    return fwd_simt<bf16_t, 128>(q, k, v, scores, idx, o, lse, lse_s, d, topk, scale, norm, outer, s);
  }
  if (d.D == 64) return fwd_simt<float, 64>(q, k, v, scores, idx, o, lse, lse_s, d, topk, scale, norm, outer, s);
  return fwd_simt<float, 128>(q, k, v, scores, idx, o, lse, lse_s, d, topk, scale, norm, outer, s);
}

hipError_t launch_bwd_simt(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* scores, const int32_t* idx,
                           const float* lse, const float* lse_s, void* dq, void* dk, void* dv,
                           float* ds, const Dims& d, int topk, float scale, bool bf16, int gate,
                           float* delta, hipStream_t s) {
  if (bf16) {
    if (d.D == 64)
      return bwd_simt<bf16_t, 64>(q, k, v, o, dout, scores, idx, lse, lse_s, dq, dk, dv, ds, d, topk, scale, gate, delta, s);
    return bwd_simt<bf16_t, 128>(q, k, v, o, dout, scores, idx, lse, lse_s, dq, dk, dv, ds, d, topk, scale, gate, delta, s);
  }
  if (d.D == 64)
    return bwd_simt<float, 64>(q, k, v, o, dout, scores, idx, lse, lse_s, dq, dk, dv, ds, d, topk, scale, gate, delta, s);
  return bwd_simt<float, 128>(q, k, v, o, dout, scores, idx, lse, lse_s, dq, dk, dv, ds, d, topk, scale, gate, delta, s);
}

}  // namespace sas
