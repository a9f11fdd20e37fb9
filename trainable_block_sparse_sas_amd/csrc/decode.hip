// Sparse decode: the new token of each sequence attends to its current block
// plus the selected history blocks, with no gate (jaehun.me review, "A
// Concrete Walkthrough", Step 6 / paper Alg. 2; block-sparse attention of the
// blog's 问题动机 section and review "Background", paper Eq. 2).  Without idx
// every history block is attended (dense decode).
//
// Work is split per attended block: a workgroup streams EPW blocks of one
// (sequence, KV head), keeps an online softmax for the G query heads of the
// group and writes a partial (max, sum, acc[D]) per head.  A second kernel
// merges the partials by their log-sum-exp.  K rows are read with 16-byte
// lane loads (four lanes per key, D/4 columns each); V is read row by row,
// one 4-byte column pair per lane, so every wave load covers whole rows.
#include "common.h"
#include "internal.h"

namespace sas {
namespace {

constexpr int kMaxG = 16;
constexpr int kKeys = 64;  // keys per LDS step

struct DecodeArgs {
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* cache_len;
  const int32_t* idx;
  float* part;  // [B, Hkv, P, G, D + 2]
  int Hq, Hkv, L, D, block, topk, C, EPW, P;
  float scale;
};

// Resolves attended entry e of (b, g) into a block index, or -1 when the
// entry is empty (invalid / repeated idx entry, beyond the dense range).
__device__ __forceinline__ int entry_block(const DecodeArgs& a, int b, int g, int e, int c) {
  if (a.idx == nullptr) {
    return e <= c ? e : -1;  // blocks 0..c-1, then the current block c
  }
  if (e == a.topk) return c;  // the current block
  if (e > a.topk) return -1;
  const int32_t* ir = a.idx + (size_t(b) * a.Hkv + g) * a.topk;
  const int m = ir[e];
  if (m < 0 || m >= c) return -1;
  for (int e2 = 0; e2 < e; ++e2)
    if (ir[e2] == m) return -1;
  return m;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_partial_kernel(DecodeArgs a) {
  constexpr int DQ = D / 4;   // K columns per lane (4 lanes per key)
  constexpr int DV = D / 64;  // V columns per lane (one wave per row)
  __shared__ float qsh[kMaxG][D];
  __shared__ float sc[kMaxG][kKeys];
  __shared__ float red[4][kMaxG][D];
  __shared__ float run_m[kMaxG], run_l[kMaxG], alpha_sh[kMaxG];
  const int part_i = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = a.Hq / a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int len = a.cache_len[b];
  len = len > a.L ? a.L : len;
  const int pos = len - 1;
  const int c = len > 0 ? pos / a.block : 0;
  const T* qb = reinterpret_cast<const T*>(a.q) + (size_t(b) * a.Hq + g * G) * D;
  for (int i = tid; i < G * D; i += 256) qsh[i / D][i % D] = to_f32(qb[i]);
  if (tid < kMaxG) {
    run_m[tid] = kNegInf;
    run_l[tid] = 0.f;
  }
  const T* kbase = reinterpret_cast<const T*>(a.kc) + (size_t(b) * a.Hkv + g) * size_t(a.L) * D;
  const T* vbase = reinterpret_cast<const T*>(a.vc) + (size_t(b) * a.Hkv + g) * size_t(a.L) * D;
  float acc[kMaxG][DV];
  for (int h = 0; h < kMaxG; ++h)
    for (int i = 0; i < DV; ++i) acc[h][i] = 0.f;
  __syncthreads();

  const int key = tid >> 2, quarter = tid & 3;
  for (int ei = 0; ei < a.EPW; ++ei) {
    const int e = part_i * a.EPW + ei;
    const int m = len > 0 ? entry_block(a, b, g, e, c) : -1;
    if (m < 0) continue;  // uniform across the workgroup
    const int j_begin = m * a.block;
    const int j_end = (m == c) ? pos + 1 : j_begin + a.block;
    for (int j0 = j_begin; j0 < j_end; j0 += kKeys) {
      // Scores: lanes 4*key .. 4*key+3 hold one key's D columns in quarters.
      const int j = j0 + key;
      float kv[DQ];
      if (j < j_end) {
        const T* kr = kbase + size_t(j) * D + quarter * DQ;
        for (int i = 0; i < DQ; i += 16 / int(sizeof(T))) {
          const uint4 raw = *reinterpret_cast<const uint4*>(kr + i);
          const T* pv = reinterpret_cast<const T*>(&raw);
          for (int u = 0; u < int(16 / sizeof(T)); ++u) kv[i + u] = to_f32(pv[u]);
        }
      } else {
        for (int i = 0; i < DQ; ++i) kv[i] = 0.f;
      }
      for (int h = 0; h < G; ++h) {
        float s = 0.f;
        for (int i = 0; i < DQ; ++i) s = fmaf(qsh[h][quarter * DQ + i], kv[i], s);
        s += shfl_xor(s, 1);
        s += shfl_xor(s, 2);
        if (quarter == 0) sc[h][key] = (j < j_end) ? s * a.scale : kNegInf;
      }
      __syncthreads();
      // Online softmax step: wave w handles heads w, w+4, ...; lane = key.
      for (int h = wave; h < G; h += 4) {
        const float x = sc[h][lane];
        float mx = x;
        for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, shfl_xor(mx, off));
        const float pm = run_m[h];
        const float nm = fmaxf(pm, mx);  // finite: every step holds >= 1 key
        const float p = exp_hw(x - nm);
        float ps = p;
        for (int off = 32; off >= 1; off >>= 1) ps += shfl_xor(ps, off);
        sc[h][lane] = p;
        if (lane == 0) {
          const float al = exp_hw(pm - nm);
          alpha_sh[h] = al;
          run_m[h] = nm;
          run_l[h] = run_l[h] * al + ps;
        }
      }
      __syncthreads();
      // Values: wave w covers keys w, w+4, ...; each lane DV adjacent columns.
      for (int h = 0; h < G; ++h) {
        const float al = alpha_sh[h];
        for (int i = 0; i < DV; ++i) acc[h][i] *= al;
      }
      for (int kk = wave; kk < kKeys; kk += 4) {
        const int jv = j0 + kk;
        if (jv >= j_end) break;
        const T* vr = vbase + size_t(jv) * D + lane * DV;
        float vv[DV];
        for (int i = 0; i < DV; ++i) vv[i] = to_f32(vr[i]);
        for (int h = 0; h < G; ++h) {
          const float p = sc[h][kk];
          for (int i = 0; i < DV; ++i) acc[h][i] = fmaf(p, vv[i], acc[h][i]);
        }
      }
      __syncthreads();
    }
  }
  // Reduce the four waves' accumulators and write the partial.
  for (int h = 0; h < G; ++h)
    for (int i = 0; i < DV; ++i) red[wave][h][lane * DV + i] = acc[h][i];
  __syncthreads();
  float* out = a.part + ((size_t(b) * a.Hkv + g) * a.P + part_i) * G * (D + 2);
  for (int i = tid; i < G * D; i += 256) {
    const int h = i / D, d = i % D;
    out[h * (D + 2) + 2 + d] = red[0][h][d] + red[1][h][d] + red[2][h][d] + red[3][h][d];
  }
  if (tid < G) {
    out[tid * (D + 2) + 0] = run_m[tid];
    out[tid * (D + 2) + 1] = run_l[tid];
  }
}

// Merge the P partials of each (b, query head) by log-sum-exp.
template <typename T, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(const float* __restrict__ part,
                                                         T* __restrict__ o,
                                                         float* __restrict__ lse, int Hq, int Hkv,
                                                         int P) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int G = Hq / Hkv, g = h / G, hh = h % G;
  const int d = threadIdx.x;
  const float* base = part + (size_t(b) * Hkv + g) * P * G * (D + 2) + hh * (D + 2);
  const size_t stride = size_t(G) * (D + 2);
  float M = kNegInf;
  for (int p = 0; p < P; ++p) M = fmaxf(M, base[p * stride]);
  float L = 0.f, acc = 0.f;
  if (M != kNegInf) {
    for (int p = 0; p < P; ++p) {
      const float mp = base[p * stride];
      if (mp == kNegInf) continue;
      const float w = exp_hw(mp - M);
      L = fmaf(base[p * stride + 1], w, L);
      acc = fmaf(base[p * stride + 2 + d], w, acc);
    }
  }
  const size_t orow = size_t(b) * Hq + h;
  o[orow * D + d] = from_f32<T>(M == kNegInf ? 0.f : acc / L);
  if (lse && d == 0) lse[orow] = (M == kNegInf) ? kNegInf : M + log_hw(L);
}

void decode_plan(int B, int Hkv, int L_max, int block, int topk, int* entries, int* epw, int* P) {
  const int C = L_max / block;
  const int E = topk >= 0 ? topk + 1 : C + 1;  // attended entries per (b, g)
  // Aim for a few thousand workgroups in total; one block per workgroup when
  // that already gives enough parallelism.
  const long target = 2048;
  long groups = long(B) * Hkv;
  int w = int((long(E) * groups + target - 1) / target);
  if (w < 1) w = 1;
  *entries = E;
  *epw = w;
  *P = (E + w - 1) / w;
}

template <typename T, int D>
hipError_t decode_t(const DecodeArgs& a0, int B, T* o, float* lse, hipStream_t s) {
  DecodeArgs a = a0;
  dim3 grid(a.P, a.Hkv, B);
  hipLaunchKernelGGL((decode_partial_kernel<T, D>), grid, dim3(256), 0, s, a);
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(a.Hq, B), dim3(D), 0, s, a.part, o, lse,
                     a.Hq, a.Hkv, a.P);
  return hipGetLastError();
}

}  // namespace

size_t decode_workspace(int B, int Hq, int Hkv, int L_max, int D, int block, int topk) {
  int E, w, P;
  decode_plan(B, Hkv, L_max, block, topk, &E, &w, &P);
  return align_up(size_t(B) * Hq * P * (D + 2) * sizeof(float));
}

hipError_t launch_decode(const void* q, const void* kc, const void* vc, const int32_t* cache_len,
                         const int32_t* idx, void* o, float* lse, int B, int Hq, int Hkv,
                         int L_max, int D, int block, int topk, float scale, bool bf16, void* ws,
                         hipStream_t s) {
  if (B == 0 || Hq == 0) return hipSuccess;
  int E, w, P;
  decode_plan(B, Hkv, L_max, block, idx ? topk : -1, &E, &w, &P);
  DecodeArgs a{q, kc, vc, cache_len, idx, (float*)ws, Hq, Hkv, L_max, D, block,
               idx ? topk : 0, L_max / block, w, P, scale};
  if (bf16) {
    if (D == 64) return decode_t<bf16_t, 64>(a, B, (bf16_t*)o, lse, s);
    return decode_t<bf16_t, 128>(a, B, (bf16_t*)o, lse, s);
  }
  if (D == 64) return decode_t<float, 64>(a, B, (float*)o, lse, s);
  return decode_t<float, 128>(a, B, (float*)o, lse, s);
}

}  // namespace sas
