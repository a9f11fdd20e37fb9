// SAS gated attention backward on the matrix cores (bf16 in, fp32 accumulate).
//
// With P = softmax(z), Delta = rowsum(dO * o) and dZ = P * (dO V^T - Delta):
//   dq = scale dZ K,  dk = scale dZ^T Q,  dv = P^T dO,
//   dbeta[t,m] = sum of dZ over the keys of gated history block m (the inner
//   gate gradient of the blog's 方法核心 section / jaehun.me review "Why the Four
//   Design Choices Matter", paper Eq. 5, times g), and
//   ds[t,m] = dbeta[t,m] - g[t,m] * sum_m' dbeta[t,m'] through log g = s - LSE(s).
// The review's kernel paragraph ("A Concrete Walkthrough") describes the
// block-wise aggregation of the log-gate gradient.
//
// Three kernels:
//   prep  Delta per row, and (sparse scope) a per-token bitmask of selected blocks.
//   dkdv  KV-major: a workgroup owns one block (64 keys, 16 per wave) of one KV
//         head and streams the query rows that attend it, 32 rows per step: the
//         own block's rows (causal) and every later row that gates the block
//         (full scope: all of them; sparse scope: the tokens whose bitmask holds
//         the block, compacted on the fly so no step carries an idle row).
//         Lane = key layout (S = Q K^T), so dV = P^T dO and dK = dS^T Q
//         contract over rows with P and dS straight from registers.
//   dq    query-major like the forward (lane = row, S^T = K Q^T), recomputing P
//         and dP^T = V dO^T per tile; dQ^T += K^T dS^T; dbeta is a lane-local
//         row sum written per (row, block), then the dense ds epilogue.
#include "common.h"
#include "internal.h"
#include "mfma.h"

namespace sas {
namespace {

constexpr int KT = 64;
constexpr int PAD = 8;

struct BwdArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  const bf16_t* o;
  const bf16_t* dout;
  const float* scores;
  const int32_t* idx;
  const float* lse;
  const float* lse_s;
  bf16_t* dq;
  bf16_t* dk;
  bf16_t* dv;
  float* ds;
  float* delta;      // workspace [B, Hq, N]
  uint32_t* selbits; // workspace [B, Hkv, N, MWB] (sparse)
  int Hq, Hkv, N, C, topk, MWB, n_tiles, n_pairs;
  float scale;
};

// ---------------------------------------------------------------- prep ------
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_mfma_kernel(const bf16_t* __restrict__ o,
                                                             const bf16_t* __restrict__ dout,
                                                             float* __restrict__ delta, size_t rows) {
  constexpr int LPR = D / 8;  // lanes per row, 16-byte loads
  const size_t row = size_t(blockIdx.x) * (256 / LPR) + threadIdx.x / LPR;
  const int sub = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const uint4 a = *reinterpret_cast<const uint4*>(o + row * D + sub * 8);
    const uint4 b = *reinterpret_cast<const uint4*>(dout + row * D + sub * 8);
    const uint32_t* aw = reinterpret_cast<const uint32_t*>(&a);
    const uint32_t* bw = reinterpret_cast<const uint32_t*>(&b);
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(bf16_lo(aw[i]), bf16_lo(bw[i]), acc);
      acc = fmaf(bf16_hi(aw[i]), bf16_hi(bw[i]), acc);
    }
  }
  for (int off = LPR / 2; off >= 1; off >>= 1) acc += shfl_xor(acc, off);
  if (row < rows && sub == 0) delta[row] = acc;
}

// One wave per token: bitmask of the token's valid selected blocks.
__global__ __launch_bounds__(256) void selbits_kernel(const int32_t* __restrict__ idx,
                                                      uint32_t* __restrict__ bits, int N, int topk,
                                                      int MWB, size_t tokens) {
  const size_t tok = size_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (tok >= tokens) return;
  const int t = int(tok % N);
  const int c = t / KT;
  const int32_t* ir = idx + tok * topk;
  for (int w0 = 0; w0 < MWB; w0 += 64) {
    const int w = w0 + lane;
    uint32_t word = 0;
    for (int e = 0; e < topk; ++e) {
      const int m = ir[e];
      if (m >= 0 && m < c && (m >> 5) == w) word |= 1u << (m & 31);
    }
    if (w < MWB) bits[tok * MWB + w] = word;
  }
}

// --------------------------------------------------------------- dK / dV ----
template <int D, int G, bool SPARSE>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int KS = D / 32;
  constexpr int ND = D / 16;
  constexpr int CH = D / 8;
  constexpr int RS = 32;       // rows per step
  constexpr int TPS = RS / G;  // tokens per step
  constexpr int QCAP = 256 + TPS;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[2][RS][D + PAD];
  __shared__ __attribute__((aligned(16))) uint16_t dOs[2][RS][D + PAD];
  __shared__ __attribute__((aligned(16))) uint16_t Qt[2][D][RS + PAD];
  __shared__ __attribute__((aligned(16))) uint16_t dOt[2][D][RS + PAD];
  __shared__ float r_lse[2][RS], r_del[2][RS], r_bias[2][RS];
  __shared__ int r_tok[2][RS];
  __shared__ int queue[QCAP];
  __shared__ int q_count, q_wave[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  int tile, pair;
  xcd_order(blockIdx.x, a.n_tiles, a.n_pairs, &tile, &pair);
  const int m = a.n_tiles - 1 - tile;  // lowest blocks (most rows) first
  const int b = pair / a.Hkv, g = pair % a.Hkv;
  const int N = a.N, C = a.C;
  const int j0 = m * KT;
  const int my_key = j0 + wave * 16 + lr;  // this lane's key (B operand rows)
  const float c1 = a.scale * kLog2e;

  // Stationary K and V fragments: lane holds key my_key, columns 32ks + 8lq.
  uint4 kf[KS], vf[KS];
  {
    const size_t kr = (size_t(b) * a.Hkv + g) * N + (my_key < N ? my_key : 0);
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = my_key < N ? *reinterpret_cast<const uint4*>(a.k + kr * D + ks * 32 + lq * 8) : make_uint4(0, 0, 0, 0);
      vf[ks] = my_key < N ? *reinterpret_cast<const uint4*>(a.v + kr * D + ks * 32 + lq * 8) : make_uint4(0, 0, 0, 0);
    }
  }
  f32x4 dk[ND], dv[ND];
  for (int nd = 0; nd < ND; ++nd) {
    dk[nd] = f32x4{0.f, 0.f, 0.f, 0.f};
    dv[nd] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Row loader: rows of one step -> registers, then LDS (row-major + transposed).
  uint4 rq[4];
  float rs_lse = 0.f, rs_del = 0.f, rs_bias = kNegInf;
  int rs_tok = -1;
  auto load_rows = [&](const int* toks, int ntok) {
    // threads 0..127: Q rows; 128..255: dO rows; 4 rows x one 16-byte chunk each
    const int half = tid >> 7, u = tid & 127;
    const int rg = u / CH, c8 = u % CH;
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * rg + r;
      rq[r] = make_uint4(0, 0, 0, 0);
      if (rg < RS / 4) {
        const int ti = row / G;
        if (ti < ntok) {
          const int t = toks[ti];
          const size_t gr = (size_t(b) * a.Hq + g * G + row % G) * N + t;
          const bf16_t* src = half ? a.dout : a.q;
          rq[r] = *reinterpret_cast<const uint4*>(src + gr * D + c8 * 8);
        }
      }
    }
    if (tid < RS) {
      const int ti = tid / G;
      rs_tok = -1;
      rs_bias = kNegInf;
      rs_lse = 0.f;
      rs_del = 0.f;
      if (ti < ntok) {
        const int t = toks[ti];
        const size_t gr = (size_t(b) * a.Hq + g * G + tid % G) * N + t;
        rs_tok = t;
        rs_lse = a.lse[gr] * kLog2e;
        rs_del = a.delta[gr];
        rs_bias = (t / KT == m) ? 0.f : (a.scores[gr * C + m] - a.lse_s[gr]) * kLog2e;
      }
    }
  };
  auto store_rows = [&](int buf) {
    const int half = tid >> 7, u = tid & 127;
    const int rg = u / CH, c8 = u % CH;
    if (rg < RS / 4) {
      uint16_t(*rm)[D + PAD] = half ? dOs[buf] : Qs[buf];
      uint16_t(*tr)[RS + PAD] = half ? dOt[buf] : Qt[buf];
      for (int r = 0; r < 4; ++r) *reinterpret_cast<uint4*>(&rm[4 * rg + r][c8 * 8]) = rq[r];
      const int kap = (4 * rg) & 31;
      const int phys = ((4 * rg) & ~31) + 8 * ((kap >> 2) & 3) + 4 * (kap >> 4);
      const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&rq[0]);
      const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&rq[1]);
      const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&rq[2]);
      const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&rq[3]);
      for (int d2 = 0; d2 < 4; ++d2) {
        const uint32_t lo0 = (w0[d2] & 0xffffu) | (w1[d2] << 16);
        const uint32_t lo1 = (w2[d2] & 0xffffu) | (w3[d2] << 16);
        const uint32_t hi0 = (w0[d2] >> 16) | (w1[d2] & 0xffff0000u);
        const uint32_t hi1 = (w2[d2] >> 16) | (w3[d2] & 0xffff0000u);
        *reinterpret_cast<uint2*>(&tr[c8 * 8 + 2 * d2][phys]) = make_uint2(lo0, lo1);
        *reinterpret_cast<uint2*>(&tr[c8 * 8 + 2 * d2 + 1][phys]) = make_uint2(hi0, hi1);
      }
    }
    if (tid < RS) {
      r_lse[buf][tid] = rs_lse;
      r_del[buf][tid] = rs_del;
      r_bias[buf][tid] = rs_bias;
      r_tok[buf][tid] = rs_tok;
    }
  };
  auto compute_step = [&](int buf) {
    f32x4 sacc[2], dpacc[2];
    for (int s = 0; s < 2; ++s) {
      sacc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
      dpacc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int ks = 0; ks < KS; ++ks) {
      for (int s = 0; s < 2; ++s) {
        const uint4 qa = *reinterpret_cast<const uint4*>(&Qs[buf][16 * s + lr][ks * 32 + lq * 8]);
        const uint4 da = *reinterpret_cast<const uint4*>(&dOs[buf][16 * s + lr][ks * 32 + lq * 8]);
        sacc[s] = mfma16(qa, kf[ks], sacc[s]);
        dpacc[s] = mfma16(da, vf[ks], dpacc[s]);
      }
    }
    // C layout: lane holds key my_key (column lr), rows 16s + 4lq + i.
    float p[2][4], dsv[2][4];
    for (int s = 0; s < 2; ++s)
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * s + 4 * lq + i;
        const int t = r_tok[buf][row];
        float pv = 0.f;
        if (t >= 0 && my_key <= t && my_key < N) {
          pv = exp2_hw(sacc[s][i] * c1 + r_bias[buf][row] - r_lse[buf][row]);
        }
        p[s][i] = pv;
        dsv[s][i] = pv * (dpacc[s][i] - r_del[buf][row]);
      }
    uint4 pa, da;
    pa.x = pack_bf16(p[0][0], p[0][1]);
    pa.y = pack_bf16(p[0][2], p[0][3]);
    pa.z = pack_bf16(p[1][0], p[1][1]);
    pa.w = pack_bf16(p[1][2], p[1][3]);
    da.x = pack_bf16(dsv[0][0], dsv[0][1]);
    da.y = pack_bf16(dsv[0][2], dsv[0][3]);
    da.z = pack_bf16(dsv[1][0], dsv[1][1]);
    da.w = pack_bf16(dsv[1][2], dsv[1][3]);
    for (int nd = 0; nd < ND; ++nd) {
      const uint4 ob = *reinterpret_cast<const uint4*>(&dOt[buf][16 * nd + lr][lq * 8]);
      const uint4 qb = *reinterpret_cast<const uint4*>(&Qt[buf][16 * nd + lr][lq * 8]);
      dv[nd] = mfma16(pa, ob, dv[nd]);
      dk[nd] = mfma16(da, qb, dk[nd]);
    }
  };

  // Steps: a list of token groups of TPS tokens.  The own block's tokens first,
  // then (full scope) every later token or (sparse) the later tokens that
  // selected block m, compacted through the queue.
  int buf = 0;
  bool have = false;  // a step is staged in LDS buffer `buf`
  auto run_tokens = [&](const int* toks, int ntok) {
    // Enqueue one step: prefetch to registers; compute the staged step; store.
    load_rows(toks, ntok);
    if (have) compute_step(buf);
    store_rows(have ? buf ^ 1 : buf);
    __syncthreads();
    if (have) buf ^= 1;
    have = true;
  };

  __shared__ int own_toks[KT];
  const int own_n = min(KT, N - j0);
  if (tid < KT) own_toks[tid] = j0 + tid;
  __syncthreads();
  for (int s0 = 0; s0 < own_n; s0 += TPS) run_tokens(own_toks + s0, min(TPS, own_n - s0));

  if (!SPARSE) {
    __shared__ int seq_toks[TPS];
    for (int t0 = j0 + KT; t0 < N; t0 += TPS) {
      if (tid < TPS) seq_toks[tid] = t0 + tid;
      __syncthreads();
      run_tokens(seq_toks, min(TPS, N - t0));
    }
  } else {
    if (tid == 0) q_count = 0;
    __syncthreads();
    const uint32_t* bits = a.selbits + (size_t(b) * a.Hkv + g) * size_t(N) * a.MWB;
    const int word = m >> 5;
    const uint32_t bit = 1u << (m & 31);
    for (int t0 = j0 + KT; t0 < N; t0 += 256) {
      const int t = t0 + tid;
      const bool sel = t < N && (bits[size_t(t) * a.MWB + word] & bit);
      const unsigned long long bal = __ballot(sel);
      if (lane == 0) q_wave[wave] = __popcll(bal);
      __syncthreads();
      int base = q_count;
      for (int w = 0; w < wave; ++w) base += q_wave[w];
      const unsigned long long lt = lane ? (~0ull >> (64 - lane)) : 0ull;
      if (sel) queue[base + __popcll(bal & lt)] = t;
      __syncthreads();
      int total = q_count + q_wave[0] + q_wave[1] + q_wave[2] + q_wave[3];
      int done = 0;
      while (total - done >= TPS) {
        run_tokens(queue + done, TPS);
        done += TPS;
      }
      // keep the remainder at the front of the queue
      const int rem = total - done;
      int keep = 0;
      if (tid < rem) keep = queue[done + tid];
      __syncthreads();
      if (tid < rem) queue[tid] = keep;
      if (tid == 0) q_count = rem;
      __syncthreads();
    }
    if (q_count > 0) run_tokens(queue, q_count);
  }
  if (have) compute_step(buf);

  // Write dK (scaled) and dV: lane holds column 16nd + lr, keys 4lq + i of the
  // wave's 16 keys.
  for (int i = 0; i < 4; ++i) {
    const int key = j0 + wave * 16 + 4 * lq + i;
    if (key >= N) continue;
    const size_t kr = ((size_t(b) * a.Hkv + g) * N + key) * D;
    for (int nd = 0; nd < ND; ++nd) {
      a.dk[kr + 16 * nd + lr] = f32_to_bf16(dk[nd][i] * a.scale);
      a.dv[kr + 16 * nd + lr] = f32_to_bf16(dv[nd][i]);
    }
  }
}

// -------------------------------------------------------------------- dQ ----
template <int D, int G, int NSUB, int WAVES, bool SPARSE>
__global__ __launch_bounds__(64 * WAVES, 2) void bwd_dq_kernel(BwdArgs a) {
  constexpr int NT = 64 * WAVES;
  constexpr int KS = D / 32;
  constexpr int MD = D / 16;
  constexpr int TOK_SUB = 16 / G;
  constexpr int ROWS_WG = 16 * NSUB * WAVES;
  constexpr int TOK_WG = ROWS_WG / G;
  constexpr int CH = D / 8;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[KT][D + PAD];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[KT][D + PAD];
  __shared__ __attribute__((aligned(16))) uint16_t Kt[D][KT + PAD];
  extern __shared__ int32_t dyn[];  // sparse: union mask | sorted idx | raw idx

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  int tile, pair;
  xcd_order(blockIdx.x, a.n_tiles, a.n_pairs, &tile, &pair);
  const int b = pair / a.Hkv, g = pair % a.Hkv;
  const int N = a.N, C = a.C;
  const int t_wg0 = tile * TOK_WG;
  const float c1 = a.scale * kLog2e;

  int row_t[NSUB], row_h[NSUB], c_sub[NSUB];
  bool sub_live[NSUB];
  for (int s = 0; s < NSUB; ++s) {
    const int sg = wave * NSUB + s;
    const int t0 = t_wg0 + sg * TOK_SUB;
    row_t[s] = t0 + lr / G;
    row_h[s] = g * G + lr % G;
    c_sub[s] = t0 / KT;
    sub_live[s] = t0 < N;
  }

  const int MW = (C + 32) >> 5;
  int32_t* umask = dyn;
  int32_t* sorted = dyn + MW;
  int32_t* raw = sorted + TOK_WG * a.topk;
  float* beta = reinterpret_cast<float*>(raw + TOK_WG * a.topk);  // [ROWS_WG][topk] (sparse)
  if (SPARSE) {
    for (int i = tid; i < MW; i += NT) umask[i] = 0;
    for (int i = tid; i < TOK_WG * a.topk; i += NT) {
      const int tok = i / a.topk, e = i % a.topk;
      const int t = t_wg0 + tok;
      int mm = -1;
      if (t < N) {
        mm = a.idx[((size_t(b) * a.Hkv + g) * N + t) * a.topk + e];
        if (mm < 0 || mm >= t / KT) mm = -1;
      }
      raw[i] = mm < 0 ? 0x7fffffff : mm;
    }
    __syncthreads();
    for (int i = tid; i < TOK_WG * a.topk; i += NT) {
      const int tok = i / a.topk, e = i % a.topk;
      const int32_t* rr = raw + tok * a.topk;
      const int mm = rr[e];
      int rank = 0;
      for (int e2 = 0; e2 < a.topk; ++e2) {
        const int m2 = rr[e2];
        rank += (m2 < mm) || (m2 == mm && e2 < e);
      }
      sorted[tok * a.topk + rank] = mm;
      if (mm != 0x7fffffff) atomicOr(&umask[mm >> 5], 1 << (mm & 31));
    }
    if (tid < WAVES * NSUB) {
      const int t0 = t_wg0 + tid * TOK_SUB;
      if (t0 < N) atomicOr(&umask[(t0 / KT) >> 5], 1 << ((t0 / KT) & 31));
    }
    __syncthreads();
    // Gate bias (base 2) of every (row, selected block), read from LDS in the loop.
    for (int i = tid; i < ROWS_WG * a.topk; i += NT) {
      const int r = i / a.topk, e = i % a.topk;
      const int sg = r >> 4, rl = r & 15;
      const int t = t_wg0 + sg * TOK_SUB + rl / G;
      const int tok = t - t_wg0;
      const int mm2 = sorted[tok * a.topk + e];
      float bv = kNegInf;
      if (t < N && mm2 != 0x7fffffff) {
        const size_t gr = (size_t(b) * a.Hq + g * G + rl % G) * N + t;
        bv = (a.scores[gr * C + mm2] - a.lse_s[gr]) * kLog2e;
      }
      beta[i] = bv;
    }
  }
  __shared__ int wg_last;
  if (tid == 0) wg_last = -1;
  __syncthreads();
  {
    int lt = -1;
    for (int s = 0; s < NSUB; ++s) lt = max(lt, sub_live[s] ? c_sub[s] : -1);
    if (lane == 0) atomicMax(&wg_last, lt);
  }
  __syncthreads();
  const int last_tile = wg_last;

  // Row state: Q and dO fragments (B operands), lse (base 2), Delta, lse_s.
  uint4 qf[NSUB][KS], of[NSUB][KS];
  float lse2[NSUB], del[NSUB], lses[NSUB], dbt[NSUB];
  f32x4 dqa[NSUB][MD];
  int cursor[NSUB];
  for (int s = 0; s < NSUB; ++s) {
    const bool ok = row_t[s] < N;
    const size_t gr = (size_t(b) * a.Hq + row_h[s]) * N + (ok ? row_t[s] : 0);
    for (int ks = 0; ks < KS; ++ks) {
      qf[s][ks] = ok ? *reinterpret_cast<const uint4*>(a.q + gr * D + ks * 32 + lq * 8) : make_uint4(0, 0, 0, 0);
      of[s][ks] = ok ? *reinterpret_cast<const uint4*>(a.dout + gr * D + ks * 32 + lq * 8) : make_uint4(0, 0, 0, 0);
    }
    lse2[s] = ok ? a.lse[gr] * kLog2e : 0.f;
    del[s] = ok ? a.delta[gr] : 0.f;
    lses[s] = ok ? a.lse_s[gr] : 0.f;
    dbt[s] = 0.f;
    cursor[s] = 0;
    for (int md = 0; md < MD; ++md) dqa[s][md] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto next_tile = [&](int mm) -> int {
    if (!SPARSE) return (mm + 1 <= last_tile) ? mm + 1 : -1;
    for (int w = (mm + 1) >> 5; w < MW; ++w) {
      uint32_t bits = uint32_t(umask[w]);
      if (w == ((mm + 1) >> 5)) bits &= ~0u << ((mm + 1) & 31);
      if (bits) {
        const int r = w * 32 + __builtin_ctz(bits);
        return r <= last_tile ? r : -1;
      }
    }
    return -1;
  };

  const bf16_t* kh = a.k + (size_t(b) * a.Hkv + g) * size_t(N) * D;
  const bf16_t* vh = a.v + (size_t(b) * a.Hkv + g) * size_t(N) * D;
  constexpr int LOADS = (KT * CH + NT - 1) / NT;
  uint4 kreg[LOADS], vreg[LOADS];
  auto load_tile = [&](int mm) {
    const int jb = mm * KT;
    for (int i = 0; i < LOADS; ++i) {
      const int chunk = tid + NT * i;
      const int key = chunk / CH, c8 = chunk % CH;
      const int j = jb + key;
      const bool ok = chunk < KT * CH && j < N;
      kreg[i] = ok ? *reinterpret_cast<const uint4*>(kh + size_t(j) * D + c8 * 8) : make_uint4(0, 0, 0, 0);
      vreg[i] = ok ? *reinterpret_cast<const uint4*>(vh + size_t(j) * D + c8 * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&]() {
    for (int i = 0; i < LOADS; ++i) {
      const int chunk = tid + NT * i;
      if (chunk >= KT * CH) continue;
      const int key = chunk / CH, c8 = chunk % CH;
      *reinterpret_cast<uint4*>(&Ks[key][c8 * 8]) = kreg[i];
      *reinterpret_cast<uint4*>(&Vs[key][c8 * 8]) = vreg[i];
      // K^T with keys permuted to the MFMA k order of dS^T.
      const int kap = key & 31;
      const int phys = (key & ~31) + 8 * ((kap >> 2) & 3) + 4 * (kap >> 4) + (kap & 3);
      const uint16_t* hv = reinterpret_cast<const uint16_t*>(&kreg[i]);
      for (int d = 0; d < 8; ++d) Kt[c8 * 8 + d][phys] = hv[d];
    }
  };

  int mm = next_tile(-1);
  if (mm >= 0) load_tile(mm);
  float s_cur[NSUB];
  for (int s = 0; s < NSUB; ++s) {
    s_cur[s] = 0.f;
    if (!SPARSE && mm >= 0 && mm < c_sub[s] && row_t[s] < N)
      s_cur[s] = a.scores[((size_t(b) * a.Hq + row_h[s]) * N + row_t[s]) * C + mm];
  }
  while (mm >= 0) {
    __syncthreads();  // previous tile's LDS reads are done
    store_tile();
    __syncthreads();
    const int m_next = next_tile(mm);
    float s_nxt[NSUB];
    for (int s = 0; s < NSUB; ++s) {
      s_nxt[s] = 0.f;
      if (!SPARSE && m_next >= 0 && m_next < c_sub[s] && row_t[s] < N)
        s_nxt[s] = a.scores[((size_t(b) * a.Hq + row_h[s]) * N + row_t[s]) * C + m_next];
    }
    if (m_next >= 0) load_tile(m_next);

    bool need[NSUB];
    float bias2[NSUB];
    bool gated[NSUB];
    for (int s = 0; s < NSUB; ++s) {
      const bool own = (mm == c_sub[s]);
      const bool hist = (mm < c_sub[s]);
      bool sel = false;
      float bsel = kNegInf;
      if (hist && row_t[s] < N) {
        if (SPARSE) {
          const int tok = row_t[s] - t_wg0;
          const int32_t* srt = sorted + tok * a.topk;
          int cu = cursor[s];
          sel = (cu < a.topk && srt[cu] == mm);
          if (sel) bsel = beta[((wave * NSUB + s) * 16 + lr) * a.topk + cu];
          while (cu < a.topk && srt[cu] == mm) ++cu;
          cursor[s] = cu;
        } else {
          sel = true;
        }
      }
      need[s] = sub_live[s] && (own || (hist && __ballot(sel) != 0ull));
      gated[s] = sel;
      float bb = kNegInf;
      if (own) bb = 0.f;
      else if (sel) bb = SPARSE ? bsel : (s_cur[s] - lses[s]) * kLog2e;
      bias2[s] = bb;
    }
    // S^T = K Q^T and dP^T = V dO^T.
    f32x4 sacc[NSUB][4], pacc[NSUB][4];
    for (int s = 0; s < NSUB; ++s)
      for (int mt = 0; mt < 4; ++mt) {
        sacc[s][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        pacc[s][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    for (int ks = 0; ks < KS; ++ks)
      for (int mt = 0; mt < 4; ++mt) {
        const uint4 kfr = *reinterpret_cast<const uint4*>(&Ks[16 * mt + lr][ks * 32 + lq * 8]);
        const uint4 vfr = *reinterpret_cast<const uint4*>(&Vs[16 * mt + lr][ks * 32 + lq * 8]);
        for (int s = 0; s < NSUB; ++s)
          if (need[s]) {
            sacc[s][mt] = mfma16(kfr, qf[s][ks], sacc[s][mt]);
            pacc[s][mt] = mfma16(vfr, of[s][ks], pacc[s][mt]);
          }
      }
    uint4 dsf[NSUB][2];
    for (int s = 0; s < NSUB; ++s) {
      if (!need[s]) continue;
      const bool own = (mm == c_sub[s]);
      float dz[4][4];
      float dsum = 0.f;
      for (int mt = 0; mt < 4; ++mt)
        for (int i = 0; i < 4; ++i) {
          const int j = mm * KT + 16 * mt + 4 * lq + i;
          float pv = 0.f;
          if (bias2[s] != kNegInf && !(own && j > row_t[s]) && row_t[s] < N)
            pv = exp2_hw(sacc[s][mt][i] * c1 + bias2[s] - lse2[s]);
          const float d = pv * (pacc[s][mt][i] - del[s]);
          dz[mt][i] = d;
          dsum += d;
        }
      if (!own && gated[s]) {
        // dbeta for (row, mm): sum over the block's 64 keys.
        dsum += shfl_xor(dsum, 16);
        dsum += shfl_xor(dsum, 32);
        dbt[s] += dsum;
        if (lq == 0) a.ds[((size_t(b) * a.Hq + row_h[s]) * N + row_t[s]) * C + mm] = dsum;
      }
      for (int kk = 0; kk < 2; ++kk) {
        dsf[s][kk].x = pack_bf16(dz[2 * kk][0], dz[2 * kk][1]);
        dsf[s][kk].y = pack_bf16(dz[2 * kk][2], dz[2 * kk][3]);
        dsf[s][kk].z = pack_bf16(dz[2 * kk + 1][0], dz[2 * kk + 1][1]);
        dsf[s][kk].w = pack_bf16(dz[2 * kk + 1][2], dz[2 * kk + 1][3]);
      }
    }
    // dQ^T += K^T dS^T.
    for (int md = 0; md < MD; ++md)
      for (int kk = 0; kk < 2; ++kk) {
        const uint4 ka = *reinterpret_cast<const uint4*>(&Kt[16 * md + lr][kk * 32 + lq * 8]);
        for (int s = 0; s < NSUB; ++s)
          if (need[s]) dqa[s][md] = mfma16(ka, dsf[s][kk], dqa[s][md]);
      }
    for (int s = 0; s < NSUB; ++s) s_cur[s] = s_nxt[s];
    mm = m_next;
  }

  // dQ (scaled): lane holds row, columns 16md + 4lq + i.
  for (int s = 0; s < NSUB; ++s) {
    if (row_t[s] >= N) continue;
    const size_t gr = (size_t(b) * a.Hq + row_h[s]) * N + row_t[s];
    for (int md = 0; md < MD; ++md) {
      uint2 w;
      w.x = pack_bf16(dqa[s][md][0] * a.scale, dqa[s][md][1] * a.scale);
      w.y = pack_bf16(dqa[s][md][2] * a.scale, dqa[s][md][3] * a.scale);
      *reinterpret_cast<uint2*>(a.dq + gr * D + 16 * md + 4 * lq) = w;
    }
  }
  // ds epilogue: ds = dbeta - g * sum(dbeta) over the history, dense; 0 beyond.
  __shared__ float tot_sh[ROWS_WG];
  for (int s = 0; s < NSUB; ++s)
    if (lq == 0) tot_sh[wave * 16 * NSUB + s * 16 + lr] = dbt[s];
  __threadfence();
  __syncthreads();
  for (int rr = 0; rr < 16 * NSUB; ++rr) {
    const int s = rr >> 4, r = rr & 15;
    const int sg = wave * NSUB + s;
    const int t = t_wg0 + sg * TOK_SUB + r / G;
    if (t >= N) continue;
    const int h = g * G + r % G;
    const int c = t / KT;
    const size_t gr = (size_t(b) * a.Hq + h) * N + t;
    const float tot = tot_sh[wave * 16 * NSUB + rr];
    const float ls = a.lse_s[gr];
    const float* srow = a.scores + gr * C;
    float* drow = a.ds + gr * C;
    // selection of this token (sparse): bitmask built by the prep kernel
    const uint32_t* bits = SPARSE ? a.selbits + ((size_t(b) * a.Hkv + g) * N + t) * a.MWB : nullptr;
    for (int m2 = lane; m2 < C; m2 += 64) {
      float out = 0.f;
      if (m2 < c) {
        const float gate = exp2_hw((srow[m2] - ls) * kLog2e);
        const bool sel = SPARSE ? ((bits[m2 >> 5] >> (m2 & 31)) & 1u) : true;
        out = (sel ? drow[m2] : 0.f) - gate * tot;
      }
      drow[m2] = out;
    }
  }
}

}  // namespace

bool bwd_mfma_supported(const Dims& d, int topk, bool sparse) {
  if (d.block != KT || (d.D != 64 && d.D != 128)) return false;
  const int G = d.G();
  if (G != 1 && G != 2 && G != 4 && G != 8) return false;
  if (sparse) {
    // LDS of the dQ kernel's sparse prologue (128 rows x topk bias table).
    if (size_t(128) * topk > 8192) return false;
    if (((d.C + 32) >> 5) > 1024) return false;
  }
  return true;
}

size_t bwd_mfma_workspace(const Dims& d, int topk, bool sparse) {
  size_t bytes = align_up(size_t(d.B) * d.Hq * d.N * sizeof(float));
  if (sparse) {
    const int MWB = (d.C + 31) / 32;
    bytes += align_up(size_t(d.B) * d.Hkv * d.N * (MWB > 0 ? MWB : 1) * sizeof(uint32_t));
  }
  (void)topk;
  return bytes;
}

template <int D, int G, bool SPARSE>
static hipError_t bwd_mfma_t(BwdArgs a, int B, hipStream_t s) {
  constexpr int NSUB = 1;  // rows per wave in the dQ kernel: 16 (register budget)
  constexpr int WAVES = SPARSE ? 8 : 4;
  constexpr int TOK_WG = 16 * NSUB * WAVES / G;
  const size_t rows = size_t(B) * a.Hq * a.N;
  SAS_LAUNCH("bwd_delta_mfma", (bwd_delta_mfma_kernel<D>), dim3((rows + 256 / (D / 8) - 1) / (256 / (D / 8))),
                     dim3(256), 0, s, a.o, a.dout, a.delta, rows);
  if (SPARSE) {
    const size_t tokens = size_t(B) * a.Hkv * a.N;
    SAS_LAUNCH("selbits", selbits_kernel, dim3((tokens + 3) / 4), dim3(256), 0, s, a.idx, a.selbits, a.N,
                       a.topk, a.MWB, tokens);
  }
  a.n_pairs = B * a.Hkv;
  a.n_tiles = (a.N + KT - 1) / KT;
  SAS_LAUNCH("bwd_dkdv", (bwd_dkdv_kernel<D, G, SPARSE>), dim3(a.n_tiles * a.n_pairs), dim3(256), 0, s, a);
  a.n_tiles = (a.N + TOK_WG - 1) / TOK_WG;
  const size_t dyn = SPARSE ? (size_t((a.C + 32) >> 5) + (2 + G) * size_t(TOK_WG) * a.topk) * 4 : 0;
  SAS_LAUNCH("bwd_dq", (bwd_dq_kernel<D, G, NSUB, WAVES, SPARSE>), dim3(a.n_tiles * a.n_pairs), dim3(64 * WAVES), dyn, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_mfma(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* scores, const int32_t* idx,
                           const float* lse, const float* lse_s, void* dq, void* dk, void* dv,
                           float* ds, const Dims& d, int topk, float scale, void* ws,
                           hipStream_t s) {
  const bool sp = idx != nullptr;
  char* w = static_cast<char*>(ws);
  float* delta = reinterpret_cast<float*>(w);
  uint32_t* selbits = reinterpret_cast<uint32_t*>(w + align_up(size_t(d.B) * d.Hq * d.N * sizeof(float)));
  BwdArgs a{(const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, (const bf16_t*)o, (const bf16_t*)dout,
            scores, idx, lse, lse_s, (bf16_t*)dq, (bf16_t*)dk, (bf16_t*)dv, ds, delta,
            sp ? selbits : nullptr, d.Hq, d.Hkv, d.N, d.C, sp ? topk : 0, (d.C + 31) / 32, 0, 0, scale};
  if (a.MWB < 1) a.MWB = 1;
  const int G = d.G();
#define SAS_BWD_CASE(DD, GG)                                                              \
  if (d.D == DD && G == GG)                                                               \
    return sp ? bwd_mfma_t<DD, GG, true>(a, d.B, s) : bwd_mfma_t<DD, GG, false>(a, d.B, s);
  SAS_BWD_CASE(128, 4)
  SAS_BWD_CASE(128, 1)
  SAS_BWD_CASE(128, 2)
  SAS_BWD_CASE(128, 8)
  SAS_BWD_CASE(64, 4)
  SAS_BWD_CASE(64, 1)
  SAS_BWD_CASE(64, 2)
  SAS_BWD_CASE(64, 8)
#undef SAS_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace sas
