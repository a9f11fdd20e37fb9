// SAS gated attention forward on the matrix cores (bf16 in, fp32 accumulate).
//
// o = softmax(scale * q K^T + bias) V with bias = 0 on the query's own block
// (causal), log g = s - LSE_s on gated history blocks and -inf elsewhere
// (blog 方法核心; jaehun.me review "New Approach", paper Eq. 9; the gate's log
// form s - LSE(s): review "Why the Four Design Choices Matter").  Tiled with an
// online softmax as in the review's kernel paragraph ("A Concrete Walkthrough").
//
// Layout.  A workgroup owns TOK_WG consecutive query tokens of one KV head and
// all G query heads of that head, i.e. 64*NSUB rows, split into 4 waves x NSUB
// subtiles of 16 rows (16/G tokens x G heads).  Everything is transposed so that
// a lane owns one query row: S^T = K Q^T and O^T = V^T P^T on
// v_mfma_f32_16x16x32_bf16, so the softmax statistics and the output rescale
// stay lane-local (the four lanes of a row only meet for the row max).  Key
// tiles are one block (64 keys): K row-major and V transposed (keys permuted to
// match the MFMA B layout of P) in double-buffered LDS.  The gate bias is
// constant over a block, so it enters once per (row, tile).
//
// Sparse scope: each token's selected blocks are sorted in LDS; the workgroup
// visits the union of its rows' blocks in ascending order and a subtile skips a
// tile no row of it selected.  Full scope visits every block up to the own one.
#include "common.h"
#include "internal.h"
#include "mfma.h"

namespace sas {
namespace {

constexpr int KT = 64;  // keys per tile = block size of this kernel
constexpr int KPAD = 8;

struct FwdArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  const float* scores;
  const int32_t* idx;
  bf16_t* o;
  float* lse;
  float* lse_s;
  int Hq, Hkv, N, C, topk, n_tiles, n_pairs;
  float scale;
};

template <int D, int G, int NSUB, int WAVES, bool SPARSE>
__global__ __launch_bounds__(64 * WAVES, 2) void fwd_mfma_kernel(FwdArgs a) {
  constexpr int NT = 64 * WAVES;  // threads
  constexpr int KS = D / 32;    // k-steps of S = K Q^T
  constexpr int MD = D / 16;    // output tiles of O^T
  constexpr int TOK_SUB = 16 / G;
  constexpr int ROWS_WG = 16 * NSUB * WAVES;
  constexpr int TOK_WG = ROWS_WG / G;
  constexpr int CH = D / 8;     // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KT][D + KPAD];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D][KT + KPAD];
  __shared__ float lses_sh[ROWS_WG];
  extern __shared__ int32_t dyn[];  // sparse: union mask | sorted idx | raw idx

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  int tile, pair;
  xcd_order(blockIdx.x, a.n_tiles, a.n_pairs, &tile, &pair);
  const int b = pair / a.Hkv, g = pair % a.Hkv;
  const int N = a.N, C = a.C;
  const int t_wg0 = tile * TOK_WG;

  // Rows of this lane, one per subtile.
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

  // ---- LSE of each row's history scores (gate normaliser) -------------------
  for (int rr = 0; rr < 16 * NSUB; ++rr) {
    const int s = rr >> 4, r = rr & 15;
    const int sg = wave * NSUB + s;
    const int t = t_wg0 + sg * TOK_SUB + r / G;
    const int h = g * G + r % G;
    float res = kNegInf;
    if (t < N) {
      const int c = t / KT;
      const float* srow = a.scores + ((size_t(b) * a.Hq + h) * N + t) * C;
      float mx = kNegInf;
      for (int m = lane; m < c; m += 64) mx = fmaxf(mx, srow[m]);
      for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, shfl_xor(mx, off));
      float sm = 0.f;
      if (c > 0) {
        for (int m = lane; m < c; m += 64) sm += exp2_hw((srow[m] - mx) * kLog2e);
        for (int off = 32; off >= 1; off >>= 1) sm += shfl_xor(sm, off);
        res = mx + log_hw(sm);
      }
      if (lane == 0) a.lse_s[(size_t(b) * a.Hq + h) * N + t] = res;
    }
    if (lane == 0) lses_sh[wave * 16 * NSUB + rr] = res;
  }

  // ---- sparse scope: per-token sorted selections and the union of blocks ----
  const int MW = (C + 32) >> 5;  // bits 0..C (the own block may be block C)
  int32_t* umask = dyn;
  int32_t* sorted = dyn + MW;                 // [TOK_WG][topk]
  int32_t* raw = sorted + TOK_WG * a.topk;
  float* beta = reinterpret_cast<float*>(raw + TOK_WG * a.topk);  // [ROWS_WG][topk] (sparse)    // [TOK_WG][topk]
  if (SPARSE) {
    for (int i = tid; i < MW; i += NT) umask[i] = 0;
    for (int i = tid; i < TOK_WG * a.topk; i += NT) {
      const int tok = i / a.topk, e = i % a.topk;
      const int t = t_wg0 + tok;
      int m = -1;
      if (t < N) {
        m = a.idx[((size_t(b) * a.Hkv + g) * N + t) * a.topk + e];
        if (m < 0 || m >= t / KT) m = -1;
      }
      raw[i] = m < 0 ? 0x7fffffff : m;
    }
    __syncthreads();
    for (int i = tid; i < TOK_WG * a.topk; i += NT) {
      const int tok = i / a.topk, e = i % a.topk;
      const int32_t* rr = raw + tok * a.topk;
      const int m = rr[e];
      int rank = 0;
      for (int e2 = 0; e2 < a.topk; ++e2) {
        const int m2 = rr[e2];
        rank += (m2 < m) || (m2 == m && e2 < e);
      }
      sorted[tok * a.topk + rank] = m;
      if (m != 0x7fffffff) atomicOr(&umask[m >> 5], 1 << (m & 31));
    }
    if (tid < WAVES * NSUB) {
      const int t0 = t_wg0 + tid * TOK_SUB;
      if (t0 < N) atomicOr(&umask[(t0 / KT) >> 5], 1 << ((t0 / KT) & 31));
    }
  }
  __syncthreads();
  if (SPARSE) {
    // Gate bias (base 2) of every (row, selected block): the main loop reads it
    // from LDS instead of gathering the score per tile.
    for (int i = tid; i < ROWS_WG * a.topk; i += NT) {
      const int r = i / a.topk, e = i % a.topk;
      const int sg = r >> 4, rl = r & 15;
      const int t = t_wg0 + sg * TOK_SUB + rl / G;
      const int tok = t - t_wg0;
      const int mm = sorted[tok * a.topk + e];
      float bv = kNegInf;
      if (t < N && mm != 0x7fffffff)
        bv = (a.scores[((size_t(b) * a.Hq + g * G + rl % G) * N + t) * C + mm] - lses_sh[r]) * kLog2e;
      beta[i] = bv;
    }
    __syncthreads();
  }

  // ---- Q fragments (B operand of S^T = K Q^T), one row per lane ----------------
  uint4 qf[NSUB][KS];
  float lses[NSUB];
  for (int s = 0; s < NSUB; ++s) {
    const bool ok = row_t[s] < N;
    const bf16_t* qr = a.q + ((size_t(b) * a.Hq + row_h[s]) * N + (ok ? row_t[s] : 0)) * D;
    for (int ks = 0; ks < KS; ++ks)
      qf[s][ks] = ok ? *reinterpret_cast<const uint4*>(qr + ks * 32 + lq * 8) : make_uint4(0, 0, 0, 0);
    lses[s] = lses_sh[wave * 16 * NSUB + s * 16 + lr];
  }
  int cursor[NSUB];
  for (int s = 0; s < NSUB; ++s) cursor[s] = 0;

  // Tiles of the workgroup: full scope 0 .. max own block; sparse: set bits.
  int last_tile = -1;
  for (int s = 0; s < NSUB; ++s) last_tile = max(last_tile, sub_live[s] ? c_sub[s] : -1);
  // every wave needs the workgroup maximum, through LDS
  __shared__ int wg_last;
  if (tid == 0) wg_last = -1;
  __syncthreads();
  if (lane == 0) atomicMax(&wg_last, last_tile);
  __syncthreads();
  last_tile = wg_last;

  auto next_tile = [&](int m) -> int {
    if (!SPARSE) return (m + 1 <= last_tile) ? m + 1 : -1;
    for (int w = (m + 1) >> 5; w < MW; ++w) {
      uint32_t bits = uint32_t(umask[w]);
      if (w == ((m + 1) >> 5)) bits &= ~0u << ((m + 1) & 31);
      if (bits) {
        const int r = w * 32 + __builtin_ctz(bits);
        return r <= last_tile ? r : -1;
      }
    }
    return -1;
  };

  const bf16_t* kh = a.k + (size_t(b) * a.Hkv + g) * size_t(N) * D;
  const bf16_t* vh = a.v + (size_t(b) * a.Hkv + g) * size_t(N) * D;
  constexpr int KLOADS = (KT * CH + NT - 1) / NT;
  constexpr int VGROUPS = 16 * CH;  // 4-key groups x 16-byte column chunks
  uint4 kreg[KLOADS];
  uint4 vreg[4];

  auto load_tile = [&](int m) {
    const int j0 = m * KT;
    for (int i = 0; i < KLOADS; ++i) {
      const int chunk = tid + NT * i;
      const int key = chunk / CH, c8 = chunk % CH;
      const int j = j0 + key;
      kreg[i] = (chunk < KT * CH && j < N) ? *reinterpret_cast<const uint4*>(kh + size_t(j) * D + c8 * 8)
                                             : make_uint4(0, 0, 0, 0);
    }
    if (tid < VGROUPS) {
      const int kg = tid / CH, c8 = tid % CH;
      for (int r = 0; r < 4; ++r) {
        const int j = j0 + 4 * kg + r;
        vreg[r] = j < N ? *reinterpret_cast<const uint4*>(vh + size_t(j) * D + c8 * 8) : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&](int buf) {
    for (int i = 0; i < KLOADS; ++i) {
      const int chunk = tid + NT * i;
      if (chunk < KT * CH) {
        const int key = chunk / CH, c8 = chunk % CH;
        *reinterpret_cast<uint4*>(&Ks[buf][key][c8 * 8]) = kreg[i];
      }
    }
    if (tid < VGROUPS) {
      const int kg = tid / CH, c8 = tid % CH;
      const int kap = (4 * kg) & 31;  // key within its 32-key group: 16*hi + 4*q
      const int phys = ((4 * kg) & ~31) + 8 * ((kap >> 2) & 3) + 4 * (kap >> 4);
      const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vreg[0]);
      const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vreg[1]);
      const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vreg[2]);
      const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vreg[3]);
      for (int d2 = 0; d2 < 4; ++d2) {
        // columns 2*d2 and 2*d2+1 of the chunk, four keys each
        const uint32_t lo0 = (w0[d2] & 0xffffu) | (w1[d2] << 16);
        const uint32_t lo1 = (w2[d2] & 0xffffu) | (w3[d2] << 16);
        const uint32_t hi0 = (w0[d2] >> 16) | (w1[d2] & 0xffff0000u);
        const uint32_t hi1 = (w2[d2] >> 16) | (w3[d2] & 0xffff0000u);
        *reinterpret_cast<uint2*>(&Vt[buf][c8 * 8 + 2 * d2][phys]) = make_uint2(lo0, lo1);
        *reinterpret_cast<uint2*>(&Vt[buf][c8 * 8 + 2 * d2 + 1][phys]) = make_uint2(hi0, hi1);
      }
    }
  };

  f32x4 oacc[NSUB][MD];
  float mrow[NSUB], lpart[NSUB];
  for (int s = 0; s < NSUB; ++s) {
    for (int md = 0; md < MD; ++md) oacc[s][md] = f32x4{0.f, 0.f, 0.f, 0.f};
    mrow[s] = kNegInf;
    lpart[s] = 0.f;
  }
  const float c1 = a.scale * kLog2e;

  int m = next_tile(-1);
  int buf = 0;
  if (m >= 0) {
    load_tile(m);
    store_tile(0);
  }
  __syncthreads();
  float s_cur[NSUB];
  for (int s = 0; s < NSUB; ++s) {
    s_cur[s] = 0.f;
    if (!SPARSE && m >= 0 && m < c_sub[s] && row_t[s] < N)
      s_cur[s] = a.scores[((size_t(b) * a.Hq + row_h[s]) * N + row_t[s]) * C + m];
  }
  while (m >= 0) {
    const int m_next = next_tile(m);
    float s_nxt[NSUB];
    for (int s = 0; s < NSUB; ++s) {
      s_nxt[s] = 0.f;
      if (!SPARSE && m_next >= 0 && m_next < c_sub[s] && row_t[s] < N)
        s_nxt[s] = a.scores[((size_t(b) * a.Hq + row_h[s]) * N + row_t[s]) * C + m_next];
    }
    if (m_next >= 0) load_tile(m_next);

    // Which subtiles take part, and each lane's bias for its row.
    bool need[NSUB];
    float bias2[NSUB];
    for (int s = 0; s < NSUB; ++s) {
      const bool own = (m == c_sub[s]);
      const bool hist = (m < c_sub[s]);
      bool sel = false;
      float bsel = kNegInf;
      if (hist && row_t[s] < N) {
        if (SPARSE) {
          const int tok = row_t[s] - t_wg0;
          const int32_t* srt = sorted + tok * a.topk;
          int cu = cursor[s];
          sel = (cu < a.topk && srt[cu] == m);
          if (sel) bsel = beta[((wave * NSUB + s) * 16 + lr) * a.topk + cu];
          while (cu < a.topk && srt[cu] == m) ++cu;
          cursor[s] = cu;
        } else {
          sel = true;
        }
      }
      const bool any = sub_live[s] && (own || (hist && __ballot(sel) != 0ull));
      need[s] = any;
      float bb = kNegInf;
      if (own) bb = 0.f;
      else if (sel) bb = SPARSE ? bsel : (s_cur[s] - lses[s]) * kLog2e;
      bias2[s] = bb;
    }

    // S^T = K Q^T for every needed subtile.
    f32x4 sacc[NSUB][4];
    for (int s = 0; s < NSUB; ++s)
      for (int mt = 0; mt < 4; ++mt) sacc[s][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int ks = 0; ks < KS; ++ks) {
      for (int mt = 0; mt < 4; ++mt) {
        const uint4 kf = *reinterpret_cast<const uint4*>(&Ks[buf][16 * mt + lr][ks * 32 + lq * 8]);
        for (int s = 0; s < NSUB; ++s)
          if (need[s]) sacc[s][mt] = mfma16(kf, qf[s][ks], sacc[s][mt]);
      }
    }
    // Online softmax (base 2) and P^T fragments.
    uint4 pf[NSUB][2];
    for (int s = 0; s < NSUB; ++s) {
      if (!need[s]) continue;
      const bool own = (m == c_sub[s]);
      float z[4][4];
      float mx = kNegInf;
      for (int mt = 0; mt < 4; ++mt)
        for (int i = 0; i < 4; ++i) {
          float v = sacc[s][mt][i] * c1 + bias2[s];
          if (own && (m * KT + 16 * mt + 4 * lq + i > row_t[s])) v = kNegInf;
          z[mt][i] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float mnew = fmaxf(mrow[s], mx);
      const float muse = (mnew == kNegInf) ? 0.f : mnew;
      const float alpha = exp2_hw(mrow[s] - muse);
      mrow[s] = mnew;
      float ps = 0.f;
      for (int mt = 0; mt < 4; ++mt)
        for (int i = 0; i < 4; ++i) {
          z[mt][i] = exp2_hw(z[mt][i] - muse);
          ps += z[mt][i];
        }
      lpart[s] = lpart[s] * alpha + ps;
      for (int md = 0; md < MD; ++md) oacc[s][md] *= alpha;
      for (int kk = 0; kk < 2; ++kk) {
        pf[s][kk].x = pack_bf16(z[2 * kk][0], z[2 * kk][1]);
        pf[s][kk].y = pack_bf16(z[2 * kk][2], z[2 * kk][3]);
        pf[s][kk].z = pack_bf16(z[2 * kk + 1][0], z[2 * kk + 1][1]);
        pf[s][kk].w = pack_bf16(z[2 * kk + 1][2], z[2 * kk + 1][3]);
      }
    }
    // O^T += V^T P^T.
    for (int md = 0; md < MD; ++md) {
      for (int kk = 0; kk < 2; ++kk) {
        const uint4 vf = *reinterpret_cast<const uint4*>(&Vt[buf][16 * md + lr][kk * 32 + lq * 8]);
        for (int s = 0; s < NSUB; ++s)
          if (need[s]) oacc[s][md] = mfma16(vf, pf[s][kk], oacc[s][md]);
      }
    }
    if (m_next >= 0) store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    for (int s = 0; s < NSUB; ++s) s_cur[s] = s_nxt[s];
    m = m_next;
  }

  // ---- epilogue ---------------------------------------------------------------
  for (int s = 0; s < NSUB; ++s) {
    float l = lpart[s];
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    if (row_t[s] >= N) continue;
    const size_t row = (size_t(b) * a.Hq + row_h[s]) * N + row_t[s];
    const float inv = 1.f / l;
    for (int md = 0; md < MD; ++md) {
      uint2 w;
      w.x = pack_bf16(oacc[s][md][0] * inv, oacc[s][md][1] * inv);
      w.y = pack_bf16(oacc[s][md][2] * inv, oacc[s][md][3] * inv);
      *reinterpret_cast<uint2*>(a.o + row * D + 16 * md + 4 * lq) = w;
    }
    if (lq == 0) a.lse[row] = (mrow[s] + __builtin_amdgcn_logf(l)) * kLn2;
  }
}

template <int D, int G, bool SPARSE>
hipError_t fwd_mfma_t(const FwdArgs& a0, int B, hipStream_t stream) {
  // Sparse scope: wider workgroups (more tokens share each K/V tile load).
  constexpr int NSUB = 2;
  constexpr int WAVES = SPARSE ? 8 : 4;
  constexpr int TOK_WG = 16 * NSUB * WAVES / G;
  FwdArgs a = a0;
  a.n_tiles = (a.N + TOK_WG - 1) / TOK_WG;
  a.n_pairs = B * a.Hkv;
  const size_t dyn = SPARSE ? (size_t((a.C + 32) >> 5) + (2 + G) * size_t(TOK_WG) * a.topk) * 4 : 0;
  hipLaunchKernelGGL((fwd_mfma_kernel<D, G, NSUB, WAVES, SPARSE>), dim3(a.n_tiles * a.n_pairs), dim3(64 * WAVES),
                     dyn, stream, a);
  return hipGetLastError();
}

}  // namespace

// Shapes the matrix-core forward covers: bf16, block 64, D 64/128, G in
// {1,2,4,8}; sparse scope needs the per-workgroup index lists to fit in LDS.
bool fwd_mfma_supported(const Dims& d, int topk, bool sparse) {
  if (d.block != KT || (d.D != 64 && d.D != 128)) return false;
  const int G = d.G();
  if (G != 1 && G != 2 && G != 4 && G != 8) return false;
  if (sparse) {
    // LDS of the sparse prologue: sorted/raw lists (tokens x topk) and the gate
    // bias table (256 rows x topk).
    if (size_t(256) * topk > 8192) return false;
    if (((d.C + 32) >> 5) > 1024) return false;
  }
  return true;
}

hipError_t launch_fwd_mfma(const void* q, const void* k, const void* v, const float* scores,
                           const int32_t* idx, void* o, float* lse, float* lse_s, const Dims& d,
                           int topk, float scale, hipStream_t s) {
  FwdArgs a{(const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, scores, idx, (bf16_t*)o, lse, lse_s,
            d.Hq, d.Hkv, d.N, d.C, idx ? topk : 0, 0, 0, scale};
  const int G = d.G();
  const bool sp = idx != nullptr;
#define SAS_FWD_CASE(DD, GG)                                             \
  if (d.D == DD && G == GG) {                                            \
    return sp ? fwd_mfma_t<DD, GG, true>(a, d.B, s) : fwd_mfma_t<DD, GG, false>(a, d.B, s); \
  }
  SAS_FWD_CASE(128, 4)
  SAS_FWD_CASE(128, 1)
  SAS_FWD_CASE(128, 2)
  SAS_FWD_CASE(128, 8)
  SAS_FWD_CASE(64, 4)
  SAS_FWD_CASE(64, 1)
  SAS_FWD_CASE(64, 2)
  SAS_FWD_CASE(64, 8)
#undef SAS_FWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace sas
