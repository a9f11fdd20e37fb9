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
// Kernels:
//   delta      Delta per row.
//   dkdv       KV-major: a workgroup owns one block (64 keys, 16 per wave) of
//              one KV head and streams the query rows that attend it, 64 rows
//              per step: the own block's rows (causal) and every later row
//              (full scope) or the block's list of selecting tokens (sparse
//              scope, sel_lists.hip).  Lane = key layout (S = Q K^T), so dV =
//              P^T dO and dK = dS^T Q contract over rows with P and dS straight
//              from registers.
//              Sparse scope: the step's dS rows also pass through LDS, where
//              each wave takes a quarter of the columns of the rows' dQ
//              shares dS K over this block (dQ^T = K^T dS^T, K^T fragments
//              held in registers) and writes them to the rows' slots; the
//              per-row dbeta is recorded per list entry.
//   rows       sparse scope, per row: dq = sum of its dQ shares, and
//              ds = dbeta - g sum(dbeta).
//   dq         full scope, query-major like the forward (lane = row, S^T =
//              K Q^T), recomputing P and dP^T = V dO^T per tile; dQ^T += K^T
//              dS^T; dbeta is a lane-local row sum written per (row, block),
//              then the dense ds epilogue.
#include "common.h"
#include "internal.h"
#include "mfma.h"
#include "tiles.h"

#include <algorithm>
#include <type_traits>

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
  uint16_t* selpre;  // workspace [B, Hkv, N, MWB + 1]: set bits before each word (sparse)
  bf16_t* dqp;       // workspace [B, Hq, N, topk + 1, D]: dQ share per slot (sparse)
  float* dbl;        // workspace [pairs, list entries, G]: dbeta per list entry and head (sparse)
  bf16_t* dummy;     // workspace, one row of D: target of the stores of rows a step does not hold (sparse)
  const float* lg2;  // optional [pairs, list entries, G]: base-2 log gate per list entry and head,
                     // saved by the forward (sparse; else the scores and LSE_s give it)
  int Hq, Hkv, N, C, topk, MWB, n_tiles, n_pairs, NB;
  float scale;
  int gate;          // gate activation (kGateSoftmax, kGateSigmoid, kGateRaw)
  int ds_hist_only;  // sparse: ds columns m >= c(t) (no history block) are not written
};

constexpr int kTokMask = 0x7fffff;  // token field of a selection-list entry
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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

// --------------------------------------------------------------- dK / dV ----
// KV-major: a workgroup owns one 64-key block m of one KV head, 16 keys per
// wave (lane = key; K and V are B operands held in registers), and streams the
// query rows that attend the block, RS = 64 rows (RS/G tokens x G heads) per
// step, through a two-stage LDS ring filled by direct global -> LDS loads: Q
// and dO rows (row-major, 16-byte chunks XOR-swizzled by row) and, per row,
// lse, Delta, the block's selector score and LSE_s.  The own block's tokens
// come first (causal mask, bias 0), then every later token (full scope) or the
// block's list of the later tokens whose selection holds m (sparse scope).
//   S = Q K^T, dP = dO V^T      A: Q / dO row fragments
//   dV += P^T dO, dK += dS^T Q  A: P^T / dS^T from registers (the permuted row
//                               order of the S accumulators); B: dO / Q read
//                               transposed from the row-major tile
//   sparse: dQ^T = K^T dS^T     A: K^T fragments in registers; B: the step's
//                               dS rows staged in LDS
// OUTER: the outer gate: history rows take no bias, g = exp(s - LSE_s)
// scales P in dV and dP in dZ, and the recorded dbeta is sum P g dP (= g dg).
template <int D, int G, bool SPARSE, bool OUTER>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(BwdArgs a, SelLists L) {
  using namespace tiles;
  constexpr int WAVES = 4;
  constexpr int NT = 64 * WAVES;
  constexpr int KS = D / 32;
  constexpr int ND = D / 16;
  constexpr int CH = D / 8;         // 16-byte chunks per row
  constexpr int RS = 64;            // rows per step
  constexpr int TPS = RS / G;       // tokens per step
  constexpr int NPIECE = RS * D * 2 / 1024;  // 1 KB loads per operand per step
  constexpr int PPW = NPIECE / WAVES;
  // Stage layout (16-bit units): Q [RS][D] | dO [RS][D] | fp32 [4][RS]
  // (lse, Delta, score of block m, LSE_s): one load target per stage.
  constexpr int ST_DO = RS * D, ST_F = 2 * RS * D;
  constexpr int STAGE = 2 * RS * D + 4 * RS * 2;
  static_assert(NPIECE % WAVES == 0 && WAVES == 4, "stat loads: one per wave");
  static_assert(RS * (D + 8) <= ST_F, "staged dQ rows fit over the Q and dO tiles");
  static_assert(RS == 64, "a lane holds the token of its own row");
  __shared__ __attribute__((aligned(16))) uint16_t R0[STAGE], R1[STAGE];
  __shared__ __attribute__((aligned(16))) int tok_sh[2][RS];  // token of each row, -1: none
  // sparse scope: the step's dS rows [row][key] (bf16, padded; the dQ
  // product's B operand) and the four waves' per-row sums of dS over their
  // keys (the dbeta records)
  constexpr int TST = KT + 8;
  __shared__ __attribute__((aligned(16))) uint16_t dst_sh[SPARSE ? RS * TST : 8];
  __shared__ __attribute__((aligned(16))) float dbs_sh[SPARSE ? WAVES * RS : 4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tile, pair;
  xcd_order(blockIdx.x, a.n_tiles, a.n_pairs, &tile, &pair);
  const int m = a.n_tiles - 1 - tile;  // lowest blocks (most rows) first
  const int b = pair / a.Hkv, g = pair % a.Hkv;
  const int N = a.N, C = a.C;
  const int j0 = m * KT;
  const float c1 = a.scale * kLog2e;
  const size_t hrow0 = (size_t(b) * a.Hq + g * G) * N;  // row index of head g*G, token 0

  // Stationary K and V fragments (B operands): lane holds key my_key, columns
  // 32 ks + 8 (lane / 16).
  uint4 kf[KS], vf[KS];
  {
    const int my_key = j0 + wave * 16 + (lane & 15);
    const size_t kr = (size_t(b) * a.Hkv + g) * N + (my_key < N ? my_key : 0);
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = my_key < N ? *reinterpret_cast<const uint4*>(a.k + kr * D + ks * 32 + (lane >> 4) * 8)
                          : make_uint4(0, 0, 0, 0);
      vf[ks] = my_key < N ? *reinterpret_cast<const uint4*>(a.v + kr * D + ks * 32 + (lane >> 4) * 8)
                          : make_uint4(0, 0, 0, 0);
    }
  }
  // Sparse scope, dQ^T = K^T dS^T: A operand of the wave's NDW 16-column d
  // tiles, lane holds column 16 (NDW wave + nd) + lane % 16 of keys
  // 32 kk + 8 (lane / 16) .. + 7 (zero beyond N).
  constexpr int NDW = SPARSE ? D / 64 : 1;
  uint4 kq[NDW][2];
  if constexpr (SPARSE) {
    const uint16_t* kh = reinterpret_cast<const uint16_t*>(a.k) + (size_t(b) * a.Hkv + g) * size_t(N) * D;
    // all loads first (keys clamped to N - 1), then the selects, so that the
    // 16 NDW loads go out together
    uint32_t h[NDW][2][8];
#pragma unroll
    for (int nd = 0; nd < NDW; ++nd)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          h[nd][kk][j] = kh[size_t(min(j0 + 32 * kk + 8 * (lane >> 4) + j, N - 1)) * D +
                            16 * (NDW * wave + nd) + (lane & 15)];
#pragma unroll
    for (int nd = 0; nd < NDW; ++nd)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        uint32_t* x = h[nd][kk];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = j0 + 32 * kk + 8 * (lane >> 4) + j < N ? x[j] : 0u;
        kq[nd][kk] = make_uint4(x[0] | (x[1] << 16), x[2] | (x[3] << 16), x[4] | (x[5] << 16), x[6] | (x[7] << 16));
      }
  }
  f32x4 dk[ND], dv[ND];
  for (int nd = 0; nd < ND; ++nd) {
    dk[nd] = f32x4{0.f, 0.f, 0.f, 0.f};
    dv[nd] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- token stream: step k < n_own covers own tokens k TPS .. (causal),
  // later steps the history: consecutive tokens (full scope) or the block's
  // list entries (sparse scope).
  const int own_n = min(KT, N - j0);
  const int n_own = (own_n + TPS - 1) / TPS;
  const uint32_t* lst = nullptr;
  int n_hist;
  if constexpr (SPARSE) {
    const uint32_t* bo = L.blkoff + size_t(pair) * (L.NB + 1) + m;
    lst = L.ents + size_t(pair) * L.ents_per_pair + bo[0];
    n_hist = int(bo[1] - bo[0]);
  } else {
    n_hist = max(0, N - (j0 + KT));
  }
  const int n_hsteps = (n_hist + TPS - 1) / TPS;
  const int n_steps = n_own + n_hsteps;
  // History steps walk the token stream from its end: step k >= n_own covers
  // stream positions hstep(k) TPS .. (descending token order).  Every
  // workgroup of a KV head then starts at the last tokens and, since a token
  // selects each of its history blocks with the same probability, the
  // resident workgroups move down the tokens together and gather the same Q
  // and dO rows at about the same time (L2 hits instead of refetches).
  auto hstep = [&](int k) { return n_hsteps - 1 - (k - n_own); };
  // sparse scope with a saved context: history rows read their log gates
  const bool use_lg2 = SPARSE && a.lg2 != nullptr;
  // sparse scope: record of row 0 of history step k is rec0 + hstep(k) RS
  const size_t rec0 = SPARSE ? (size_t(pair) * L.ents_per_pair + (lst - (L.ents + size_t(pair) * L.ents_per_pair))) * G
                             : 0;
  // Token of the i-th token slot of step k, in two parts.  tok_raw issues
  // the slot's list-entry load (sparse history steps; own steps read a valid
  // word of the workspace) and returns the word unexamined; tok_fin makes it
  // the slot's token (-1: none).  tok_fin runs a step later, after that
  // step's wait for its ring stage: a use of the loaded word right away would
  // make the wave wait for the tile loads issued before it as well (vector
  // memory operations complete in order), i.e. for the next step's tiles.
  auto tok_raw = [&](int k, int i) -> uint32_t {
    if constexpr (SPARSE) {
      const bool own = k < n_own;
      const int p = hstep(k) * TPS + i;
      return (own ? L.ents : lst)[own ? 0 : min(max(p, 0), max(n_hist - 1, 0))];
    } else {
      return 0u;
    }
  };
  auto tok_fin = [&](int k, int i, uint32_t e) -> int {
    const bool own = k < n_own;
    const int p = own ? k * TPS + i : hstep(k) * TPS + i;
    const int lim = own ? own_n : n_hist;
    int t = own ? j0 + p : j0 + KT + p;
    if constexpr (SPARSE) {
      if (!own) t = int(e);  // token | rank << 23 (rank < 256: stays positive)
    }
    return p < lim ? t : -1;
  };

  // token of a valid token slot (sparse history slots also carry the rank)
  auto tok_of = [](int t) { return SPARSE ? t & kTokMask : t; };
  auto rst = [&](auto tag) -> uint16_t* {
    if constexpr (decltype(tag)::value == 0) return R0;
    else return R1;
  };
  // Per-lane offsets that stay fixed from step to step, kept in registers: the
  // Q / dO source of each 1 KB piece relative to token 0 and the row whose
  // token it gathers, the stat row base of the lane's row, and the LDS
  // offsets of the transposed reads of the Q / dO tile.
  int prow[PPW];
  size_t poff[PPW];
#pragma unroll
  for (int i = 0; i < PPW; ++i) {
    const int sl = 64 * (wave * PPW + i) + lane;  // 16-byte slot: row r, stored chunk pc
    const int r = sl / CH, pc = sl % CH;
    prow[i] = r;
    poff[i] = (hrow0 + size_t(r % G) * N) * D + ((pc ^ k_swz<D>(r)) * 8);
  }
  const size_t srow = hrow0 + size_t(lane % G) * N;
  int troff[ND][2][2];
  {
    const int lr = lane & 15, lq = lane >> 4;
    const int trow = 4 * lq + (lr >> 2), tcol = 4 * (lr & 3);
#pragma unroll
    for (int nd = 0; nd < ND; ++nd)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int ra = 32 * kk + 16 * h + trow;
          const int col = 16 * nd + tcol;
          troff[nd][kk][h] = ra * D + (((col >> 3) ^ k_swz<D>(ra)) << 3) + (col & 7);
        }
  }
  // Loads of step k into stage `tag`; tk: token of the lane's row ln of the
  // step (ln: opaque lane index).
  auto issue = [&](auto tag, int k, int tk, int ln) {
    constexpr int P = decltype(tag)::value;
    const int phase = k < n_own ? 0 : 1;
    uint16_t* st = rst(tag);
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
      const int j = wave * PPW + i;  // 1 KB piece of the Q (dO) tile
      const int t = __shfl(tk, prow[i], 64);
      const size_t off = poff[i] + size_t(t >= 0 ? tok_of(t) : 0) * D;
      __builtin_amdgcn_global_load_lds(a.q + off, (lds_ptr_t)(st + j * 512), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(a.dout + off, (lds_ptr_t)(st + ST_DO + j * 512), 16, 0, 0);
    }
    {
      const int r = ln;  // stat `wave` of row r
      const int t = tk;
      const size_t gr = srow + (t >= 0 ? tok_of(t) : 0);
      // slot 2 of a history row: its saved base-2 log gate (the record of
      // row r of the step, as for dbeta), else its score (slot 3: LSE_s).
      // Own-block rows use neither; they read lse there, which always exists.
      const float* s2 = use_lg2 ? a.lg2 + rec0 + (t >= 0 ? size_t(hstep(k)) * RS + r : 0)
                                : a.scores + gr * C + m;
      // (slot 3, LSE_s, is not needed with saved log gates: that wave reads
      // the lse word again, one the workgroup has just fetched)
      const float* src = wave == 0 ? a.lse + gr
                       : wave == 1 ? a.delta + gr
                       : wave == 2 ? (phase == 1 ? s2 : a.lse + gr)
                                   : (use_lg2 ? a.lse : a.lse_s) + gr;
      __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(st + ST_F + wave * RS * 2), 4, 0, 0);
      if (wave == 0) tok_sh[P][r] = t;
    }
  };

  // One step on stage `tag`; MK: own-block rows (causal, bias 0) else gated history rows.
  auto compute = [&](auto tag, auto mkt, int ln, int kcur) {
    constexpr int P = decltype(tag)::value;
    constexpr bool MK = decltype(mkt)::value;
    const uint16_t* Qs = rst(tag);
    const uint16_t* dOs = Qs + ST_DO;
    const float* F = reinterpret_cast<const float*>(Qs + ST_F);
    const int lr = ln & 15, lq = ln >> 4;
    const int key = j0 + wave * 16 + lr;
    // S and dP for the 64 rows: 4 row subtiles of 16 (A row 16 rs + lr,
    // k = d chunk 4 ks + lq stored at chunk (4 ks + lq) ^ k_swz(row), which
    // depends on lr alone).
    const int qsw = k_swz<D>(lr);
    f32x4 sacc[4], pacc[4];
#pragma unroll
    for (int rs = 0; rs < 4; ++rs) {
      sacc[rs] = f32x4{0.f, 0.f, 0.f, 0.f};
      pacc[rs] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int rs = 0; rs < 4; ++rs) {
        const int off = (16 * rs + lr) * D + (((4 * ks + lq) ^ qsw) * 8);
        const uint4 qa = *reinterpret_cast<const uint4*>(Qs + off);
        const uint4 oa = *reinterpret_cast<const uint4*>(dOs + off);
        sacc[rs] = mfma16(qa, kf[ks], sacc[rs]);
        pacc[rs] = mfma16(oa, vf[ks], pacc[rs]);
      }
    // P and dS: lane holds key `key`, rows 16 rs + 4 lq + i.
    uint4 pa[2], dsa[2];
    float dsum[SPARSE ? 16 : 1];
#pragma unroll
    for (int rs = 0; rs < 4; ++rs) {
      const int r0 = 16 * rs + 4 * lq;
      const float4 lse = *reinterpret_cast<const float4*>(F + r0);
      const float4 del = *reinterpret_cast<const float4*>(F + RS + r0);
      const float4 sc = *reinterpret_cast<const float4*>(F + 2 * RS + r0);
      const float4 lss = *reinterpret_cast<const float4*>(F + 3 * RS + r0);
      const int4 tk = *reinterpret_cast<const int4*>(&tok_sh[P][r0]);
      const float lv[4] = {lse.x, lse.y, lse.z, lse.w}, dl[4] = {del.x, del.y, del.z, del.w};
      const float sv[4] = {sc.x, sc.y, sc.z, sc.w}, ls[4] = {lss.x, lss.y, lss.z, lss.w};
      const int tv[4] = {tk.x, tk.y, tk.z, tk.w};
      float p[4], d[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // base-2 log gate of a history row, then the base-2 logit offset:
        // bias - lse
        const float lg = use_lg2 ? sv[i] : (sv[i] - ls[i]) * kLog2e;
        const float off = (MK || OUTER) ? -lv[i] * kLog2e : lg - lv[i] * kLog2e;
        float x = fmaf(sacc[rs][i], c1, off);
        const bool ok = tv[i] >= 0 && key < N && (!MK || key <= tv[i]);
        x = ok ? x : kNegInf;
        p[i] = exp2_hw(x);
        if constexpr (OUTER && !MK) {
          const float gf = ok ? exp2_hw(lg) : 0.f;
          const float gdp = gf * pacc[rs][i];
          d[i] = p[i] * (gdp - dl[i]);
          if constexpr (SPARSE) dsum[4 * rs + i] = p[i] * gdp;  // g dg, in dbeta's place
          p[i] *= gf;                                         // g P for dV
        } else {
          d[i] = p[i] * (pacc[rs][i] - dl[i]);
        }
      }
      const int kk = rs >> 1;
      const uint32_t d01 = pack_bf16(d[0], d[1]), d23 = pack_bf16(d[2], d[3]);
      if (rs & 1) {
        pa[kk].z = pack_bf16(p[0], p[1]);
        pa[kk].w = pack_bf16(p[2], p[3]);
        dsa[kk].z = d01;
        dsa[kk].w = d23;
      } else {
        pa[kk].x = pack_bf16(p[0], p[1]);
        pa[kk].y = pack_bf16(p[2], p[3]);
        dsa[kk].x = d01;
        dsa[kk].y = d23;
      }
      if constexpr (SPARSE) {
        // dS rows for the dQ pass (the bf16 values of the MFMA operand), and
        // this wave's share of the row sums
        uint16_t* col = dst_sh + r0 * TST + wave * 16 + lr;
        col[0] = uint16_t(d01);
        col[TST] = uint16_t(d01 >> 16);
        col[2 * TST] = uint16_t(d23);
        col[3 * TST] = uint16_t(d23 >> 16);
        if constexpr (!(OUTER && !MK)) {
#pragma unroll
          for (int i = 0; i < 4; ++i) dsum[4 * rs + i] = d[i];
        }
      }
    }
    // dV += P^T dO, dK += dS^T Q.  B operand (32 rows x 16 columns) read
    // transposed: lane s of group lq points at row 32 kk + 4 lq + s / 4 (and
    // + 16), column 16 nd + 4 (s % 4).
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int oa = troff[nd][kk][0], ob = troff[nd][kk][1];
        const uint2 o0 = lds_read_tr16(dOs + oa), o1 = lds_read_tr16(dOs + ob);
        const uint2 q0 = lds_read_tr16(Qs + oa), q1 = lds_read_tr16(Qs + ob);
        dv[nd] = mfma16(pa[kk], make_uint4(o0.x, o0.y, o1.x, o1.y), dv[nd]);
        dk[nd] = mfma16(dsa[kk], make_uint4(q0.x, q0.y, q1.x, q1.y), dk[nd]);
      }
    }
    if constexpr (SPARSE) {
      // Sum over the wave's 16 keys (lanes lr): afterwards lane lr holds
      // value lr, i.e. row 16 (lr / 4) + 4 lq + lr % 4.
#pragma unroll
      for (int M = 8, n = 16; M >= 1; M >>= 1, n >>= 1) {
        const bool hi = (lr & M) != 0;
#pragma unroll
        for (int j = 0; j < n / 2; ++j) {
          const float send = hi ? dsum[j] : dsum[j + n / 2];
          const float keep = hi ? dsum[j + n / 2] : dsum[j];
          dsum[j] = keep + __uint_as_float(lanes_xor(__float_as_uint(send), M, ln));
        }
      }
      dbs_sh[wave * RS + 16 * (lr >> 2) + 4 * lq + (lr & 3)] = dsum[0];
      ring_barrier();  // the step's dS rows and row sums are complete
      const int* tkr = tok_sh[P];
      // dbeta records: history rows r of step k are consecutive (entry, head)
      // records
      const int tid = wave * 64 + ln;
      if (!MK && tid < RS && tkr[tid] >= 0) {
        const float db = dbs_sh[tid] + dbs_sh[RS + tid] + dbs_sh[2 * RS + tid] + dbs_sh[3 * RS + tid];
        a.dbl[rec0 + size_t(hstep(kcur)) * RS + tid] = db;
      }
      // The rows' dQ shares over this block: dQ^T = K^T dS^T (B operand: row
      // 16 rs + lr, keys 32 kk + 8 lq .. of the dS rows), unscaled.  Lane
      // holds columns 16 (NDW wave + nd) + 4 lq .. + 3 of its row; they are
      // staged as bf16 rows over the step's consumed Q and dO tiles, then
      // leave as whole rows, 16 bytes a lane, to the row's slot (own rows:
      // slot topk; history rows: the entry's rank).  The stores are
      // non-temporal: the shares are read once, by the rows kernel, and kept
      // out of the way of the gathered Q and dO rows in L2 (the kernel ran
      // 7% faster than with 8-byte pieces stored straight from registers).
      constexpr int WST = D + 8;
      uint16_t* wst = rst(tag);
#pragma unroll
      for (int rs = 0; rs < 4; ++rs) {
        const int r = 16 * rs + lr;
        const uint4 b0 = *reinterpret_cast<const uint4*>(dst_sh + r * TST + 8 * lq);
        const uint4 b1 = *reinterpret_cast<const uint4*>(dst_sh + r * TST + 32 + 8 * lq);
        // The row's address is formed once and kept opaque: built from the
        // stage array in few steps, every store keeps the array's alias
        // scope, so the compiler sees it cannot touch the other stage and
        // does not wait here for that stage's loads (a longer address chain
        // lost the scope on the second tile's store and drained them).
        int wo = r * WST + 16 * NDW * wave + 4 * lq;
        asm volatile("" : "+v"(wo));
        uint16_t* wrow = wst + wo;
#pragma unroll
        for (int nd = 0; nd < NDW; ++nd) {
          f32x4 acc = mfma16(kq[nd][0], b0, f32x4{0.f, 0.f, 0.f, 0.f});
          acc = mfma16(kq[nd][1], b1, acc);
          *reinterpret_cast<uint2*>(wrow + 16 * nd) =
              make_uint2(pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3]));
        }
      }
      ring_barrier();  // the staged dQ rows are complete
#pragma unroll
      for (int u = 0; u < RS * CH / NT; ++u) {
        const int r = (u * NT + tid) / CH, cc = (u * NT + tid) % CH;
        const int e = tkr[r];
        // rows the step does not hold store to the dummy row, so that every
        // step issues the same stores (the next step's wait leaves them in
        // flight)
        const int slot = MK ? a.topk : e >> 23;
        bf16_t* dst = e >= 0 ? a.dqp + ((hrow0 + size_t(r % G) * N + (e & kTokMask)) * (a.topk + 1) + slot) * D
                             : a.dummy;
        const uint4 v = *reinterpret_cast<const uint4*>(wst + r * WST + cc * 8);
        __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(dst + cc * 8));
      }
    }
  };

  // ---- the ring: step k computes stage k % 2 and loads step k + 1 into the other
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using Own = std::integral_constant<bool, true>;
  using Hist = std::integral_constant<bool, false>;
  // the lane's row: step 0's token, and step 1's raw list word
  if (n_steps > 0) issue(S0{}, 0, tok_fin(0, lane / G, tok_raw(0, lane / G)), lane);
  uint32_t raw1 = n_steps > 0 ? tok_raw(min(1, n_steps - 1), lane / G) : 0u;
  wait_vm<0>();
  // One step on stage `tag`: wait for its rows, load step k + 1 into the
  // other stage and the raw list words of step k + 2 (the last step's again
  // past the end: an unconditional load, never examined), compute.
  auto step = [&](auto tag, auto mkt, int k) {
    using Pn = std::integral_constant<int, decltype(tag)::value ^ 1>;
    int ln = lane;
    asm volatile("" : "+v"(ln));
    // this stage's rows and the list words; at sparse scope every step ends
    // with the same RS * CH / NT share stores, which stay in flight (before
    // the first step nothing is in flight)
    wait_vm<SPARSE ? RS * CH / NT : 0>();
    ring_barrier();
    if (k + 1 < n_steps) issue(Pn{}, k + 1, tok_fin(k + 1, ln / G, raw1), ln);
    const uint32_t raw2 = tok_raw(min(k + 2, n_steps - 1), ln / G);
    compute(tag, mkt, ln, k);
    raw1 = raw2;
  };
  // Own-block steps (one variant per loop: no accumulator merges), then the
  // history on the stage where the first loop stopped.
  int k = 0;
  for (; k + 1 < n_own; k += 2) {
    step(S0{}, Own{}, k);
    step(S1{}, Own{}, k + 1);
  }
  if (k < n_own) {
    step(S0{}, Own{}, k);
    ++k;
  }
  if ((k & 1) && k < n_steps) {
    step(S1{}, Hist{}, k);
    ++k;
  }
  for (; k + 1 < n_steps; k += 2) {
    step(S0{}, Hist{}, k);
    step(S1{}, Hist{}, k + 1);
  }
  if (k < n_steps) step(S0{}, Hist{}, k);


  // Write dK (scaled) and dV: lane holds column 16 nd + lr of keys 4 lq + i of
  // the wave's 16.
  const int lr = lane & 15, lq = lane >> 4;
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

// Per sparse-scope row, one wave:
//   dq = scale * (sum of the row's dQ share slots: its selected blocks' slots
//        0 .. nsel-1 and the own block's slot topk), and
//   ds[m] = (m selected ? dbeta[slot(m)] : 0) - g[m] * sum(dbeta) for the
//        history blocks m < c, g = exp(s - LSE_s); 0 from the own block on
//        (slot(m) = rank of m among the row's selected blocks; its dbeta is
//        the record of the row's entry in m's list, pos[token][slot]);
//        GATE: the gate activation, whose chain rule gate_ds applies (the
//        softmax gate's is the formula above); hist_only: the columns from
//        the own block on are not written.
// Each lane takes 2 dq columns and 8 consecutive blocks per pass.
template <int D, int GATE>
__global__ __launch_bounds__(256) void rows_sparse_kernel(
    const bf16_t* __restrict__ dqp, const float* __restrict__ dbl, const uint32_t* __restrict__ pos,
    size_t ents_per_pair, const float* __restrict__ scores,
    const float* __restrict__ lse_s, const uint32_t* __restrict__ selbits,
    const uint16_t* __restrict__ selpre, bf16_t* __restrict__ dq, float* __restrict__ ds, int Hq, int G,
    int N, int C, int MWB, int topk, float scale, size_t rows, int hist_only) {
  constexpr int LPS = D / 2;       // lanes per slot (2 columns each)
  constexpr int SG = 64 / LPS;     // slots per pass
  const size_t row = size_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int t = int(row % N);
  const size_t bh = row / N;
  const size_t tok = (bh / Hq * (Hq / G) + (bh % Hq) / G) * N + t;
  const int c = min(t / KT, C);
  const int nsel = selpre[tok * (MWB + 1) + MWB];
  const int topk1 = topk + 1;

  // dbeta of slot s2: record pos[tok][s2] of the pair's list entries, head h.
  // Lane s2 (< 64) fetches slot s2's value once; the ds loop takes it by
  // shuffle.  The address loads go out before the dQ slot loads, so both
  // gathers overlap.
  const int h = int(bh % Hq) % G;
  const float* dbp = dbl + (bh / Hq * (Hq / G) + (bh % Hq) / G) * ents_per_pair * G + h;
  const uint32_t* ps = pos + tok * topk;
  const uint32_t pl = lane < nsel ? ps[lane] : 0u;

  // ---- dq: the slot loads of up to 16 slots per round trip
  {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(dqp) + row * size_t(topk1) * LPS + lane % LPS;
    float a0 = 0.f, a1 = 0.f;
    constexpr int U = 16;
    // the own block's slot first, then the selected slots s2 = lane / LPS + SG j
    uint32_t wo = lane < LPS ? src[size_t(topk) * LPS] : 0u;
    for (int s0 = lane / LPS; s0 < nsel; s0 += U * SG) {
      uint32_t w[U];
#pragma unroll
      for (int u = 0; u < U; ++u)  // (non-temporal: each share is read once)
        w[u] = s0 + u * SG < nsel ? __builtin_nontemporal_load(src + size_t(s0 + u * SG) * LPS) : 0u;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        a0 += bf16_lo(w[u]);
        a1 += bf16_hi(w[u]);
      }
    }
    a0 += bf16_lo(wo);
    a1 += bf16_hi(wo);
    if (SG == 2) {
      a0 += shfl_xor(a0, 32);
      a1 += shfl_xor(a1, 32);
    }
    if (lane < LPS) reinterpret_cast<uint32_t*>(dq)[row * LPS + lane] = pack_bf16(a0 * scale, a1 * scale);
  }

  // ---- ds
  const float dbl_lane = lane < nsel ? dbp[size_t(pl) * G] : 0.f;
  float tot = dbl_lane;
  for (int s2 = lane + 64; s2 < nsel; s2 += 64) tot += dbp[size_t(ps[s2]) * G];
  for (int off = 32; off >= 1; off >>= 1) tot += shfl_xor(tot, off);
  const float ls = lse_s[row];
  const float* srow = scores + row * C;
  float* drow = ds + row * C;
  const uint32_t* bits = selbits + tok * MWB;
  const bool vec = (C & 3) == 0;
  const int ncol = hist_only ? c : C;  // columns written (hist_only: the history)
  int run = 0;
  for (int m0 = 0; m0 < ncol; m0 += 512) {
    const int col0 = m0 + 8 * lane;
    const uint32_t b8 = col0 < c ? (bits[col0 >> 5] >> (col0 & 31)) & 0xffu : 0u;
    const int cnt = __popc(b8);
    int incl = cnt;
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    const int excl = run + incl - cnt;
    run += __shfl(incl, 63, 64);
    // dbeta of this lane's 8 blocks; the shuffles run with every lane active
    // (a lane reading an inactive lane's register would get 0)
    float dbv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int s2 = excl + __popc(b8 & ((1u << i) - 1u));
      const float sh = __shfl(dbl_lane, s2 & 63, 64);
      dbv[i] = ((b8 >> i) & 1u) ? (s2 < 64 ? sh : dbp[size_t(ps[s2]) * G]) : 0.f;
    }
    float out[8];
    if (col0 < c && vec && col0 + 8 <= C) {
      const float4 sa = *reinterpret_cast<const float4*>(srow + col0);
      const float4 sb = *reinterpret_cast<const float4*>(srow + col0 + 4);
      const float sv[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) out[i] = col0 + i < c ? gate_ds(GATE, dbv[i], sv[i] - ls, tot) : 0.f;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int m2 = col0 + i;
        out[i] = m2 < c ? gate_ds(GATE, dbv[i], srow[m2] - ls, tot) : 0.f;
      }
    }
    if (vec && col0 + 8 <= ncol) {  // non-temporal: nothing here reads ds again
      typedef float f32x4v __attribute__((ext_vector_type(4)));
      __builtin_nontemporal_store(f32x4v{out[0], out[1], out[2], out[3]}, reinterpret_cast<f32x4v*>(drow + col0));
      __builtin_nontemporal_store(f32x4v{out[4], out[5], out[6], out[7]},
                                  reinterpret_cast<f32x4v*>(drow + col0 + 4));
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (col0 + i < ncol) drow[col0 + i] = out[i];
    }
  }
}

// -------------------------------------------------------------------- dQ ----
// Query-major, the forward's structure: a workgroup owns TOK_WG tokens
// of one KV head (all G query heads: 16 * NSUB * WAVES rows, a lane per row)
// and streams the tiles its rows attend through an NST-stage LDS ring filled by
// direct global -> LDS loads of K and V, row-major: A operands of S^T = K Q^T
// and dP^T = V dO^T, and (read transposed) of dQ^T = K^T dS^T.
// Per tile and row: P = exp2(S scale log2e + bias - lse log2e),
// dZ = P (dP - Delta), dbeta = sum of dZ over the tile (gated history tiles
// only, written to ds as scratch), dZ packed to bf16 for the dQ product.  Own
// blocks run in a second, masked loop.  The epilogue writes dq and turns the
// row's dbeta into ds = dbeta - g sum(dbeta) (dense over the history).  This
// is the full-scope dQ; at sparse scope the dK/dV kernel writes per-block dQ
// shares that the rows kernel sums.
template <int D, int G, int NSUB, int WAVES, int NST, bool OUTER>
__global__ __launch_bounds__(64 * WAVES, WAVES >= 8 ? 2 : 1) void bwd_dq_kernel(BwdArgs a) {
  using namespace tiles;
  constexpr int NT = 64 * WAVES;
  constexpr int KS = D / 32;
  constexpr int MD = D / 16;
  constexpr int TOK_SUB = 16 / G;
  constexpr int ROWS_WG = 16 * NSUB * WAVES;
  constexpr int TOK_WG = ROWS_WG / G;
  constexpr int CH = D / 8;
  constexpr int NKL = KT * D * 2 / 1024;  // 1 KB wave loads per operand tile
  constexpr int LPW = NKL / WAVES;
  constexpr int L = 2 * LPW + 1;          // loads per wave per tile
  static_assert(NKL % WAVES == 0, "tile loads must split evenly over the waves");
  static_assert(16 * NSUB <= 64, "one score load covers a wave's rows");
  static_assert(NST == 2 || NST == 3, "two or three ring stages");
  __shared__ __attribute__((aligned(16))) uint16_t K0[KT * D], K1[KT * D], K2[NST > 2 ? KT * D : 8];
  __shared__ __attribute__((aligned(16))) uint16_t V0[KT * D], V1[KT * D], V2[NST > 2 ? KT * D : 8];
  __shared__ __attribute__((aligned(16))) float S0[WAVES * 64], S1[WAVES * 64], S2[NST < 3 ? 1 : WAVES * 64];
  __shared__ float tot_sh[ROWS_WG];
  // per row: lse (base 2), Delta, LSE_s -- read per step rather than held in
  // registers across the tile loop
  __shared__ float rstat[ROWS_WG][4];
  __shared__ int wg_last;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  int tile, pair;
  xcd_order(blockIdx.x, a.n_tiles, a.n_pairs, &tile, &pair);
  const int b = pair / a.Hkv, g = pair % a.Hkv;
  const int N = a.N, C = a.C;
  const int t_wg0 = tile * TOK_WG;
  const float c1 = a.scale * kLog2e;

  // Row of subtile s for lane row index r (0..15): token and query head.
  auto tok_of = [&](int s, int r) { return t_wg0 + (wave * NSUB + s) * TOK_SUB + r / G; };
  auto head_of = [&](int r) { return g * G + r % G; };
  int c_sub[NSUB];
  bool sub_live[NSUB];
  for (int s = 0; s < NSUB; ++s) {
    const int t0 = t_wg0 + (wave * NSUB + s) * TOK_SUB;
    c_sub[s] = t0 / KT;
    sub_live[s] = t0 < N;
  }

  if (tid == 0) wg_last = -1;
  __syncthreads();
  {
    int lt = -1;
    for (int s = 0; s < NSUB; ++s) lt = max(lt, sub_live[s] ? c_sub[s] : -1);
    if (lane == 0) atomicMax(&wg_last, lt);
  }
  __syncthreads();
  const int last_tile = wg_last;

  // ---- row state: Q and dO fragments (B operands), lse, Delta, lse_s ----------
  uint4 qf[NSUB][KS], of[NSUB][KS];
  float dbt[NSUB];
  f32x4 dqa[NSUB][MD];
  for (int s = 0; s < NSUB; ++s) {
    const int rt = tok_of(s, lr);
    const bool ok = rt < N;
    const size_t gr = (size_t(b) * a.Hq + head_of(lr)) * N + (ok ? rt : 0);
    for (int ks = 0; ks < KS; ++ks) {
      qf[s][ks] = ok ? *reinterpret_cast<const uint4*>(a.q + gr * D + ks * 32 + lq * 8) : make_uint4(0, 0, 0, 0);
      of[s][ks] = ok ? *reinterpret_cast<const uint4*>(a.dout + gr * D + ks * 32 + lq * 8) : make_uint4(0, 0, 0, 0);
    }
    if (lq == 0) {
      float* rs = rstat[(wave * NSUB + s) * 16 + lr];
      rs[0] = ok ? a.lse[gr] * kLog2e : 0.f;
      rs[1] = ok ? a.delta[gr] : 0.f;
      rs[2] = ok ? a.lse_s[gr] : 0.f;
    }
    dbt[s] = 0.f;
    for (int md = 0; md < MD; ++md) dqa[s][md] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto next_tile = [&](int mm) -> int { return (mm + 1 <= last_tile) ? mm + 1 : -1; };


  // ---- direct global -> LDS tile loads ------------------------------------------
  const bf16_t* kh = a.k + (size_t(b) * a.Hkv + g) * size_t(N) * D;
  const bf16_t* vh = a.v + (size_t(b) * a.Hkv + g) * size_t(N) * D;
  auto kst = [&](auto tag) -> uint16_t* {
    constexpr int P = decltype(tag)::value;
    if constexpr (P == 0) return K0;
    else if constexpr (P == 1) return K1;
    else return K2;
  };
  auto vst = [&](auto tag) -> uint16_t* {
    constexpr int P = decltype(tag)::value;
    if constexpr (P == 0) return V0;
    else if constexpr (P == 1) return V1;
    else return V2;
  };
  auto sst = [&](auto tag) -> float* {
    constexpr int P = decltype(tag)::value;
    if constexpr (P == 0) return S0;
    else if constexpr (P == 1) return S1;
    else return S2;
  };
  // ln: this lane's index, recomputed per step (see step).
  auto issue = [&](int m, auto tag, int ln) {
    uint16_t* kd = kst(tag);
    uint16_t* vd = vst(tag);
    if (m * KT + KT <= N) {
      const bf16_t* kt = kh + size_t(m) * KT * D;
      const bf16_t* vt = vh + size_t(m) * KT * D;
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        // 16-byte piece: tile row r, stored chunk pc, source chunk pc ^ k_swz(r)
        const int sl = 64 * (wave * LPW + i) + ln;
        const int r = sl / CH, pc = sl % CH;
        const uint32_t off = uint32_t(r * D + (pc ^ k_swz<D>(r)) * 8);
        __builtin_amdgcn_global_load_lds(kt + off, (lds_ptr_t)(kd + (wave * LPW + i) * 512), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vt + off, (lds_ptr_t)(vd + (wave * LPW + i) * 512), 16, 0, 0);
      }
    } else {
      // tail tile: keys past N repeat key N-1 (their logits are masked)
      for (int i = 0; i < LPW; ++i) {
        const int j = wave * LPW + i;
        const int sl = 64 * j + ln;
        const int r = sl / CH, pc = sl % CH;
        const size_t key = size_t(min(m * KT + r, N - 1));
        const int c = pc ^ k_swz<D>(r);
        __builtin_amdgcn_global_load_lds(kh + key * D + c * 8, (lds_ptr_t)(kd + j * 512), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vh + key * D + c * 8, (lds_ptr_t)(vd + j * 512), 16, 0, 0);
      }
    }
    {
      // score of row (ln % (16 NSUB)) of this wave, block m
      const int sr = ln % (16 * NSUB);
      const int st = min(tok_of(sr >> 4, sr & 15), N - 1);
      const float* sp = a.scores + ((size_t(b) * a.Hq + head_of(sr & 15)) * N + st) * C + min(m, C - 1);
      __builtin_amdgcn_global_load_lds(sp, (lds_ptr_t)(sst(tag) + wave * 64), 4, 0, 0);
    }
  };
  auto wait_tile = [&](int after) {
    switch (after) {
      case 0: wait_vm<0>(); break;
      case 1: wait_vm<L>(); break;
      default: wait_vm<(NST > 2 ? 2 * L : L)>(); break;
    }
  };

  int tq[NST];
  tq[0] = next_tile(-1);
  for (int i = 1; i < NST; ++i) tq[i] = tq[i - 1] >= 0 ? next_tile(tq[i - 1]) : -1;
  if (tq[0] >= 0) issue(tq[0], std::integral_constant<int, 0>{}, lane);
  if (NST > 2 && tq[1] >= 0) issue(tq[1], std::integral_constant<int, 1>{}, lane);

  auto step = [&](auto tag, auto mkt) {
    constexpr int P = decltype(tag)::value;
    constexpr bool MK = decltype(mkt)::value;
    const int m = tq[0];
    // Every lane-dependent offset below derives from an opaque copy of the lane
    // index, so none of them is kept live (or spilled) across the loop.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lr = ln & 15, lq = ln >> 4;
    int after = 0;
    for (int i = 1; i < NST - 1; ++i) after += tq[i] >= 0;
    wait_tile(after);
    ring_barrier();
    if (tq[NST - 1] >= 0) issue(tq[NST - 1], std::integral_constant<int, (P + NST - 1) % NST>{}, ln);
    const uint16_t* Ks = kst(tag);
    const uint16_t* Vs = vst(tag);
    const float* Ss = sst(tag);
    int nmask = 0;
    float bias2[NSUB], gsc[NSUB];
    bool gated[NSUB];
    int row_t[NSUB];
    float lse2[NSUB], del[NSUB];
    for (int s = 0; s < NSUB; ++s) {
      row_t[s] = tok_of(s, lr);
      const float4 rs = *reinterpret_cast<const float4*>(rstat[(wave * NSUB + s) * 16 + lr]);
      lse2[s] = rs.x;
      del[s] = rs.y;
      const float lses = rs.z;
      const bool own = (m == c_sub[s]);
      const bool hist = (m < c_sub[s]);
      bool sel = false;
      float bsel = kNegInf;
      if (hist && row_t[s] < N) {
        sel = true;
        bsel = (Ss[wave * 64 + 16 * s + lr] - lses) * kLog2e;
      }
      const bool nd = sub_live[s] && (own || (hist && __ballot(sel) != 0ull));
      nmask |= int(nd) << s;
      gated[s] = sel;
      // bias minus the row's lse (base 2); -inf where the row skips the tile.
      // OUTER: no bias, the gate g scales dP in dZ and in g dg (dbeta's place).
      const bool valid = row_t[s] < N && (own || sel);
      bias2[s] = valid ? (own || OUTER ? 0.f : bsel) - lse2[s] : kNegInf;
      gsc[s] = OUTER && sel && !own ? exp2_hw(bsel) : 1.f;
    }
    nmask = __builtin_amdgcn_readfirstlane(nmask);
    if (nmask) {
      // MFMA operand reads (the forward's addressing): K and V rows key =
      // 16 mt + lr, chunk (4 ks + lq) ^ k_swz(lr); K^T rows d = 16 md + lr,
      // chunk (4 kk + lq) ^ vt_swz(lr).
      const int ksw = k_swz<D>(lr);
      const uint32_t kb = lr * D + ((lq ^ (ksw & 3)) * 8), kx = (ksw >> 2) * 32;
      // One 16-key slice (mt) at a time: S^T = K Q^T and dP^T = V dO^T over the
      // k steps, then dZ = P (dP - Delta) for those keys, packed into dZ^T
      // fragments (keys 16 mt .. 16 mt + 15 are half of the k range of kk = mt/2).
      uint4 dsf[NSUB][2];
      float dsum[NSUB];
#pragma unroll
      for (int s = 0; s < NSUB; ++s) dsum[s] = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 sa[NSUB], pa[NSUB];
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
          sa[s] = f32x4{0.f, 0.f, 0.f, 0.f};
          pa[s] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint32_t off = mt * 16 * D + (((ks * 32) ^ kx) + kb);
          const uint4 kf = *reinterpret_cast<const uint4*>(Ks + off);
          const uint4 vf = *reinterpret_cast<const uint4*>(Vs + off);
#pragma unroll
          for (int s = 0; s < NSUB; ++s) {
            sa[s] = mfma16(kf, qf[s][ks], sa[s]);
            pa[s] = mfma16(vf, of[s][ks], pa[s]);
          }
        }
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
          float dz[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float x = fmaf(sa[s][i], c1, bias2[s]);
            if (MK && m * KT + 16 * mt + 4 * lq + i > row_t[s]) x = kNegInf;
            if constexpr (OUTER) {
              const float pv = exp2_hw(x), gdp = gsc[s] * pa[s][i];
              dz[i] = pv * (gdp - del[s]);
              dsum[s] += pv * gdp;
            } else {
              dz[i] = exp2_hw(x) * (pa[s][i] - del[s]);
              dsum[s] += dz[i];
            }
          }
          if (mt & 1) {
            dsf[s][mt >> 1].z = pack_bf16(dz[0], dz[1]);
            dsf[s][mt >> 1].w = pack_bf16(dz[2], dz[3]);
          } else {
            dsf[s][mt >> 1].x = pack_bf16(dz[0], dz[1]);
            dsf[s][mt >> 1].y = pack_bf16(dz[2], dz[3]);
          }
        }
      }
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        const float tsum = sum_xrows(dsum[s]);
        if (gated[s]) {
          dbt[s] += tsum;
          if (lq == 0) a.ds[((size_t(b) * a.Hq + head_of(lr)) * N + row_t[s]) * C + m] = tsum;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // dQ^T += K^T dS^T
#pragma unroll
      for (int md = 0; md < MD; ++md) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          // K^T fragment (A: d rows, keys along k in the dS^T order), read
          // transposed from the row-major K tile: lane s of group lq points at
          // key 32 kk + 4 lq + s / 4 (and + 16), column 16 md + 4 (s % 4).
          const int ra = 32 * kk + 4 * lq + (lr >> 2), rb = ra + 16;
          const int col = 16 * md + 4 * (lr & 3);
          const uint2 k0 = lds_read_tr16(Ks + ra * D + ((((col >> 3) ^ k_swz<D>(ra)) << 3) + (col & 7)));
          const uint2 k1 = lds_read_tr16(Ks + rb * D + ((((col >> 3) ^ k_swz<D>(rb)) << 3) + (col & 7)));
          const uint4 ka = make_uint4(k0.x, k0.y, k1.x, k1.y);
#pragma unroll
          for (int s = 0; s < NSUB; ++s) dqa[s][md] = mfma16(ka, dsf[s][kk], dqa[s][md]);
        }
      }
    }
    for (int i = 0; i < NST - 1; ++i) tq[i] = tq[i + 1];
    tq[NST - 1] = tq[NST - 2] >= 0 ? next_tile(tq[NST - 2]) : -1;
  };
  using Unmasked = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;
  const int c_first = t_wg0 / KT;
  int ph = 0;
  while (true) {
    if (tq[0] < 0 || tq[0] >= c_first) { ph = 0; break; }
    step(std::integral_constant<int, 0>{}, Unmasked{});
    if (tq[0] < 0 || tq[0] >= c_first) { ph = 1; break; }
    step(std::integral_constant<int, 1>{}, Unmasked{});
    if constexpr (NST > 2) {
      if (tq[0] < 0 || tq[0] >= c_first) { ph = 2; break; }
      step(std::integral_constant<int, (NST > 2 ? 2 : 0)>{}, Unmasked{});
    }
  }
  while (tq[0] >= 0) {
    if (ph == 0) step(std::integral_constant<int, 0>{}, Masked{});
    else if (ph == 1) step(std::integral_constant<int, 1>{}, Masked{});
    else step(std::integral_constant<int, (NST > 2 ? 2 : 0)>{}, Masked{});
    ph = ph + 1 == NST ? 0 : ph + 1;
  }

  // ---- epilogue: dQ (scaled), then ds = dbeta - g sum(dbeta) -----------------
  for (int s = 0; s < NSUB; ++s) {
    const int rt = tok_of(s, lr);
    if (rt >= N) continue;
    const size_t gr = (size_t(b) * a.Hq + head_of(lr)) * N + rt;
    for (int md = 0; md < MD; ++md) {
      uint2 w;
      w.x = pack_bf16(dqa[s][md][0] * a.scale, dqa[s][md][1] * a.scale);
      w.y = pack_bf16(dqa[s][md][2] * a.scale, dqa[s][md][3] * a.scale);
      *reinterpret_cast<uint2*>(a.dq + gr * D + 16 * md + 4 * lq) = w;
    }
  }
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
    if (a.gate == kGateSoftmax) {
      for (int m2 = lane; m2 < C; m2 += 64) {
        float out = 0.f;
        if (m2 < c) out = gate_ds(kGateSoftmax, drow[m2], srow[m2] - ls, tot);
        drow[m2] = out;
      }
    } else {
      for (int m2 = lane; m2 < C; m2 += 64) {
        float out = 0.f;
        if (m2 < c) out = gate_ds(a.gate, drow[m2], srow[m2] - ls, tot);
        drow[m2] = out;
      }
    }
  }
}

}  // namespace

bool bwd_mfma_supported(const Dims& d, int topk, bool sparse) {
  if (d.block != KT || (d.D != 64 && d.D != 128)) return false;
  if (d.C < 1) return false;
  const int G = d.G();
  if (G != 1 && G != 2 && G != 4 && G != 8) return false;
  // sparse scope: list entries hold the token in 23 bits and the slot in 9,
  // work items the block in 16 bits
  if (sparse && (d.N > (1 << 22) || topk > 256)) return false;
  return true;
}

// Workspace: Delta per row | (sparse) selection lists, the dQ share slots
// and the dbeta records.

struct BwdWs {
  size_t delta, lists, dqp, dbl, dummy, total;
};

static BwdWs bwd_ws_layout(const Dims& d, int topk, bool sparse) {
  BwdWs w{};
  const size_t rows = size_t(d.B) * d.Hq * d.N;
  w.delta = 0;
  size_t at = align_up(rows * sizeof(float));
  if (sparse) {
    size_t lb = 0;
    sel_lists_layout(d.B, d.Hkv, d.N, d.C, topk, KT, kListChunk, nullptr, &lb);
    w.lists = at;
    at += align_up(lb);
    w.dqp = at;
    at += align_up(rows * size_t(topk + 1) * d.D * sizeof(bf16_t));
    w.dbl = at;
    at += align_up(size_t(d.B) * d.Hkv * d.N * size_t(topk > 0 ? topk : 1) * d.G() * sizeof(float));
    w.dummy = at;
    at += align_up(size_t(d.D) * sizeof(bf16_t));
  }
  w.total = at;
  return w;
}

size_t bwd_mfma_workspace(const Dims& d, int topk, bool sparse) {
  return bwd_ws_layout(d, topk, sparse).total;
}

template <int D, int G>
static void launch_dq_sparse(BwdArgs a, const SelLists& L, size_t rows, hipStream_t s) {
#define SAS_ROWS_SPARSE(GT)                                                                                 \
  SAS_LAUNCH("rows_sparse", (rows_sparse_kernel<D, GT>), dim3((rows + 3) / 4), dim3(256), 0, s, a.dqp, a.dbl, \
             L.pos, L.ents_per_pair, a.scores, a.lse_s, a.selbits, a.selpre, a.dq, a.ds, a.Hq, G, a.N, a.C,   \
             a.MWB, a.topk, a.scale, rows, a.ds_hist_only)
  if (a.gate == kGateSigmoid) SAS_ROWS_SPARSE(kGateSigmoid);
  else if (a.gate == kGateRaw) SAS_ROWS_SPARSE(kGateRaw);
  else SAS_ROWS_SPARSE(kGateSoftmax);
#undef SAS_ROWS_SPARSE
}

template <int D, int G>
static void launch_dq_full(BwdArgs a, hipStream_t s) {
  constexpr int NSUB = 2, WAVES = 8, NST = 2;
  constexpr int TOK_WG = 16 * NSUB * WAVES / G;
  a.n_tiles = (a.N + TOK_WG - 1) / TOK_WG;
  if (a.gate == kGateOuter)
    SAS_LAUNCH("bwd_dq", (bwd_dq_kernel<D, G, NSUB, WAVES, NST, true>), dim3(a.n_tiles * a.n_pairs),
               dim3(64 * WAVES), 0, s, a);
  else
    SAS_LAUNCH("bwd_dq", (bwd_dq_kernel<D, G, NSUB, WAVES, NST, false>), dim3(a.n_tiles * a.n_pairs),
               dim3(64 * WAVES), 0, s, a);
}

template <int D, int G, bool SPARSE>
static hipError_t bwd_mfma_t(BwdArgs a, const SelLists& L, int B, hipStream_t s) {
  const size_t rows = size_t(B) * a.Hq * a.N;
  SAS_LAUNCH("bwd_delta_mfma", (bwd_delta_mfma_kernel<D>), dim3((rows + 256 / (D / 8) - 1) / (256 / (D / 8))),
             dim3(256), 0, s, a.o, a.dout, a.delta, rows);
  if (SPARSE && a.lg2 == nullptr) {  // (with a saved context the lists are there already)
    const hipError_t e = launch_sel_lists(a.idx, L, B, a.Hkv, a.N, a.C, a.topk, KT, s);
    if (e != hipSuccess) return e;
  }
  a.n_pairs = B * a.Hkv;
  a.n_tiles = (a.N + KT - 1) / KT;
  if (a.gate == kGateOuter)
    SAS_LAUNCH("bwd_dkdv", (bwd_dkdv_kernel<D, G, SPARSE, true>), dim3(a.n_tiles * a.n_pairs), dim3(256), 0, s, a, L);
  else
    SAS_LAUNCH("bwd_dkdv", (bwd_dkdv_kernel<D, G, SPARSE, false>), dim3(a.n_tiles * a.n_pairs), dim3(256), 0, s, a, L);
  if (SPARSE)
    launch_dq_sparse<D, G>(a, L, rows, s);
  else
    launch_dq_full<D, G>(a, s);
  return hipGetLastError();
}

hipError_t launch_bwd_mfma(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* scores, const int32_t* idx,
                           const float* lse, const float* lse_s, void* dq, void* dk, void* dv,
                           float* ds, const Dims& d, int topk, float scale, int gate, void* ws,
                           hipStream_t s, const void* ctx) {
  const bool sp = idx != nullptr;
  char* w = static_cast<char*>(ws);
  const BwdWs W = bwd_ws_layout(d, topk, sp);
  SelLists L{};
  // the lists: from the forward's saved context, or built into the workspace
  SparseCtx C{};
  if (sp && ctx) C = sparse_ctx_layout(d, topk, static_cast<char*>(const_cast<void*>(ctx)), nullptr);
  if (sp) L = ctx ? C.L : sel_lists_layout(d.B, d.Hkv, d.N, d.C, topk, KT, kListChunk, w + W.lists, nullptr);
  BwdArgs a{};
  a.q = (const bf16_t*)q;
  a.k = (const bf16_t*)k;
  a.v = (const bf16_t*)v;
  a.o = (const bf16_t*)o;
  a.dout = (const bf16_t*)dout;
  a.scores = scores;
  a.idx = idx;
  a.lse = lse;
  a.lse_s = lse_s;
  a.dq = (bf16_t*)dq;
  a.dk = (bf16_t*)dk;
  a.dv = (bf16_t*)dv;
  a.ds = ds;
  a.delta = reinterpret_cast<float*>(w + W.delta);
  if (sp) {
    a.selbits = L.bits;
    a.selpre = L.pre;
    a.dqp = reinterpret_cast<bf16_t*>(w + W.dqp);
    a.lg2 = C.lg2;
    a.ds_hist_only = ctx != nullptr;  // the saved-context backward leaves them to the caller
    a.dbl = reinterpret_cast<float*>(w + W.dbl);
    a.dummy = reinterpret_cast<bf16_t*>(w + W.dummy);
  }
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.N = d.N;
  a.C = d.C;
  a.topk = sp ? topk : 0;
  a.MWB = sp ? L.MWB : 1;
  a.NB = (d.N + KT - 1) / KT;
  a.scale = scale;
  a.gate = gate;
  const int G = d.G();
#define SAS_BWD_CASE(DD, GG)                                                                        \
  if (d.D == DD && G == GG)                                                                         \
    return sp ? bwd_mfma_t<DD, GG, true>(a, L, d.B, s) : bwd_mfma_t<DD, GG, false>(a, L, d.B, s);
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
