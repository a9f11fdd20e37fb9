// SAS gated attention forward at sparse scope, key-major over the selection
// lists (bf16 in, fp32 accumulate).
//
// The output of a row is a softmax over its own block (causal, bias 0) and its
// Top-K history blocks (bias log g = s - LSE_s): blog 方法核心; jaehun.me review
// "New Approach", paper Eq. 9, with the sparse branch's Top-K gate of "Why the
// Four Design Choices Matter".  A softmax over a union of blocks splits into
// per-block pieces: with m_b the block's max logit and l_b its sum of
// exp(logit - m_b), o = sum_b e^(m_b - M) (P_b V_b) / sum_b e^(m_b - M) l_b,
// M = max_b m_b, and LSE = M + log sum_b e^(m_b - M) l_b (the same merge the
// review's kernel paragraph, "A Concrete Walkthrough", applies tile by tile).
//
// fwd_sel  Persistent workgroups walk the work items of the selection lists (a
//          block's own tokens, or a run of its list entries within one token
//          span).  For an item of block m each wave owns 16 of its rows per
//          step and all 64 keys: lane = row, S^T = K Q^T with K from the
//          block's LDS tile, the row's block max and sum lane-local plus two
//          shuffles, and O^T = V^T P^T with P^T straight from the S^T
//          fragments (keys of a 32-wide k step in the order {4 lq + i, 16 +
//          4 lq + i}) and V^T laid out per lane in LDS in the same order.  The
//          block's unnormalised P V goes to the row's slot (rank of m among
//          the row's selected blocks, topk for the own block) and (m_b, l_b)
//          to a record per list entry and head (own block: per row).
// combine  One wave per row merges its slots into o and the LSE.
#include "common.h"
#include "internal.h"
#include "mfma.h"
#include "tiles.h"

#include <algorithm>
#include <type_traits>

namespace sas {
namespace {

constexpr int KT = 64;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct FwdSelArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  const float* gates;  // [pairs * N][topk][G]: base-2 log gate of each (token, slot) and head
  bf16_t* op;     // [B, Hq, N, topk + 1, D]: unnormalised P V of each slot
  float2* stl;    // [pairs, list entries, G]: (m_b, l_b) per list entry and head
  float2* sto;    // [B, Hq, N]: (m_b, l_b) of the own block
  bf16_t* o;
  float* lse;
  float* dummy;   // line that absorbs masked stores
  float* lg2;     // optional [pairs, list entries, G]: the base-2 log gate of each
                  // history (entry, head), kept for the backward
  int Hq, Hkv, N, C, topk, n_pairs;
  float scale;
};

// OUTER: the outer gate (no bias; P scaled by g = exp(s - LSE_s) in P V only,
// l from the unscaled P), so the combine's merge stays as it is.
template <int D, int G, bool OUTER>
__global__ __launch_bounds__(1024) void fwd_sel_kernel(FwdSelArgs a, SelLists L) {
  using namespace tiles;
  constexpr int WAVES = 16;
  constexpr int KS = D / 32;
  constexpr int ND = D / 16;
  constexpr int CH = D / 8;              // 16-byte chunks per row
  constexpr int RPL = 64 / CH;           // rows per wave-wide 16-byte access
  constexpr int STG = 16 * D;            // per wave stage: Q of 16 rows
  constexpr int NLD = 16 / RPL;          // wave DMA instructions per step
  constexpr int NSTORE = NLD + 1;        // stores per step: P V rows + (m, l)
  // Vector memory operations a step leaves in flight at its end: at least
  // this many are issued after the next step's tile loads (own items: the
  // entry load and the NSTORE stores; history items also the bias load
  // and, with a saved context, the log-gate store), and they complete in
  // order, so waiting until at most this many are outstanding means the
  // tiles have landed.
  constexpr int NAFTER = NSTORE + 1;
  static_assert(KT * D <= WAVES * STG, "V tile fits in the stage area");
  static_assert(16 % G == 0, "a 16-row group holds whole tokens");
  __shared__ __attribute__((aligned(16))) uint16_t Ksh[KT * D];   // K, row-major, swizzled
  __shared__ __attribute__((aligned(16))) uint4 VTa[2 * ND * 64];  // A operands of O^T, per lane
  __shared__ __attribute__((aligned(16))) uint16_t S0[WAVES * STG];
  __shared__ __attribute__((aligned(16))) uint16_t S1[WAVES * STG];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = a.N, C = a.C, pairs = a.n_pairs;
  const int topk1 = a.topk + 1;
  const float c1 = a.scale * kLog2e;
  const int total = pairs * L.maxitems;
  using S0t = std::integral_constant<int, 0>;
  using S1t = std::integral_constant<int, 1>;

  for (int vi = blockIdx.x; vi < total; vi += gridDim.x) {
    const int pair = vi % pairs, item = vi / pairs;
    if (item >= int(L.nitems[pair])) continue;
    const uint4 it = reinterpret_cast<const uint4*>(L.items)[size_t(pair) * L.maxitems + item];
    const int m = int(it.x & 0xffffu);
    const bool own_item = (it.x >> 31) != 0;
    const int b = pair / a.Hkv, g = pair % a.Hkv;
    const int j0 = m * KT;
    const int ntok = own_item ? min(KT, N - j0) : int(it.z - it.y);
    const uint32_t* ep = L.ents + size_t(pair) * L.ents_per_pair + it.y;
    const int nrows = ntok * G;
    const int ngroups = (nrows + 15) >> 4;
    const int nk = ngroups > wave ? (ngroups - wave + WAVES - 1) / WAVES : 0;
    const size_t hrow0 = (size_t(b) * a.Hq + g * G) * N;

    // ---- K tile (kept) and V tile (over stage 0) into LDS, then the A
    // operands of O^T (V^T, keys in the P^T order) laid out per lane.
    __syncthreads();  // the previous item is done with the tiles and stages
    {
      const bf16_t* kh = a.k + (size_t(b) * a.Hkv + g) * size_t(N) * D;
      const bf16_t* vh = a.v + (size_t(b) * a.Hkv + g) * size_t(N) * D;
      constexpr int KPIECE = KT * D * 2 / 1024;
      for (int j = wave; j < KPIECE; j += WAVES) {
        const int r = RPL * j + lane / CH, pc = lane % CH;
        const size_t key = size_t(min(j0 + r, N - 1));
        const int c = (pc ^ k_swz<D>(r)) * 8;
        dma16_to_lds(kh + key * D + c, Ksh + j * 512);
        dma16_to_lds(vh + key * D + c, S0 + j * 512);
      }
    }
    wait_vm<0>();
    __syncthreads();
    {
      const int lr = lane & 15, lq = lane >> 4;
      for (int u = wave; u < 2 * ND; u += WAVES) {
        const int kk = u / ND, md = u % ND;
        const int ka = 32 * kk + 4 * lq + (lr >> 2), kb = ka + 16;
        const int col = 16 * md + 4 * (lr & 3);
        const uint2 v0 = lds_read_tr16(S0 + ka * D + ((((col >> 3) ^ k_swz<D>(ka)) << 3) + (col & 7)));
        const uint2 v1 = lds_read_tr16(S0 + kb * D + ((((col >> 3) ^ k_swz<D>(kb)) << 3) + (col & 7)));
        VTa[u * 64 + lane] = make_uint4(v0.x, v0.y, v1.x, v1.y);
      }
    }
    __syncthreads();  // V tile read before stage 0 is reloaded; V^T operands written
    if (nk == 0) continue;

    // Lane constants of the item: row r_j = RPL j + lane / CH of a group is
    // loaded by this lane at chunk lane % CH; its head is r % G.
    size_t qoff[NLD], ooff[NLD];
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const int r = RPL * j + lane / CH, pc = lane % CH;
      const size_t hr = hrow0 + size_t(r % G) * N;
      qoff[j] = hr * D + ((pc ^ k_swz<D>(r)) * 8);
      ooff[j] = hr * size_t(topk1) * D + pc * 8;  // slot row of token 0, this lane's chunk
    }
    const size_t rbase = hrow0 + size_t((lane & 15) % G) * N;  // the lane's row lr
    // (m, l) records of the item's list entries: row q of the item is record q
    float2* stl_item = a.stl + (size_t(pair) * L.ents_per_pair + it.y) * G;
    float* lg2_item = a.lg2 == nullptr ? nullptr : a.lg2 + (size_t(pair) * L.ents_per_pair + it.y) * G;

    // Entry of row lr of group gk: token | slot << 23 (own block: slot
    // topk), in two parts.  entry_raw issues the list load (own items read a
    // valid word) and returns the word unexamined; entry_fin makes the entry.
    // The loaded word is first examined a step later, after that step's wait:
    // examining it at once would make the wave wait for the Q tile loads
    // issued before it as well (vector memory operations complete in order).
    auto entry_raw = [&](int gk, int lr) -> uint32_t {
      const int p = min((16 * gk + lr) / G, ntok - 1);
      return (own_item ? L.ents : ep)[own_item ? 0 : p];
    };
    auto entry_fin = [&](int gk, int lr, uint32_t v) -> uint32_t {
      const int p = min((16 * gk + lr) / G, ntok - 1);
      return own_item ? (uint32_t(j0 + p) | (uint32_t(a.topk) << 23)) : v;
    };
    auto stg = [&](auto tag) -> uint16_t* {
      if constexpr (decltype(tag)::value == 0) return S0 + wave * STG;
      else return S1 + wave * STG;
    };
    auto issue = [&](auto tag, int gk, uint32_t e, int ln) {
      uint16_t* st = stg(tag);
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        const int r = RPL * j + ln / CH;
        const uint32_t er = uint32_t(__shfl(int(e), r, 64));
        const uint32_t t = 16 * gk + r < nrows ? (er & 0x7fffffu) : 0u;
        dma16_to_lds(a.q + qoff[j] + size_t(t) * D, st + j * 512);
      }
    };
    // The row's log gate in base 2, (s - LSE_s) log2 e (own block: 0), from
    // the list build's record of the entry's (token, slot).  Split like the
    // entries: bias_raw loads it, bias_fin takes it a step later.
    const float* gate_row = a.gates + size_t(pair) * N * a.topk * G + (lane & 15) % G;
    auto bias_raw = [&](uint32_t e) -> float {
      if (own_item) return 0.f;
      return gate_row[(size_t(e & 0x7fffffu) * a.topk + (e >> 23)) * G];
    };
    auto bias_fin = [&](float r) -> float { return own_item ? 0.f : r; };

    auto compute = [&](auto tag, auto maskt, int gk, uint32_t e, float bias, int ln) {
      constexpr bool MASK = decltype(maskt)::value;
      uint16_t* Qs = stg(tag);
      const int lr = ln & 15, lq = ln >> 4;
      const int qsw = k_swz<D>(lr);  // = k_swz(16 kt + lr) for every kt
      f32x4 sacc[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) sacc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int off = lr * D + (((4 * ks + lq) ^ qsw) * 8);
        const uint4 qb = *reinterpret_cast<const uint4*>(Qs + off);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          sacc[kt] = mfma16(*reinterpret_cast<const uint4*>(Ksh + 16 * kt * D + off), qb, sacc[kt]);
      }
      const bool valid = 16 * gk + lr < nrows;
      const int t = int(e & 0x7fffffu);
      // keys a row may see: all (gated block), key <= t (own block), none
      // (rows past the item)
      const int tlim = valid ? (own_item ? t : 0x7fffffff) : -1;
      float x[4][4];
      float mx = kNegInf;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[kt][i] = fmaf(sacc[kt][i], c1, OUTER ? 0.f : bias);
          if (MASK) x[kt][i] = j0 + 16 * kt + 4 * lq + i <= tlim ? x[kt][i] : kNegInf;
          mx = fmaxf(mx, x[kt][i]);
        }
      mx = max_xrows(mx);
      const float ms = mx == kNegInf ? 0.f : mx;
      float l = 0.f;
      uint4 pb[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float p[8];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[4 * h + i] = exp2_hw(x[2 * kk + h][i] - ms);
            l += p[4 * h + i];
          }
        if constexpr (OUTER) {
          const float gate = exp2_hw(bias);  // g (own block: 1)
#pragma unroll
          for (int j = 0; j < 8; ++j) p[j] *= gate;  // the gate scales P V only
        }
        pb[kk] = make_uint4(pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]),
                            pack_bf16(p[6], p[7]));
      }
      l = sum_xrows(l);
      f32x4 oacc[ND];
#pragma unroll
      for (int md = 0; md < ND; ++md) oacc[md] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int md = 0; md < ND; ++md) oacc[md] = mfma16(VTa[(kk * ND + md) * 64 + ln], pb[kk], oacc[md]);
      // O^T fragments to the wave's stage (Q consumed) as rows, chunk c of row
      // r at c ^ (r % CH), then whole rows out.  Rows past the item go to the
      // dummy line, so each step issues the same count of stores.
      uint16_t* W = Qs;
#pragma unroll
      for (int md = 0; md < ND; ++md) {
        uint2 w;
        w.x = pack_bf16(oacc[md][0], oacc[md][1]);
        w.y = pack_bf16(oacc[md][2], oacc[md][3]);
        const int c = (2 * md + (lq >> 1)) ^ (lr % CH);
        *reinterpret_cast<uint2*>(W + lr * D + c * 8 + 4 * (lq & 1)) = w;
      }
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        const int r = RPL * j + ln / CH, cc = ln % CH;
        const uint32_t er = uint32_t(__shfl(int(e), r, 64));
        const uint4 v = *reinterpret_cast<const uint4*>(W + r * D + ((cc ^ (r % CH)) * 8));
        bf16_t* dp = 16 * gk + r < nrows
                         ? a.op + ooff[j] + (size_t(er & 0x7fffffu) * topk1 + (er >> 23)) * D
                         : reinterpret_cast<bf16_t*>(a.dummy) + cc * 8;
        // non-temporal: the slots are read once, by the combine kernel; kept
        // out of the way of the gathered query rows in L2 (measured 17%
        // faster kernel)
        __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(dp));
      }
      float2* sp = !valid ? reinterpret_cast<float2*>(a.dummy + 64)
                          : (own_item ? a.sto + rbase + t : stl_item + 16 * gk + lr);
      *sp = make_float2(mx, l);
      // the row's log gate for the backward (history rows)
      if (lg2_item != nullptr && !own_item && valid && lq == 0) lg2_item[16 * gk + lr] = bias;
    };

    // pipeline over this wave's groups gk = wave + WAVES k.  The raw words
    // of group k + 1 (entry, and the bias inputs) are loaded during step k - 1
    // and step k (unconditional loads: past the last group they repeat it,
    // never examined) and examined at the start of step k + 1.
    const int glast = wave + WAVES * (nk - 1);
    uint32_t e0 = entry_fin(wave, lane & 15, entry_raw(wave, lane & 15));
    uint32_t r1 = entry_raw(min(wave + WAVES, glast), lane & 15);
    issue(S0t{}, wave, e0, lane);
    float b0 = bias_fin(bias_raw(e0));
    float br1 = 0.f;
    wait_vm<0>();
    auto step = [&](auto tag, auto maskt, int k) {
      using Pn = std::integral_constant<int, decltype(tag)::value ^ 1>;
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int gk = wave + WAVES * k;
      const uint32_t e1 = entry_fin(gk + WAVES, ln & 15, r1);
      if (k + 1 < nk) {
        issue(Pn{}, gk + WAVES, e1, ln);
        br1 = bias_raw(e1);
      }
      const uint32_t r2 = entry_raw(min(gk + 2 * WAVES, glast), ln & 15);
      compute(tag, maskt, gk, e0, b0, ln);
      wait_vm<NAFTER>();
      e0 = e1;
      r1 = r2;
      b0 = bias_fin(br1);
    };
    // own items mask the keys after the row's token; history items need no
    // mask (a row past the item computes finite values from token 0's Q, and
    // its outputs go to the dummy line).  One loop per variant.
    auto steps = [&](auto maskt) {
      for (int k = 0; k < nk; k += 2) {
        step(S0t{}, maskt, k);
        if (k + 1 < nk) step(S1t{}, maskt, k + 1);
      }
    };
    if (own_item) steps(std::true_type{});
    else steps(std::false_type{});
  }
}

// Index into [B, Hq, N] rows of the r-th row in token-major order: the G query
// heads of one KV head and token are consecutive.
__device__ __forceinline__ size_t token_major_row(size_t r, int G, int N) {
  const size_t rest = r / G;
  return (rest / N * G + r % G) * N + rest % N;
}

// One wave per row (rows in token-major order, so that the G heads of a token
// read its (m, l) records together: 2% faster than head-major at 32K): o = sum_b e^(m_b - M) (P V)_b / sum_b e^(m_b - M) l_b over
// the own block and the row's selected blocks (slot s2 < nsel: block of rank
// s2, (m, l) in the record pos[token][s2] of the pair's list entries), and
// LSE = (M + log2 sum_b e^(m_b - M) l_b) ln 2 (logits in base 2 until here).
template <int D>
__global__ __launch_bounds__(256) void fwd_combine_kernel(FwdSelArgs a, SelLists L, int G, size_t rows) {
  constexpr int LPS = D / 2;    // lanes per slot (2 columns each)
  constexpr int SG = 64 / LPS;  // slots per pass
  const size_t r = size_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const int Hq = a.Hq, N = a.N, topk = a.topk;
  const size_t row = token_major_row(r, G, N);
  const int t = int(row % N);
  const size_t bh = row / N;
  const size_t pair = bh / Hq * (Hq / G) + (bh % Hq) / G;
  const size_t tok = pair * N + t;
  const int h = int(bh % Hq) % G;
  const int nsel = L.pre[tok * (L.MWB + 1) + L.MWB];
  const uint32_t* ps = L.pos + tok * topk;
  const float2* stl = a.stl + pair * L.ents_per_pair * G + h;
  auto st = [&](int s2) -> float2 { return stl[size_t(ps[s2]) * G]; };
  const float2 so = a.sto[row];
  // slot statistics lane-parallel (lane j: slot c0 + j), M over all of them
  float M = so.x;
  float2 ml0 = make_float2(kNegInf, 0.f);  // first 64 slots kept in registers
  for (int c0 = 0; c0 < nsel; c0 += 64) {
    const int s2 = c0 + lane;
    const float2 ml = s2 < nsel ? st(s2) : make_float2(kNegInf, 0.f);
    if (c0 == 0) ml0 = ml;
    M = fmaxf(M, ml.x);
  }
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, shfl_xor(M, off));
  // every row sees its own token, so M is finite
  const uint32_t* src = reinterpret_cast<const uint32_t*>(a.op) + row * size_t(topk + 1) * LPS + lane % LPS;
  const float wo = exp2_hw(so.x - M);
  float lsum = 0.f;
  float a0 = 0.f, a1 = 0.f;
  for (int c0 = 0; c0 < nsel; c0 += 64) {
    const int s2 = c0 + lane;
    const float2 ml = c0 == 0 ? ml0 : (s2 < nsel ? st(s2) : make_float2(kNegInf, 0.f));
    const float wl = exp2_hw(ml.x - M);  // 0 past nsel
    lsum += wl * ml.y;
    const int n = min(64, nsel - c0);
    // Every lane runs the same iterations: the shuffles read other lanes'
    // weights, and a lane reading an inactive lane's register gets 0.  Lane
    // half hf (SG = 2: two slots per pass) takes slot j0 + hf; past n it
    // reads a valid slot with weight 0.
    const int hf = lane / LPS;
    int j0 = 0;
    for (; j0 + 8 * SG <= n; j0 += 8 * SG) {
      uint32_t x[8];
      float w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int sl = j0 + u * SG + hf;  // < n
        x[u] = __builtin_nontemporal_load(src + size_t(c0 + sl) * LPS);  // read once
        w[u] = __shfl(wl, sl, 64);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        a0 = fmaf(w[u], bf16_lo(x[u]), a0);
        a1 = fmaf(w[u], bf16_hi(x[u]), a1);
      }
    }
    for (; j0 < n; j0 += SG) {
      const int sl = j0 + hf < n ? j0 + hf : j0;
      const uint32_t x = src[size_t(c0 + sl) * LPS];
      const float w = __shfl(wl, sl, 64);
      const float ww = j0 + hf < n ? w : 0.f;
      a0 = fmaf(ww, bf16_lo(x), a0);
      a1 = fmaf(ww, bf16_hi(x), a1);
    }
  }
  for (int off = 32; off >= 1; off >>= 1) lsum += shfl_xor(lsum, off);
  lsum += wo * so.y;
  if (lane < LPS) {
    const uint32_t x = src[size_t(topk) * LPS];
    a0 = fmaf(wo, bf16_lo(x), a0);
    a1 = fmaf(wo, bf16_hi(x), a1);
  }
  if (SG == 2) {
    a0 += shfl_xor(a0, 32);
    a1 += shfl_xor(a1, 32);
  }
  if (lane < LPS) {
    const float inv = 1.f / lsum;
    reinterpret_cast<uint32_t*>(a.o)[row * LPS + lane] = pack_bf16(a0 * inv, a1 * inv);
    if (lane == 0) a.lse[row] = (M + __builtin_amdgcn_logf(lsum)) * kLn2;
  }
}

struct FwdSelWs {
  size_t lists, gates, op, stl, sto, dummy, total;
};

FwdSelWs fwd_sel_layout(const Dims& d, int topk) {
  FwdSelWs w{};
  const size_t rows = size_t(d.B) * d.Hq * d.N;
  size_t lb = 0;
  sel_lists_layout(d.B, d.Hkv, d.N, d.C, topk, KT, kListChunk, nullptr, &lb);
  size_t at = 0;
  w.lists = at;
  at += align_up(lb);
  w.gates = at;
  at += align_up(size_t(d.B) * d.Hkv * d.N * size_t(topk > 0 ? topk : 1) * d.G() * sizeof(float));
  w.op = at;
  at += align_up(rows * size_t(topk + 1) * d.D * sizeof(bf16_t));
  w.stl = at;
  at += align_up(size_t(d.B) * d.Hkv * d.N * size_t(topk > 0 ? topk : 1) * d.G() * sizeof(float2));
  w.sto = at;
  at += align_up(rows * sizeof(float2));
  w.dummy = at;
  at += align_up(512);
  w.total = at;
  return w;
}

template <int D, int G>
hipError_t fwd_sel_t(const FwdSelArgs& a, const SelLists& L, int B, bool outer, hipStream_t s) {
  const size_t rows = size_t(B) * a.Hq * a.N;
  // persistent: one workgroup per compute unit (the LDS stages fill it)
  const int grid = std::min(a.n_pairs * L.maxitems, num_cus());
  if (outer)
    SAS_LAUNCH("fwd_sel", (fwd_sel_kernel<D, G, true>), dim3(grid), dim3(1024), 0, s, a, L);
  else
    SAS_LAUNCH("fwd_sel", (fwd_sel_kernel<D, G, false>), dim3(grid), dim3(1024), 0, s, a, L);
  SAS_LAUNCH("fwd_combine", (fwd_combine_kernel<D>), dim3((rows + 3) / 4), dim3(256), 0, s, a, L, G, rows);
  return hipGetLastError();
}

}  // namespace

size_t fwd_sel_workspace(const Dims& d, int topk) { return fwd_sel_layout(d, topk).total; }

// Sparse-scope forward over the selection lists (LSE_s already in lse_s).
// ctx (optional): the lists are built there instead of in the workspace, and
// the history entries' log gates are recorded beside them for the backward.
// gates (optional): the (token, slot) log gates, already written by the
// gated Top-K; else the list build writes them from the scores.
hipError_t launch_fwd_sel(const void* q, const void* k, const void* v, const float* scores,
                          const int32_t* idx, void* o, float* lse, const float* lse_s, const Dims& d,
                          int topk, float scale, bool outer, void* ws, hipStream_t s, void* ctx,
                          const float* gates) {
  char* w = static_cast<char*>(ws);
  const FwdSelWs W = fwd_sel_layout(d, topk);
  SparseCtx C{};
  if (ctx) C = sparse_ctx_layout(d, topk, static_cast<char*>(ctx), nullptr);
  const SelLists L =
      ctx ? C.L : sel_lists_layout(d.B, d.Hkv, d.N, d.C, topk, KT, kListChunk, w + W.lists, nullptr);
  const SelGates sg{scores, lse_s, reinterpret_cast<float*>(w + W.gates), d.Hkv, d.G(), d.C};
  const hipError_t e = launch_sel_lists(idx, L, d.B, d.Hkv, d.N, d.C, topk, KT, s, gates ? nullptr : &sg);
  if (e != hipSuccess) return e;
  FwdSelArgs a{};
  a.q = (const bf16_t*)q;
  a.k = (const bf16_t*)k;
  a.v = (const bf16_t*)v;
  a.gates = gates ? gates : sg.out;
  a.op = reinterpret_cast<bf16_t*>(w + W.op);
  a.stl = reinterpret_cast<float2*>(w + W.stl);
  a.sto = reinterpret_cast<float2*>(w + W.sto);
  a.o = (bf16_t*)o;
  a.lse = lse;
  a.dummy = reinterpret_cast<float*>(w + W.dummy);
  a.lg2 = C.lg2;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.N = d.N;
  a.C = d.C;
  a.topk = topk;
  a.n_pairs = d.B * d.Hkv;
  a.scale = scale;
  const int G = d.G();
#define SAS_FWDSEL_CASE(DD, GG) \
  if (d.D == DD && G == GG) return fwd_sel_t<DD, GG>(a, L, d.B, outer, s);
  SAS_FWDSEL_CASE(128, 4)
  SAS_FWDSEL_CASE(128, 1)
  SAS_FWDSEL_CASE(128, 2)
  SAS_FWDSEL_CASE(128, 8)
  SAS_FWDSEL_CASE(64, 4)
  SAS_FWDSEL_CASE(64, 1)
  SAS_FWDSEL_CASE(64, 2)
  SAS_FWDSEL_CASE(64, 8)
#undef SAS_FWDSEL_CASE
  return hipErrorInvalidValue;
}

}  // namespace sas
