// SAS gated attention forward on the matrix cores (bf16 in, fp32 accumulate).
//
// o = softmax(scale * q K^T + bias) V with bias = 0 on the query's own block
// (causal), log g = s - LSE_s on gated history blocks and -inf elsewhere
// (blog 方法核心; jaehun.me review "New Approach", paper Eq. 9; the gate's log
// form s - LSE(s): review "Why the Four Design Choices Matter").  Tiled with an
// online softmax as in the review's kernel paragraph ("A Concrete Walkthrough").
//
// Layout.  A workgroup owns TOK_WG consecutive query tokens of one KV head and
// all G query heads of that head, 16*NSUB*WAVES rows, split into WAVES waves x
// NSUB subtiles of 16 rows (16/G tokens x G heads).  Everything is transposed so
// a lane owns one query row: S^T = K Q^T and O^T = V^T P^T on
// v_mfma_f32_16x16x32_bf16, so the softmax statistics and the output rescale
// stay lane-local (the four lanes of a row only meet for the row max).  A key
// tile is one block (64 keys).  The gate bias is constant over a block, so it
// enters once per (row, tile).
//
// Tile pipeline.  Tiles stream through an NST-stage ring in LDS filled by
// direct global->LDS loads (global_load_lds_dwordx4), so NST-1 tiles are in
// flight without holding registers.  K is copied from the caller's tensor into
// an XOR-swizzled layout (conflict-free 16-byte MFMA operand reads); V comes
// from a per-block transposed copy in the workspace, written by vt_kernel with
// the keys permuted to the MFMA k order of P^T and the same kind of swizzle.
// Each K stage also holds the rows' selector scores of its tile.
//
// This kernel is the full-scope forward: a workgroup visits every block up
// to its last own block.  Sparse scope is key-major over the selection lists
// (attn_fwd_sel.hip).
#include "common.h"
#include "internal.h"
#include "mfma.h"
#include "tiles.h"

#include <type_traits>

namespace sas {
namespace {

using namespace tiles;


struct FwdArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  const bf16_t* vt;  // workspace: transposed, permuted, swizzled V blocks
  const float* scores;
  bf16_t* o;
  float* lse;
  float* lse_s;
  int Hq, Hkv, N, C, n_tiles, n_pairs, NB;
  float scale;
  int s_stride;  // floats between score rows: C, or 0 (every row reads one shared row)
};

// LSE_s of every query row over its history scores (the gate normaliser):
// one wave per row, a single pass of running (max, sum) per lane, then a
// butterfly merge.  Rows without history get -inf.
__global__ __launch_bounds__(256) void lse_rows_kernel(const float* __restrict__ scores,
                                                       float* __restrict__ lse_s, int N, int C,
                                                       int block, size_t rows) {
  const size_t row = size_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int t = int(row % size_t(N));
  const int c = min(t / block, C);
  const float* srow = scores + row * size_t(C);
  // chunks of 512 history scores: lane holds 4 + 4 consecutive ones, all
  // loaded before the chunk's max and exp sum
  const bool vec = (C & 3) == 0;
  float mx = kNegInf, sm = 0.f;
  for (int m0 = 0; m0 < c; m0 += 512) {
    float x[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int mb = m0 + 256 * h + 4 * lane;
      float4 v = make_float4(kNegInf, kNegInf, kNegInf, kNegInf);
      if (vec && mb + 3 < c) {
        v = *reinterpret_cast<const float4*>(srow + mb);
      } else if (mb < c) {
        v.x = srow[mb];
        v.y = mb + 1 < c ? srow[mb + 1] : kNegInf;
        v.z = mb + 2 < c ? srow[mb + 2] : kNegInf;
        v.w = mb + 3 < c ? srow[mb + 3] : kNegInf;
      }
      x[4 * h + 0] = v.x;
      x[4 * h + 1] = v.y;
      x[4 * h + 2] = v.z;
      x[4 * h + 3] = v.w;
    }
    float cm = x[0];
#pragma unroll
    for (int u = 1; u < 8; ++u) cm = fmaxf(cm, x[u]);
    const float nm = fmaxf(mx, cm);
    if (nm != kNegInf) {
      float add = 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) add += exp2_hw((x[u] - nm) * kLog2e);
      sm = (mx == kNegInf ? 0.f : sm * exp2_hw((mx - nm) * kLog2e)) + add;
      mx = nm;
    }
  }
  for (int off = 32; off >= 1; off >>= 1) {
    const float mo = shfl_xor(mx, off), so = shfl_xor(sm, off);
    const float mn = fmaxf(mx, mo);
    if (mn != kNegInf) sm = sm * exp2_hw((mx - mn) * kLog2e) + so * exp2_hw((mo - mn) * kLog2e);
    mx = mn;
  }
  if (lane == 0) lse_s[row] = c > 0 ? mx + log_hw(sm) : kNegInf;
}

// OUTER: the outer gate (no bias on gated tiles; P scaled by g = exp(s -
// LSE_s) in P V only, the row sum l from the unscaled P).
template <int D, int G, int NSUB, int WAVES, int NST, bool OUTER>
__global__ __launch_bounds__(64 * WAVES, 2) void fwd_mfma_kernel(FwdArgs a) {
  constexpr int NT = 64 * WAVES;
  constexpr int KS = D / 32;    // k-steps of S = K Q^T
  constexpr int MD = D / 16;    // output tiles of O^T
  constexpr int TOK_SUB = 16 / G;
  constexpr int ROWS_WG = 16 * NSUB * WAVES;
  constexpr int TOK_WG = ROWS_WG / G;
  constexpr int CH = D / 8;               // 16-byte chunks per K row
  constexpr int NKL = KT * D * 2 / 1024;  // 1 KB wave loads per K (and per V) tile
  constexpr int LPW = NKL / WAVES;        // per wave, per operand
  constexpr int L = 2 * LPW + 1;          // DMA instructions per wave per tile
  static_assert(NKL % WAVES == 0, "tile loads must split evenly over the waves");
  static_assert(16 * NSUB <= 64, "one score load covers a wave's rows");
  static_assert(NSUB == 1 || NSUB == 2, "one or two subtiles per wave");
  // One array per ring stage: the compiler can then tell a stage being read
  // from the stages the in-flight loads write, and adds no waits of its own.
  // Each K stage also holds the rows' selector scores of its tile (WAVES * 64
  // fp32 after the keys), so a stage is two load targets, not three.
  constexpr int KX = KT * D + WAVES * 64 * 2;
  __shared__ __attribute__((aligned(16))) uint16_t K0[KX], K1[KX], K2[NST > 2 ? KX : 8],
      K3[NST > 3 ? KX : 8];
  __shared__ __attribute__((aligned(16))) uint16_t V0[D * KT], V1[D * KT], V2[NST > 2 ? D * KT : 8],
      V3[NST > 3 ? D * KT : 8];
  __shared__ float lses_sh[ROWS_WG];
  __shared__ int wg_last;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  int tile, pair;
  xcd_order(blockIdx.x, a.n_tiles, a.n_pairs, &tile, &pair);
  const int b = pair / a.Hkv, g = pair % a.Hkv;
  const int N = a.N, C = a.C;
  const int t_wg0 = tile * TOK_WG;

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

  // ---- gate normaliser LSE_s of each row (written by lse_rows_kernel) ---------
  for (int i = tid; i < ROWS_WG; i += NT) {
    const int sg = i >> 4, r = i & 15;
    const int t = t_wg0 + sg * TOK_SUB + r / G;
    lses_sh[i] = t < N ? a.lse_s[(size_t(b) * a.Hq + g * G + r % G) * N + t] : kNegInf;
  }
  __syncthreads();

  if (tid == 0) wg_last = -1;
  __syncthreads();
  {
    int lt = -1;
    for (int s = 0; s < NSUB; ++s) lt = max(lt, sub_live[s] ? c_sub[s] : -1);
    if (lane == 0) atomicMax(&wg_last, lt);
  }
  __syncthreads();
  const int last_tile = wg_last;

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

  auto next_tile = [&](int m) -> int { return (m + 1 <= last_tile) ? m + 1 : -1; };

  // ---- direct global -> LDS tile loads ------------------------------------------
  const bf16_t* kh = a.k + (size_t(b) * a.Hkv + g) * size_t(N) * D;
  const bf16_t* vth = a.vt + (size_t(b) * a.Hkv + g) * size_t(a.NB) * KT * D;
  // this lane's score row: the wave's rows 16s + lr, repeated
  const int srow_i = lane % (16 * NSUB);
  const int s_s = srow_i >> 4, s_lr = srow_i & 15;
  const int s_t = min(t_wg0 + (wave * NSUB + s_s) * TOK_SUB + s_lr / G, N - 1);
  const float* s_base = a.scores + ((size_t(b) * a.Hq + g * G + s_lr % G) * N + s_t) * size_t(a.s_stride);
  auto kst = [&](auto tag) -> uint16_t* {
    constexpr int P = decltype(tag)::value;
    if constexpr (P == 0) return K0;
    else if constexpr (P == 1) return K1;
    else if constexpr (P == 2) return K2;
    else return K3;
  };
  auto vst = [&](auto tag) -> uint16_t* {
    constexpr int P = decltype(tag)::value;
    if constexpr (P == 0) return V0;
    else if constexpr (P == 1) return V1;
    else if constexpr (P == 2) return V2;
    else return V3;
  };
  auto sst = [&](auto tag) -> float* { return reinterpret_cast<float*>(kst(tag) + KT * D); };
  // This lane's 16-byte piece i of a K tile, as an element offset in the tile:
  // tile row r, stored chunk pc, source chunk pc ^ k_swz(r).
  uint32_t k_goff[LPW];
  for (int i = 0; i < LPW; ++i) {
    const int sl = 64 * (wave * LPW + i) + lane;
    const int r = sl / CH, pc = sl % CH;
    k_goff[i] = uint32_t(r * D + (pc ^ k_swz<D>(r)) * 8);
  }
  auto issue = [&](int m, auto tag) {
    uint16_t* kd = kst(tag);
    uint16_t* vd = vst(tag);
    if (m * KT + KT <= N) {
      // whole tile: uniform tile base plus this lane's offset inside the tile
      const bf16_t* kt = kh + size_t(m) * KT * D;
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        uint32_t off = k_goff[i];
        asm volatile("" : "+v"(off));
        __builtin_amdgcn_global_load_lds(kt + off, (lds_ptr_t)(kd + (wave * LPW + i) * 512), 16, 0, 0);
      }
    } else {
      // tail tile: keys past N repeat key N-1 (their logits are masked)
      for (int i = 0; i < LPW; ++i) {
        const int j = wave * LPW + i;  // 1 KB piece of the tile
        const int sl = 64 * j + lane;  // 16-byte slot
        const int r = sl / CH, pc = sl % CH;
        const int key = min(m * KT + r, N - 1);
        const int c = pc ^ k_swz<D>(r);
        __builtin_amdgcn_global_load_lds(kh + size_t(key) * D + c * 8, (lds_ptr_t)(kd + j * 512), 16, 0, 0);
      }
    }
    for (int i = 0; i < LPW; ++i) {
      const int j = wave * LPW + i;
      __builtin_amdgcn_global_load_lds(vth + size_t(m) * KT * D + (64 * j + lane) * 8,
                                       (lds_ptr_t)(vd + j * 512), 16, 0, 0);
    }
    __builtin_amdgcn_global_load_lds(s_base + min(m, C - 1), (lds_ptr_t)(sst(tag) + wave * 64), 4, 0, 0);
  };
  auto wait_tile = [&](int after) {
    // wait until at most `after` later tiles' loads are still outstanding
    switch (after) {
      case 0: wait_vm<0>(); break;
      case 1: wait_vm<L>(); break;
      case 2: wait_vm<2 * L>(); break;
      default: wait_vm<3 * L>(); break;
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
  // MFMA operand reads.  K row key = 16 mt + lr holds chunk (4 ks + lq) at
  // chunk (4 ks + lq) ^ sw with sw = k_swz(key) (a function of lr alone); the
  // XOR splits into a lane part (low two bits) and (ks ^ (sw >> 2)) * 4.
  // V^T row d = 16 md + lr likewise with sw = vt_swz(lr).
  const int ksw = k_swz<D>(lr), vsw = vt_swz(lr);
  const uint32_t k_base = lr * D + ((lq ^ (ksw & 3)) * 8), k_xor = (ksw >> 2) * 32;
  const uint32_t v_base = lr * KT + ((lq ^ (vsw & 3)) * 8), v_xor = (vsw >> 2) * 32;

  int tq[NST];
  tq[0] = next_tile(-1);
  for (int i = 1; i < NST; ++i) tq[i] = tq[i - 1] >= 0 ? next_tile(tq[i - 1]) : -1;
  if (tq[0] >= 0) issue(tq[0], std::integral_constant<int, 0>{});
  if (NST > 2 && tq[1] >= 0) issue(tq[1], std::integral_constant<int, 1>{});
  if (NST > 3 && tq[2] >= 0) issue(tq[2], std::integral_constant<int, 2>{});

  // One pipeline step on ring stage P; returns false once the tiles are done.
  // One pipeline step on ring stage P for tile tq[0] >= 0.  MK: the tile may be
  // a subtile's own block (keys above the row are masked).
  auto step = [&](auto tag, auto mkt) {
    constexpr int P = decltype(tag)::value;
    constexpr bool MK = decltype(mkt)::value;
    const int m = tq[0];
    int after = 0;
    for (int i = 1; i < NST - 1; ++i) after += tq[i] >= 0;
    wait_tile(after);
    ring_barrier();
    if (tq[NST - 1] >= 0) issue(tq[NST - 1], std::integral_constant<int, (P + NST - 1) % NST>{});
    const uint16_t* Ks = kst(tag);
    const uint16_t* Vs = vst(tag);
    const float* Ss = sst(tag);
    // Which subtiles take part (a wave-uniform bit mask), and each lane's bias
    // for its row (base 2; -inf where the row does not attend the tile).
    int nmask = 0;
    float bias2[NSUB], gsc[NSUB];
    for (int s = 0; s < NSUB; ++s) {
      const bool own = (m == c_sub[s]);
      const bool hist = (m < c_sub[s]);
      bool sel = false;
      float bsel = kNegInf;
      if (hist && row_t[s] < N) {
        sel = true;
        bsel = (Ss[wave * 64 + 16 * s + lr] - lses[s]) * kLog2e;
      }
      const bool nd = sub_live[s] && (own || (hist && __ballot(sel) != 0ull));
      nmask |= int(nd) << s;
      bias2[s] = own ? 0.f : (sel ? (OUTER ? 0.f : bsel) : kNegInf);
      gsc[s] = OUTER && !own && sel ? exp2_hw(bsel) : 1.f;
    }
    nmask = __builtin_amdgcn_readfirstlane(nmask);

    // Straight-line compute of the subtiles in SM.
    auto compute = [&](auto smt) {
      constexpr int SM = decltype(smt)::value;
      f32x4 sacc[NSUB][4];
#pragma unroll
      for (int s = 0; s < NSUB; ++s)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) sacc[s][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      // S^T = K Q^T
      // Operand offsets: a lane base plus an XOR term per k step (one v_xad at
      // the use); opaque, so no register is kept per (stage, step).
      uint32_t kb = k_base, kx = k_xor, vb = v_base, vx = v_xor;
      asm volatile("" : "+v"(kb), "+v"(kx), "+v"(vb), "+v"(vx));
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const uint4 kf = *reinterpret_cast<const uint4*>(Ks + mt * 16 * D + (((ks * 32) ^ kx) + kb));
#pragma unroll
          for (int s = 0; s < NSUB; ++s)
            if ((SM >> s) & 1) sacc[s][mt] = mfma16(kf, qf[s][ks], sacc[s][mt]);
        }
      }
      // Online softmax (base 2).  The bias is constant over the tile, so the
      // row max is scale * max(S) + bias.  The running max moves only when it
      // grows by more than 2^8, which bounds every P by 256 and skips most
      // rescales of the output accumulators.
      uint4 pf[NSUB][2];
#pragma unroll
      for (int s = 0; s < NSUB; ++s) {
        if (!((SM >> s) & 1)) continue;
        if (MK) {
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (m * KT + 16 * mt + 4 * lq + i > row_t[s]) sacc[s][mt][i] = kNegInf;
        }
        float mr = kNegInf;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          mr = fmaxf(fmaxf(mr, fmaxf(sacc[s][mt][0], sacc[s][mt][1])), fmaxf(sacc[s][mt][2], sacc[s][mt][3]));
        mr = max_xrows(mr);
        const float mx = mr * c1 + bias2[s];
        const bool upd = mx > mrow[s] + 8.f;
        if (__any(upd)) {
          const float alpha = upd ? exp2_hw(mrow[s] - mx) : 1.f;
          mrow[s] = upd ? mx : mrow[s];
          lpart[s] *= alpha;
#pragma unroll
          for (int md = 0; md < MD; ++md) oacc[s][md] *= alpha;
        }
        const float off = bias2[s] - (mrow[s] == kNegInf ? 0.f : mrow[s]);
        float ps = 0.f;
        float z[4][4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            z[mt][i] = exp2_hw(fmaf(sacc[s][mt][i], c1, off));
            ps += z[mt][i];
          }
        lpart[s] += ps;
        if constexpr (OUTER) {
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) z[mt][i] *= gsc[s];  // the gate scales P V only
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          pf[s][kk].x = pack_bf16(z[2 * kk][0], z[2 * kk][1]);
          pf[s][kk].y = pack_bf16(z[2 * kk][2], z[2 * kk][3]);
          pf[s][kk].z = pack_bf16(z[2 * kk + 1][0], z[2 * kk + 1][1]);
          pf[s][kk].w = pack_bf16(z[2 * kk + 1][2], z[2 * kk + 1][3]);
        }
      }
      // Keep the V^T operand reads below the softmax (register pressure).
      
      // O^T += V^T P^T
#pragma unroll
      for (int md = 0; md < MD; ++md) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const uint4 vf = *reinterpret_cast<const uint4*>(Vs + md * 16 * KT + (((kk * 32) ^ vx) + vb));
#pragma unroll
          for (int s = 0; s < NSUB; ++s)
            if ((SM >> s) & 1) oacc[s][md] = mfma16(vf, pf[s][kk], oacc[s][md]);
        }
      }
    };
    if (nmask) {
      // every subtile of the wave (a subtile without the tile has bias -inf
      // on all rows and adds nothing)
      compute(std::integral_constant<int, (1 << NSUB) - 1>{});
    }
    for (int i = 0; i < NST - 1; ++i) tq[i] = tq[i + 1];
    tq[NST - 1] = tq[NST - 2] >= 0 ? next_tile(tq[NST - 2]) : -1;
  };
  // History tiles of every subtile (no masking), then the workgroup's own
  // blocks (masked), continuing the ring where the first loop stopped.
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
      step(std::integral_constant<int, 2>{}, Unmasked{});
    }
    if constexpr (NST > 3) {
      if (tq[0] < 0 || tq[0] >= c_first) { ph = 3; break; }
      step(std::integral_constant<int, 3>{}, Unmasked{});
    }
  }
  while (tq[0] >= 0) {
    if (ph == 0) step(std::integral_constant<int, 0>{}, Masked{});
    else if (ph == 1) step(std::integral_constant<int, 1>{}, Masked{});
    else if (NST > 2 && ph == 2) step(std::integral_constant<int, (NST > 2 ? 2 : 0)>{}, Masked{});
    else if (NST > 3) step(std::integral_constant<int, (NST > 3 ? 3 : 0)>{}, Masked{});
    ph = ph + 1 == NST ? 0 : ph + 1;
  }

  // ---- epilogue ---------------------------------------------------------------
  for (int s = 0; s < NSUB; ++s) {
    const float l = sum_xrows(lpart[s]);
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

template <int D, int G>
hipError_t fwd_mfma_t(const FwdArgs& a0, int B, int norm, bool outer, hipStream_t stream) {
  constexpr int NSUB = 2;
  constexpr int WAVES = 8;
  constexpr int NST = 2;
  constexpr int TOK_WG = 16 * NSUB * WAVES / G;
  FwdArgs a = a0;
  a.n_tiles = (a.N + TOK_WG - 1) / TOK_WG;
  a.n_pairs = B * a.Hkv;
  const size_t rows = size_t(B) * a.Hq * a.N;
  if (norm == 1)
    SAS_LAUNCH("lse_rows", lse_rows_kernel, dim3(unsigned((rows + 3) / 4)), dim3(256), 0, stream, a.scores,
               a.lse_s, a.N, a.C, KT, rows);
  SAS_LAUNCH("vt", (vt_kernel<D>), dim3(a.NB, a.Hkv, B), dim3(256), 0, stream, a.v,
                     const_cast<bf16_t*>(a.vt), a.Hkv, a.N, a.NB);
  if (outer)
    SAS_LAUNCH("fwd_mfma", (fwd_mfma_kernel<D, G, NSUB, WAVES, NST, true>), dim3(a.n_tiles * a.n_pairs),
               dim3(64 * WAVES), 0, stream, a);
  else
    SAS_LAUNCH("fwd_mfma", (fwd_mfma_kernel<D, G, NSUB, WAVES, NST, false>), dim3(a.n_tiles * a.n_pairs),
               dim3(64 * WAVES), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

// Shapes the matrix-core forward covers: bf16, block 64, D 64/128, G in
// {1,2,4,8}, at least one complete block; sparse scope (key-major over the
// selection lists) packs a token into 23 bits of a list entry and a block
// into 16 bits of a work item.
// LSE_s of every row on its own (any dtype: it reads only the fp32 scores).
hipError_t launch_lse_rows(const float* scores, float* lse_s, const Dims& d, hipStream_t s) {
  const size_t rows = size_t(d.B) * d.Hq * d.N;
  if (rows == 0) return hipSuccess;
  SAS_LAUNCH("lse_rows", lse_rows_kernel, dim3(unsigned((rows + 3) / 4)), dim3(256), 0, s, scores, lse_s, d.N,
             d.C, d.block, rows);
  return hipGetLastError();
}

bool fwd_mfma_supported(const Dims& d, int topk, bool sparse) {
  if (d.block != KT || (d.D != 64 && d.D != 128)) return false;
  if (d.C < 1) return false;
  const int G = d.G();
  if (G != 1 && G != 2 && G != 4 && G != 8) return false;
  if (sparse && (d.N > (1 << 22) || topk > 256)) return false;
  return true;
}

size_t fwd_mfma_workspace(const Dims& d, int topk, bool sparse) {
  if (sparse) return fwd_sel_workspace(d, topk);
  const int NB = (d.N + KT - 1) / KT;
  return align_up(size_t(d.B) * d.Hkv * NB * KT * d.D * sizeof(bf16_t));
}

hipError_t launch_fwd_mfma(const void* q, const void* k, const void* v, const float* scores,
                           const int32_t* idx, void* o, float* lse, float* lse_s, const Dims& d,
                           int topk, float scale, int norm, bool outer, void* ws, hipStream_t s, void* ctx,
                           const float* gates) {
  FwdArgs a{(const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, (const bf16_t*)ws, scores,
            (bf16_t*)o, lse, lse_s, d.Hq, d.Hkv, d.N, d.C, 0, 0, (d.N + KT - 1) / KT, scale, d.C};
  const int G = d.G();
  if (idx != nullptr) {
    // sparse scope: the gate normaliser (norm 1: the softmax gate's, computed
    // here; 2: given; 0: lse_s already holds 0), then the key-major forward
    const size_t rows = size_t(d.B) * d.Hq * d.N;
    if (norm == 1)
      SAS_LAUNCH("lse_rows", lse_rows_kernel, dim3(unsigned((rows + 3) / 4)), dim3(256), 0, s, scores, lse_s,
                 d.N, d.C, KT, rows);
    return launch_fwd_sel(q, k, v, scores, idx, o, lse, lse_s, d, topk, scale, outer, ws, s, ctx, gates);
  }
#define SAS_FWD_CASE(DD, GG) \
  if (d.D == DD && G == GG) return fwd_mfma_t<DD, GG>(a, d.B, norm, outer, s);
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

// Full-scope forward whose history rows all read one shared row of scores
// (score row stride 0): with that row and lse_s zero, the raw gate's bias is
// 0 on every history block, i.e. plain causal attention (prefill).  ws: the
// V^T blocks (fwd_mfma_workspace).
hipError_t launch_fwd_mfma_shared_row(const void* q, const void* k, const void* v, const float* score_row,
                                      const float* lse_s, void* o, float* lse, const Dims& d, float scale,
                                      void* ws, hipStream_t s) {
  FwdArgs a{(const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)v, (const bf16_t*)ws, score_row,
            (bf16_t*)o, lse, const_cast<float*>(lse_s), d.Hq, d.Hkv, d.N, d.C, 0, 0, (d.N + KT - 1) / KT, scale, 0};
  const int G = d.G();
#define SAS_FWD_CASE(DD, GG) \
  if (d.D == DD && G == GG) return fwd_mfma_t<DD, GG>(a, d.B, false, false, s);
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
