// Sparse decode: the new token of each sequence attends to its current block
// plus the selected history blocks, with no gate (jaehun.me review, "A
// Concrete Walkthrough", Step 6 / paper Alg. 2; block-sparse attention of the
// blog's 问题动机 section and review "Background", paper Eq. 2).  Without idx
// every history block is attended (dense decode).
//
// Work is split per attended block: a workgroup streams EPW blocks of one
// (sequence, KV head) in 64-key chunks, keeps an online softmax for the G query
// heads of the group and writes a partial (max, sum, acc[D]) per head; a second
// kernel merges the partials by their log-sum-exp.  Every lane loads 16-byte
// pieces: K as four lanes per key (D/4 columns each), V as D/8 lanes per row,
// so a wave load covers whole rows.  The next chunk's K and V are in flight
// while the current one is computed; one barrier per chunk (scores in
// double-buffered LDS; every wave redoes the per-head softmax statistics).
#include "common.h"
#include "internal.h"
#include "mfma.h"
#include "tiles.h"

namespace sas {
namespace {

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
  const int32_t* table;  // null: kc, vc [B, Hkv, L, D]; else pages [num_pages, Hkv, block, D]
};

constexpr int kMaxTopk = 256;

// Resolves attended entry e of (b, g) into a block index, or -1 when the
// entry is empty (invalid / repeated idx entry, beyond the dense range).  ir:
// the (b, g) row of idx, staged in LDS.
__device__ __forceinline__ int entry_block(const DecodeArgs& a, const int32_t* ir, int e, int c) {
  if (a.idx == nullptr) {
    return e <= c ? e : -1;  // blocks 0..c-1, then the current block c
  }
  if (e == a.topk) return c;  // the current block
  if (e > a.topk) return -1;
  const int m = ir[e];
  if (m < 0 || m >= c) return -1;
  for (int e2 = 0; e2 < e; ++e2)
    if (ir[e2] == m) return -1;
  return m;
}

// ONE: every workgroup has exactly one attended entry of at most 64 keys
// (EPW = 1, block <= 64): no next-step prefetch registers, so more
// workgroups fit on a compute unit and all of them are resident at once.
template <typename T, int D, int G, bool ONE>
__global__ __launch_bounds__(256, ONE ? 2 : 1) void decode_partial_kernel(DecodeArgs a) {
  constexpr int DQ = D / 4;                 // K columns per lane (4 lanes per key)
  constexpr int VE = 16 / int(sizeof(T));   // V columns per 16-byte load
  constexpr int LPV = D / VE;               // lanes per V row
  constexpr int VSLOT = 64 / LPV;           // V rows per wave load
  constexpr int VKEYS = kKeys / 4 / VSLOT;  // V rows per lane per block
  constexpr int KLD = DQ / VE;              // 16-byte K loads per lane
  __shared__ __attribute__((aligned(16))) float qsh[G][D];
  __shared__ float sc[2][G][kKeys];
  __shared__ float red[4][G][D];
  __shared__ int32_t ir_sh[kMaxTopk];
  const int part_i = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (a.idx != nullptr)
    for (int i = tid; i < a.topk; i += 256) ir_sh[i] = a.idx[(size_t(b) * a.Hkv + g) * a.topk + i];
  int len = a.cache_len[b];
  len = len > a.L ? a.L : len;
  const int pos = len - 1;
  const int c = len > 0 ? pos / a.block : 0;
  const T* qb = reinterpret_cast<const T*>(a.q) + (size_t(b) * a.Hq + g * G) * D;
  for (int i = tid; i < G * D; i += 256) qsh[i / D][i % D] = to_f32(qb[i]);
  const T* kbase = reinterpret_cast<const T*>(a.kc) + (size_t(b) * a.Hkv + g) * size_t(a.L) * D;
  const T* vbase = reinterpret_cast<const T*>(a.vc) + (size_t(b) * a.Hkv + g) * size_t(a.L) * D;
  const int key = tid >> 2, quarter = tid & 3;     // K phase
  const int vch = lane % LPV, vslot = lane / LPV;  // V phase

  float m_run[G], l_run[G], acc[G][VE];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = kNegInf;
    l_run[h] = 0.f;
#pragma unroll
    for (int i = 0; i < VE; ++i) acc[h][i] = 0.f;
  }

  // The (block, key range) of each of this workgroup's steps; steps of one
  // block beyond 64 keys (block > 64) follow in order.
  auto step_range = [&](int e, int& j0, int& j_end) -> bool {
    const int m = len > 0 ? entry_block(a, ir_sh, e, c) : -1;
    if (m < 0) return false;
    j0 = m * a.block;
    j_end = (m == c) ? pos + 1 : j0 + a.block;
    return true;
  };
  uint4 kr[KLD], vr[VKEYS];
  auto load = [&](int j0, int j_end, uint4* kd, uint4* vd) {
    const int j = j0 + key;
    for (int i = 0; i < KLD; ++i)
      kd[i] = j < j_end ? *reinterpret_cast<const uint4*>(kbase + size_t(j) * D + quarter * DQ + i * VE)
                        : make_uint4(0, 0, 0, 0);
    for (int r = 0; r < VKEYS; ++r) {
      const int jv = j0 + wave * (kKeys / 4) + r * VSLOT + vslot;
      vd[r] = jv < j_end ? *reinterpret_cast<const uint4*>(vbase + size_t(jv) * D + vch * VE)
                         : make_uint4(0, 0, 0, 0);
    }
  };

  // Walk the (entry, 64-key chunk) steps with the next step's loads in flight.
  int e = part_i * a.EPW, e_end = e + a.EPW;
  int j0 = 0, j_end = 0;
  bool have = false;
  __syncthreads();  // ir_sh ready
  while (e < e_end && !(have = step_range(e, j0, j_end))) ++e;
  if (have) load(j0, j_end, kr, vr);
  __syncthreads();  // qsh ready
  int buf = 0;
  while (have) {
    // next step
    int ne = e, nj0 = j0 + kKeys, nj_end = j_end;
    bool nhave = !ONE && nj0 < j_end;
    if (!ONE && !nhave) {
      ++ne;
      while (ne < e_end && !(nhave = step_range(ne, nj0, nj_end))) ++ne;
    }
    uint4 kn[ONE ? 1 : KLD], vn[ONE ? 1 : VKEYS];
    if constexpr (!ONE)
      if (nhave) load(nj0, nj_end, kn, vn);
    // scores of this chunk's 64 keys
    const int j = j0 + key;
    {
      float kf[DQ];
      for (int i = 0; i < KLD; ++i) {
        const T* pv = reinterpret_cast<const T*>(&kr[i]);
        for (int u = 0; u < VE; ++u) kf[i * VE + u] = to_f32(pv[u]);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float sdot = 0.f;
        const float4* qv = reinterpret_cast<const float4*>(&qsh[h][quarter * DQ]);
        for (int i = 0; i < DQ / 4; ++i) {
          const float4 qq = qv[i];
          sdot = fmaf(qq.x, kf[4 * i], sdot);
          sdot = fmaf(qq.y, kf[4 * i + 1], sdot);
          sdot = fmaf(qq.z, kf[4 * i + 2], sdot);
          sdot = fmaf(qq.w, kf[4 * i + 3], sdot);
        }
        sdot += shfl_xor(sdot, 1);
        sdot += shfl_xor(sdot, 2);
        if (quarter == 0) sc[buf][h][key] = j < j_end ? sdot * a.scale : kNegInf;
      }
    }
    __syncthreads();
    // online softmax, every wave for every head (lane = key)
    float p[G], alpha[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float x = sc[buf][h][lane];
      float mx = x;
      for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, shfl_xor(mx, off));
      const float nm = fmaxf(m_run[h], mx);  // finite: every chunk holds a key
      p[h] = exp2_hw((x - nm) * kLog2e);
      float ps = p[h];
      for (int off = 32; off >= 1; off >>= 1) ps += shfl_xor(ps, off);
      alpha[h] = exp2_hw((m_run[h] - nm) * kLog2e);
      l_run[h] = l_run[h] * alpha[h] + ps;
      m_run[h] = nm;
    }
    // values: this lane's VKEYS rows, VE columns each
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < VE; ++i) acc[h][i] *= alpha[h];
    for (int r = 0; r < VKEYS; ++r) {
      const int kk = wave * (kKeys / 4) + r * VSLOT + vslot;
      const T* pv = reinterpret_cast<const T*>(&vr[r]);
      float vf[VE];
      for (int u = 0; u < VE; ++u) vf[u] = to_f32(pv[u]);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float ph = __shfl(p[h], kk, 64);
#pragma unroll
        for (int i = 0; i < VE; ++i) acc[h][i] = fmaf(ph, vf[i], acc[h][i]);
      }
    }
    // advance
    have = nhave;
    e = ne;
    j0 = nj0;
    j_end = nj_end;
    if constexpr (!ONE) {
      for (int i = 0; i < KLD; ++i) kr[i] = kn[i];
      for (int r = 0; r < VKEYS; ++r) vr[r] = vn[r];
    }
    buf ^= 1;
  }
  // Sum the V slots of each wave, then the four waves, and write the partial.
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i = 0; i < VE; ++i)
      for (int off = LPV; off < 64; off <<= 1) acc[h][i] += shfl_xor(acc[h][i], off);
  if (vslot == 0)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < VE; ++i) red[wave][h][vch * VE + i] = acc[h][i];
  __syncthreads();
  float* out = a.part + ((size_t(b) * a.Hkv + g) * a.P + part_i) * G * (D + 2);
  for (int i = tid; i < G * D; i += 256) {
    const int h = i / D, d = i % D;
    out[h * (D + 2) + 2 + d] = red[0][h][d] + red[1][h][d] + red[2][h][d] + red[3][h][d];
  }
  if (tid < G) {
#pragma unroll
    for (int h = 0; h < G; ++h)
      if (h == tid) {
        out[h * (D + 2) + 0] = m_run[h];
        out[h * (D + 2) + 1] = l_run[h];
      }
  }
}

// bf16 on the matrix cores.  Same work split and partial format; per 64-key
// step the G query heads are the rows of one 16-row tile:
//   S = Q K^T   A: the head rows (lane (lq, lr): head lr, 16-byte column
//               chunks lq KS .. lq KS + KS - 1), B: wave w's 16 keys straight
//               from HBM in the same column order (64 contiguous bytes per lane)
//   O += P V    A: P rows from LDS (bf16), B: V read transposed from a
//               row-major LDS tile filled by direct global -> LDS copies; the
//               32 keys of a k step in the order {4 lq + i, 16 + 4 lq + i}.
// Wave w scores keys 16 w .. 16 w + 15 and owns O columns of 16-column tiles
// w DTW .. w DTW + DTW - 1.  Per step: the wave's row maxima (DPP within the
// 16-lane rows) meet in LDS, then the P tile and row sums; the next step's K
// and V are loaded once every wave is past the previous step's P V.  ONE: a
// single step per workgroup (one entry of at most 64 keys), so one V stage
// and no next-step registers: more workgroups fit on a compute unit.
template <int D, int G, bool ONE>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeArgs a) {
  using namespace tiles;
  constexpr int KS = D / 32;            // k steps of S
  constexpr int CH = D / 8;             // 16-byte chunks per V row
  constexpr int DTW = D / 16 / 4;       // O column tiles per wave
  constexpr int VPL = kKeys * CH / 256;  // direct V copies per lane per step
  constexpr int PST = kKeys + 8;        // P row stride (bf16)
  static_assert(G <= 16 && DTW >= 1, "one 16-row tile of heads");
  __shared__ __attribute__((aligned(16))) uint16_t Vs[ONE ? 1 : 2][kKeys * D];
  __shared__ __attribute__((aligned(16))) uint16_t Ps[16 * PST];
  __shared__ __attribute__((aligned(16))) float redm[4][16];
  __shared__ __attribute__((aligned(16))) float reds[4][16];
  __shared__ int32_t ir_sh[kMaxTopk];
  const int part_i = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const bf16_t* qb = reinterpret_cast<const bf16_t*>(a.q) + (size_t(b) * a.Hq + g * G) * D;
  uint4 qa[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qa[ks] = lr < G ? *reinterpret_cast<const uint4*>(qb + lr * D + (lq * KS + ks) * 8) : make_uint4(0, 0, 0, 0);
  if (a.idx != nullptr)
    for (int i = tid; i < a.topk; i += 256) ir_sh[i] = a.idx[(size_t(b) * a.Hkv + g) * a.topk + i];
  int len = a.cache_len[b];
  len = len > a.L ? a.L : len;
  const int pos = len - 1;
  const int c = len > 0 ? pos / a.block : 0;
  // row 0 of block m of this (b, g): contiguous cache or the block's page
  auto block_base = [&](const void* base, int m) -> const bf16_t* {
    const bf16_t* p = reinterpret_cast<const bf16_t*>(base);
    if (a.table) return p + (size_t(a.table[size_t(b) * a.C + m]) * a.Hkv + g) * size_t(a.block) * D;
    return p + ((size_t(b) * a.Hkv + g) * size_t(a.L) + size_t(m) * a.block) * D;
  };

  auto step_range = [&](int e, int& j0, int& j_end) -> bool {
    const int m = len > 0 ? entry_block(a, ir_sh, e, c) : -1;
    if (m < 0) return false;
    j0 = m * a.block;
    j_end = (m == c) ? pos + 1 : j0 + a.block;
    return true;
  };
  // K of the wave's 16 keys into registers, V of the step's 64 keys into LDS
  // stage `st` (rows beyond j_end repeat row j0: finite, and their P is 0).
  // A step never leaves its block: positions j map to row j - m b of block m.
  auto issue = [&](int j0, int j_end, uint4* kd, int st) {
    const int m = j0 / a.block, jb = m * a.block;
    const bf16_t* kb = block_base(a.kc, m) - size_t(jb) * D;
    const bf16_t* vb = block_base(a.vc, m) - size_t(jb) * D;
    const int j = j0 + wave * 16 + lr;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kd[ks] = j < j_end ? *reinterpret_cast<const uint4*>(kb + size_t(j) * D + (lq * KS + ks) * 8)
                         : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int piece = wave * VPL + i;  // 1 KB of the tile
      const int sl = 64 * piece + lane;  // 16-byte slot: row r, stored chunk pc
      const int r = sl / CH, pc = sl % CH;
      const int jr = j0 + r < j_end ? j0 + r : j0;
      dma16_to_lds(vb + size_t(jr) * D + ((pc ^ k_swz<D>(r)) * 8), Vs[st] + piece * 512);
    }
  };

  float m_run[4], l_run[4];
  f32x4 acc[DTW];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m_run[i] = kNegInf;
    l_run[i] = 0.f;
  }
#pragma unroll
  for (int t = 0; t < DTW; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  int e = part_i * a.EPW;
  const int e_end = e + a.EPW;
  int j0 = 0, j_end = 0;
  bool have = false;
  __syncthreads();  // ir_sh
  while (e < e_end && !(have = step_range(e, j0, j_end))) ++e;
  uint4 kf[KS], kn[ONE ? 1 : KS];
  if (have) issue(j0, j_end, kf, 0);
  int st = 0;
  while (have) {
    // the next step (another 64 keys of this block, or the next valid entry)
    int ne = e, nj0 = j0 + kKeys, nj_end = j_end;
    bool nhave = !ONE && nj0 < j_end;
    if (!ONE && !nhave) {
      ++ne;
      while (ne < e_end && !(nhave = step_range(ne, nj0, nj_end))) ++ne;
    }
    wait_vm<VPL>();  // this step's K (its V may still be in flight)
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sacc = mfma16(qa[ks], kf[ks], sacc);
    // lane (lq, lr): heads 4 lq + i, key j0 + 16 wave + lr
    const bool kin = j0 + wave * 16 + lr < j_end;
    float x[4], wm[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = (kin && 4 * lq + i < G) ? sacc[i] * a.scale : kNegInf;
      wm[i] = x[i];
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1)
#pragma unroll
      for (int i = 0; i < 4; ++i) wm[i] = fmaxf(wm[i], __uint_as_float(lanes_xor(__float_as_uint(wm[i]), off, lane)));
    if (lr == 0) *reinterpret_cast<float4*>(&redm[wave][4 * lq]) = make_float4(wm[0], wm[1], wm[2], wm[3]);
    ring_barrier();  // A: every wave is past the previous step's P V
    if constexpr (!ONE)
      if (nhave) issue(nj0, nj_end, kn, st ^ 1);
    float p[4], alpha[4], ws[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float cm = m_run[i];
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) cm = fmaxf(cm, redm[w2][4 * lq + i]);
      const bool live = cm != kNegInf;
      p[i] = live ? exp2_hw((x[i] - cm) * kLog2e) : 0.f;
      alpha[i] = live ? exp2_hw((m_run[i] - cm) * kLog2e) : 1.f;
      m_run[i] = cm;
      ws[i] = p[i];
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1)
#pragma unroll
      for (int i = 0; i < 4; ++i) ws[i] += __uint_as_float(lanes_xor(__float_as_uint(ws[i]), off, lane));
    if (lr == 0) *reinterpret_cast<float4*>(&reds[wave][4 * lq]) = make_float4(ws[0], ws[1], ws[2], ws[3]);
#pragma unroll
    for (int i = 0; i < 4; ++i) Ps[(4 * lq + i) * PST + wave * 16 + lr] = f32_to_bf16(p[i]);
    if (!ONE && nhave) wait_vm<KS + VPL>();  // this step's V has landed
    else wait_vm<0>();
    ring_barrier();  // B: P, the row sums and V are complete
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float cs = reds[0][4 * lq + i] + reds[1][4 * lq + i] + reds[2][4 * lq + i] + reds[3][4 * lq + i];
      l_run[i] = l_run[i] * alpha[i] + cs;
    }
#pragma unroll
    for (int t = 0; t < DTW; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t][i] *= alpha[i];
    const uint16_t* Vt = Vs[st];
    const int trow = 4 * lq + (lr >> 2), tcol = 4 * (lr & 3);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint2 p0 = *reinterpret_cast<const uint2*>(Ps + lr * PST + 32 * kk + 4 * lq);
      const uint2 p1 = *reinterpret_cast<const uint2*>(Ps + lr * PST + 32 * kk + 16 + 4 * lq);
      const uint4 pa = make_uint4(p0.x, p0.y, p1.x, p1.y);
#pragma unroll
      for (int t = 0; t < DTW; ++t) {
        const int ra = 32 * kk + trow, rb = ra + 16;
        const int col = 16 * (wave * DTW + t) + tcol;
        const uint2 v0 = lds_read_tr16(Vt + ra * D + (((col >> 3) ^ k_swz<D>(ra)) << 3) + (col & 7));
        const uint2 v1 = lds_read_tr16(Vt + rb * D + (((col >> 3) ^ k_swz<D>(rb)) << 3) + (col & 7));
        acc[t] = mfma16(pa, make_uint4(v0.x, v0.y, v1.x, v1.y), acc[t]);
      }
    }
    have = nhave;
    e = ne;
    j0 = nj0;
    j_end = nj_end;
    if constexpr (!ONE) {
      st ^= 1;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[ks] = kn[ks];
    }
  }
  // the partial: (max, sum) per head, then the unnormalised P V columns
  float* out = a.part + ((size_t(b) * a.Hkv + g) * a.P + part_i) * G * (D + 2);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * lq + i;
    if (h < G) {
      if (wave == 0 && lr == 0) {
        out[h * (D + 2) + 0] = m_run[i];
        out[h * (D + 2) + 1] = l_run[i];
      }
#pragma unroll
      for (int t = 0; t < DTW; ++t) out[h * (D + 2) + 2 + 16 * (wave * DTW + t) + lr] = acc[t][i];
    }
  }
}

// Merge the P partials of each (b, query head) by log-sum-exp.  Thread d owns
// column d: the first kMergeRegs partials' column values are loaded together
// with the (max, sum) pairs (lane-parallel), so the merge costs one memory
// round trip when P <= kMergeRegs; the weights go through LDS.
constexpr int kMergeMax = 8192;  // partials per (b, g); decode_plan keeps P <= max(8192 / (B Hkv), 2049)
constexpr int kMergeRegs = 48;

template <typename T, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(const float* __restrict__ part,
                                                         T* __restrict__ o,
                                                         float* __restrict__ lse, int Hq, int Hkv,
                                                         int P) {
  __shared__ float w_sh[kMergeMax];
  __shared__ float red[D / 64];
  const int h = blockIdx.x, b = blockIdx.y;
  const int G = Hq / Hkv, g = h / G, hh = h % G;
  const int d = threadIdx.x, lane = d & 63, wave = d >> 6;
  const float* base = part + (size_t(b) * Hkv + g) * P * G * (D + 2) + hh * (D + 2);
  const size_t stride = size_t(G) * (D + 2);
  float x[kMergeRegs];
#pragma unroll
  for (int p = 0; p < kMergeRegs; ++p) x[p] = p < P ? base[p * stride + 2 + d] : 0.f;
  float M = kNegInf;
  for (int p = d; p < P; p += D) M = fmaxf(M, base[p * stride]);
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, shfl_xor(M, off));
  if (lane == 0) red[wave] = M;
  __syncthreads();
  M = red[0];
  for (int w = 1; w < D / 64; ++w) M = fmaxf(M, red[w]);
  __syncthreads();
  float L = 0.f;
  for (int p = d; p < P; p += D) {
    const float mp = base[p * stride];
    const float w = (M == kNegInf || mp == kNegInf) ? 0.f : exp_hw(mp - M);
    w_sh[p] = w;
    L = fmaf(base[p * stride + 1], w, L);
  }
  for (int off = 32; off >= 1; off >>= 1) L += shfl_xor(L, off);
  if (lane == 0) red[wave] = L;
  __syncthreads();
  L = 0.f;
  for (int w = 0; w < D / 64; ++w) L += red[w];
  float acc = 0.f;
#pragma unroll
  for (int p = 0; p < kMergeRegs; ++p)
    if (p < P) acc = fmaf(x[p], w_sh[p], acc);
  for (int p = kMergeRegs; p < P; ++p) acc = fmaf(base[p * stride + 2 + d], w_sh[p], acc);
  const size_t orow = size_t(b) * Hq + h;
  o[orow * D + d] = from_f32<T>(M == kNegInf ? 0.f : acc / L);
  if (lse && d == 0) lse[orow] = (M == kNegInf) ? kNegInf : M + log_hw(L);
}

void decode_plan(int B, int Hkv, int L_max, int block, int topk, int* entries, int* epw, int* P) {
  const int C = L_max / block;
  const int E = topk >= 0 ? topk + 1 : C + 1;  // attended entries per (b, g)
  // One block per workgroup up to 8192 workgroups (the single-step kernel
  // keeps no next-step registers and is about twice as fast per block as the
  // streaming one); beyond that, blocks per workgroup for about 2048.
  const long target = 2048;
  const long groups = long(B) * Hkv;
  int w = long(E) * groups <= 4 * target ? 1 : int((long(E) * groups + target - 1) / target);
  if (w < 1) w = 1;
  *entries = E;
  *epw = w;
  *P = (E + w - 1) / w;
}

template <int D>
hipError_t decode_mfma_t(const DecodeArgs& a, int B, bf16_t* o, float* lse, hipStream_t s) {
  dim3 grid(a.P, a.Hkv, B);
  const bool one = a.EPW == 1 && a.block <= kKeys;
  switch (a.Hq / a.Hkv) {
#define SAS_DECM_G(GG)                                                                                 \
  case GG:                                                                                             \
    if (one)                                                                                           \
      SAS_LAUNCH("decode_partial", (decode_mfma_kernel<D, GG, true>), grid, dim3(256), 0, s, a);       \
    else                                                                                               \
      SAS_LAUNCH("decode_partial", (decode_mfma_kernel<D, GG, false>), grid, dim3(256), 0, s, a);      \
    break;
    SAS_DECM_G(1) SAS_DECM_G(2) SAS_DECM_G(3) SAS_DECM_G(4) SAS_DECM_G(5) SAS_DECM_G(6) SAS_DECM_G(7)
    SAS_DECM_G(8) SAS_DECM_G(9) SAS_DECM_G(10) SAS_DECM_G(11) SAS_DECM_G(12) SAS_DECM_G(13) SAS_DECM_G(14)
    SAS_DECM_G(15) SAS_DECM_G(16)
#undef SAS_DECM_G
    default: return hipErrorInvalidValue;
  }
  SAS_LAUNCH("decode_merge", (decode_merge_kernel<bf16_t, D>), dim3(a.Hq, B), dim3(D), 0, s, a.part, o,
             lse, a.Hq, a.Hkv, a.P);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t decode_t(const DecodeArgs& a0, int B, T* o, float* lse, hipStream_t s) {
  DecodeArgs a = a0;
  dim3 grid(a.P, a.Hkv, B);
  const bool one = a.EPW == 1 && a.block <= kKeys;
  switch (a.Hq / a.Hkv) {
#define SAS_DEC_G(GG)                                                                                 \
  case GG:                                                                                            \
    if (one)                                                                                          \
      SAS_LAUNCH("decode_partial", (decode_partial_kernel<T, D, GG, true>), grid, dim3(256), 0, s, a); \
    else                                                                                              \
      SAS_LAUNCH("decode_partial", (decode_partial_kernel<T, D, GG, false>), grid, dim3(256), 0, s, a); \
    break;
    SAS_DEC_G(1) SAS_DEC_G(2) SAS_DEC_G(3) SAS_DEC_G(4) SAS_DEC_G(5) SAS_DEC_G(6) SAS_DEC_G(7)
    SAS_DEC_G(8) SAS_DEC_G(9) SAS_DEC_G(10) SAS_DEC_G(11) SAS_DEC_G(12) SAS_DEC_G(13) SAS_DEC_G(14)
    SAS_DEC_G(15) SAS_DEC_G(16)
#undef SAS_DEC_G
    default: return hipErrorInvalidValue;
  }
  SAS_LAUNCH("decode_merge", (decode_merge_kernel<T, D>), dim3(a.Hq, B), dim3(D), 0, s, a.part, o, lse,
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
                         hipStream_t s, const int32_t* table) {
  if (B == 0 || Hq == 0) return hipSuccess;
  int E, w, P;
  decode_plan(B, Hkv, L_max, block, idx ? topk : -1, &E, &w, &P);
  if (P > kMergeMax) return hipErrorInvalidValue;  // decode_plan keeps P <= 8192
  DecodeArgs a{q, kc, vc, cache_len, idx, (float*)ws, Hq, Hkv, L_max, D, block,
               idx ? topk : 0, L_max / block, w, P, scale, table};
  if (bf16) {
    if (D == 64) return decode_mfma_t<64>(a, B, (bf16_t*)o, lse, s);
    return decode_mfma_t<128>(a, B, (bf16_t*)o, lse, s);
  }
  if (D == 64) return decode_t<float, 64>(a, B, (float*)o, lse, s);
  return decode_t<float, 128>(a, B, (float*)o, lse, s);
}

}  // namespace sas
