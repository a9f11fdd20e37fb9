// Backward of the mean-pool selector: the last link of the gradient path from
// the output through the gate to the selector (jaehun.me review, "A Concrete
// Walkthrough", Step 5; pooling-based block summaries, review "Our
// Perspective").  The score is s[t,m] = scale q_t . K̄_m for history blocks
// m < c(t) = t / b, with K̄_m the mean of complete block m of K.  For an
// upstream ds:
//   dq[t]   = scale sum_{m < c(t)} ds[t,m] K̄_m
//   dK̄_m    = scale sum_{h of the group} sum_{t: m < c(t)} ds[h,t,m] q[h,t]
//   dk[j]   = dK̄_{j / b} / b for j in a complete block, 0 in the tail.
//
// bf16 runs on the matrix cores (ds rounded to bf16 as an operand, fp32
// accumulation); fp32 runs plain per-element loops.
//   dq:      a workgroup owns 64 query rows of one head (16 per wave, all D
//            columns) and walks the history blocks in chunks of 64: A = the
//            rows' ds (fp32 -> bf16 in registers, keys of a 32-wide k step in
//            the order {4 lq + i, 16 + 4 lq + i}), B = K̄ of the chunk, staged
//            row-major in LDS and read transposed.
//   dK̄:      a workgroup owns 64 blocks x D of one KV head and one chunk of
//            tokens (all heads of the group); both operands run over tokens,
//            so the ds tile (bf16) and the q tile sit row-major in LDS and
//            both are read transposed.  Each token chunk writes an fp32
//            partial; a second kernel sums the partials in chunk order (no
//            atomics) and spreads dK̄ over the tokens of each block.
#include "common.h"
#include "internal.h"
#include "mfma.h"
#include "tiles.h"

#include <type_traits>

namespace sas {
namespace {

constexpr int kSelTok = 1024;  // tokens per dK̄ chunk (bf16 path)

struct SelArgs {
  const void* q;
  const void* kbar;
  const float* ds;
  void* dq;
  void* dk;
  float* dkbar;     // optional
  float* part;      // workspace [nch, B, Hkv, C, D]
  int B, Hq, Hkv, N, D, block, C, nch, tch;
  float scale;
  int accumulate;
};

// Whether token chunk ch holds a query whose history reaches block m0.
__device__ __forceinline__ bool chunk_active(int ch, int tch, int N, int block, int m0) {
  const int t_last = min(N, (ch + 1) * tch) - 1;
  return ch * tch < N && t_last / block > m0;
}

template <typename T>
__device__ __forceinline__ T add_out(const T* p, float v, int accumulate) {
  return from_f32<T>(accumulate ? to_f32(*p) + v : v);
}

// ------------------------------------------------------------ dq (bf16) ----
template <int D>
__global__ __launch_bounds__(256) void sel_dq_kernel(SelArgs a) {
  using namespace tiles;
  constexpr int ND = D / 16;
  constexpr int CH = D / 8;
  constexpr int VPL = 64 * CH / 256;  // direct K̄ copies per lane per chunk
  __shared__ __attribute__((aligned(16))) uint16_t Ks[64 * D];
  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int G = a.Hq / a.Hkv, g = h / G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int N = a.N, C = a.C;
  const int t = tile * 64 + wave * 16 + lr;  // this lane's A row
  const int c_t = t < N ? min(t / a.block, C) : 0;
  const int c_max = min((min(N, tile * 64 + 64) - 1) / a.block, C);
  const float* dsr = a.ds + ((size_t(b) * a.Hq + h) * N + (t < N ? t : 0)) * size_t(C);
  const bool vec4 = (C & 3) == 0;  // ds rows start 16-byte aligned
  const bf16_t* kb = reinterpret_cast<const bf16_t*>(a.kbar) + (size_t(b) * a.Hkv + g) * size_t(C) * D;
  f32x4 acc[ND];
#pragma unroll
  for (int nd = 0; nd < ND; ++nd) acc[nd] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int trow = 4 * lq + (lr >> 2), tcol = 4 * (lr & 3);
  for (int m0 = 0; m0 < c_max; m0 += 64) {
    __syncthreads();  // every wave is done with the previous chunk
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int piece = wave * VPL + i;
      const int sl = 64 * piece + lane;
      const int r = sl / CH, pc = sl % CH;
      const int m = m0 + r < C ? m0 + r : C - 1;  // rows past C: a real row, weight 0
      dma16_to_lds(kb + size_t(m) * D + ((pc ^ k_swz<D>(r)) * 8), Ks + piece * 512);
    }
    // this lane's ds for the chunk: keys m0 + 32 kk + {4 lq + i, 16 + 4 lq + i}
    uint4 da[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      float v[8];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int mb = m0 + 32 * kk + 16 * half + 4 * lq;
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (vec4 && mb + 3 < c_t) {
          x = *reinterpret_cast<const float4*>(dsr + mb);
        } else if (mb < c_t) {
          x.x = dsr[mb];
          x.y = mb + 1 < c_t ? dsr[mb + 1] : 0.f;
          x.z = mb + 2 < c_t ? dsr[mb + 2] : 0.f;
          x.w = mb + 3 < c_t ? dsr[mb + 3] : 0.f;
        }
        v[4 * half + 0] = x.x;
        v[4 * half + 1] = x.y;
        v[4 * half + 2] = x.z;
        v[4 * half + 3] = x.w;
      }
      da[kk] = make_uint4(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]),
                          pack_bf16(v[6], v[7]));
    }
    wait_vm<0>();
    __syncthreads();  // K̄ chunk in LDS
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ra = 32 * kk + trow, rb = ra + 16;
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) {
        const int col = 16 * nd + tcol;
        const uint2 k0 = lds_read_tr16(Ks + ra * D + (((col >> 3) ^ k_swz<D>(ra)) << 3) + (col & 7));
        const uint2 k1 = lds_read_tr16(Ks + rb * D + (((col >> 3) ^ k_swz<D>(rb)) << 3) + (col & 7));
        acc[nd] = mfma16(da[kk], make_uint4(k0.x, k0.y, k1.x, k1.y), acc[nd]);
      }
    }
  }
  // lane (lq, lr): rows tile 64 + 16 wave + 4 lq + i, column 16 nd + lr
  bf16_t* dq = reinterpret_cast<bf16_t*>(a.dq) + (size_t(b) * a.Hq + h) * size_t(N) * D;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tr = tile * 64 + wave * 16 + 4 * lq + i;
    if (tr >= N) continue;
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) {
      bf16_t* p = dq + size_t(tr) * D + 16 * nd + lr;
      *p = add_out<bf16_t>(p, acc[nd][i] * a.scale, a.accumulate);
    }
  }
}

// ----------------------------------------------------------- dK̄ (bf16) ----
// Workgroup: MT = 128 blocks of one KV head and one token chunk; wave w owns
// blocks m0 + 32 w .. m0 + 32 w + 31 (two 16-block tiles) x all D columns.
// Steps of 64 tokens of one head run through two LDS stages: while a step's
// products run, the next step's q rows (direct global -> LDS copies) and ds
// values (registers, bf16 into LDS after the barrier) are in flight.
template <int D>
__global__ __launch_bounds__(256, 2) void sel_dkbar_kernel(SelArgs a) {
  using namespace tiles;
  constexpr int ND = D / 16;
  constexpr int CH = D / 8;
  constexpr int QPL = 64 * CH / 256;  // direct q copies per lane per step
  constexpr int MT = 128;             // blocks per workgroup
  constexpr int DST = MT;             // ds tile row (bf16)
  constexpr int SPT = 32;             // ds values per thread per step
  __shared__ __attribute__((aligned(16))) uint16_t Q0[64 * D], Q1[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t S0[64 * DST], S1[64 * DST];
  const int ch = blockIdx.x, mtile = blockIdx.y, bg = blockIdx.z;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int N = a.N, C = a.C;
  const int m0 = mtile * MT;
  if (!chunk_active(ch, a.tch, N, a.block, m0)) return;  // nothing of this chunk reaches the tile
  // first token whose history holds block m0, and the chunk's token range
  const int t_begin = max(ch * a.tch, (m0 + 1) * a.block);
  const int t_end = min(N, (ch + 1) * a.tch);
  const int nt = (t_end - t_begin + 63) / 64;  // steps per head
  const int nsteps = G * nt;
  const bool vec4 = (C & 3) == 0;
  f32x4 acc[2][ND];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) acc[u][nd] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int trow = 4 * lq + (lr >> 2), tcol = 4 * (lr & 3);
  // ds staging: thread -> row sr (of 64), columns sc0 .. sc0 + 31
  const int sr = tid >> 2, sc0 = (tid & 3) * SPT;
  float v[SPT];
  auto load_ds = [&](int s) {
    const int h = g * G + s / nt, t0 = t_begin + (s % nt) * 64;
    const int tt = t0 + sr;
    const int ct = tt < t_end ? min(tt / a.block, C) : 0;  // row tt's history: m < ct
    const float* src = a.ds + ((size_t(b) * a.Hq + h) * N + (tt < t_end ? tt : t0)) * size_t(C) + m0 + sc0;
#pragma unroll
    for (int j = 0; j < SPT; j += 4) {
      const int m = m0 + sc0 + j;
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (vec4 && m + 3 < ct) {
        x = *reinterpret_cast<const float4*>(src + j);
      } else if (m < ct) {
        x.x = src[j];
        x.y = m + 1 < ct ? src[j + 1] : 0.f;
        x.z = m + 2 < ct ? src[j + 2] : 0.f;
        x.w = m + 3 < ct ? src[j + 3] : 0.f;
      }
      v[j] = x.x;
      v[j + 1] = x.y;
      v[j + 2] = x.z;
      v[j + 3] = x.w;
    }
  };
  auto stq = [&](auto tag) -> uint16_t* {
    if constexpr (decltype(tag)::value == 0) return Q0;
    else return Q1;
  };
  auto sts = [&](auto tag) -> uint16_t* {
    if constexpr (decltype(tag)::value == 0) return S0;
    else return S1;
  };
  auto issue_q = [&](auto tag, int s) {
    const int h = g * G + s / nt, t0 = t_begin + (s % nt) * 64;
    const bf16_t* qh = reinterpret_cast<const bf16_t*>(a.q) + (size_t(b) * a.Hq + h) * size_t(N) * D;
    uint16_t* dst = stq(tag);
#pragma unroll
    for (int i = 0; i < QPL; ++i) {
      const int piece = wave * QPL + i;
      const int sl = 64 * piece + lane;
      const int r = sl / CH, pc = sl % CH;
      const int tq = t0 + r < t_end ? t0 + r : t0;  // rows past the range: a real row, weight 0
      dma16_to_lds(qh + size_t(tq) * D + ((pc ^ k_swz<D>(r)) * 8), dst + piece * 512);
    }
  };
  auto store_ds = [&](auto tag) {
    uint16_t* dst = sts(tag);
#pragma unroll
    for (int cc = 0; cc < SPT / 8; ++cc) {
      const int c8 = (sc0 >> 3) + cc;
      *reinterpret_cast<uint4*>(dst + sr * DST + ((c8 ^ (sr & 15)) << 3)) =
          make_uint4(pack_bf16(v[8 * cc + 0], v[8 * cc + 1]), pack_bf16(v[8 * cc + 2], v[8 * cc + 3]),
                     pack_bf16(v[8 * cc + 4], v[8 * cc + 5]), pack_bf16(v[8 * cc + 6], v[8 * cc + 7]));
    }
  };
  auto compute = [&](auto tag) {
    const uint16_t* Qs = stq(tag);
    const uint16_t* Ds = sts(tag);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int ra = 32 * kk + trow, rb = ra + 16;
      uint4 dsa[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int dcol = 32 * wave + 16 * u + tcol;
        const uint2 d0 = lds_read_tr16(Ds + ra * DST + (((dcol >> 3) ^ (ra & 15)) << 3) + (dcol & 7));
        const uint2 d1 = lds_read_tr16(Ds + rb * DST + (((dcol >> 3) ^ (rb & 15)) << 3) + (dcol & 7));
        dsa[u] = make_uint4(d0.x, d0.y, d1.x, d1.y);
      }
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) {
        const int col = 16 * nd + tcol;
        const uint2 q0 = lds_read_tr16(Qs + ra * D + (((col >> 3) ^ k_swz<D>(ra)) << 3) + (col & 7));
        const uint2 q1 = lds_read_tr16(Qs + rb * D + (((col >> 3) ^ k_swz<D>(rb)) << 3) + (col & 7));
        const uint4 qb = make_uint4(q0.x, q0.y, q1.x, q1.y);
        acc[0][nd] = mfma16(dsa[0], qb, acc[0][nd]);
        acc[1][nd] = mfma16(dsa[1], qb, acc[1][nd]);
      }
    }
  };
  using T0 = std::integral_constant<int, 0>;
  using T1 = std::integral_constant<int, 1>;
  // one step on stage `tag`: its ds into LDS, barrier, the next step's loads
  // into the other stage, the products
  auto step = [&](auto tag, int s) {
    using Tn = std::integral_constant<int, decltype(tag)::value ^ 1>;
    store_ds(tag);
    wait_vm<0>();
    __syncthreads();  // this stage complete; every wave is done with the other
    if (s + 1 < nsteps) {
      issue_q(Tn{}, s + 1);
      load_ds(s + 1);
    }
    compute(tag);
  };
  issue_q(T0{}, 0);
  load_ds(0);
  int s = 0;
  for (; s + 1 < nsteps; s += 2) {
    step(T0{}, s);
    step(T1{}, s + 1);
  }
  if (s < nsteps) step(T0{}, s);
  // lane (lq, lr): block m0 + 32 wave + 16 u + 4 lq + i, column 16 nd + lr
  float* out = a.part + ((size_t(ch) * a.B * a.Hkv + bg) * C) * D;
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + wave * 32 + 16 * u + 4 * lq + i;
      if (m >= C) continue;
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) out[size_t(m) * D + 16 * nd + lr] = acc[u][nd][i] * a.scale;
    }
}

// ------------------------------------------------------ fp32 (per element) --
template <int D>
__global__ __launch_bounds__(D) void sel_dq_f32_kernel(SelArgs a) {
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z, d = threadIdx.x;
  const int G = a.Hq / a.Hkv, g = h / G;
  const int C = a.C, c = min(t / a.block, C);
  const float* dsr = a.ds + ((size_t(b) * a.Hq + h) * a.N + t) * size_t(C);
  const float* kb = reinterpret_cast<const float*>(a.kbar) + (size_t(b) * a.Hkv + g) * size_t(C) * D;
  float acc = 0.f;
  for (int m = 0; m < c; ++m) acc = fmaf(dsr[m], kb[size_t(m) * D + d], acc);
  float* p = reinterpret_cast<float*>(a.dq) + ((size_t(b) * a.Hq + h) * a.N + t) * D + d;
  *p = (a.accumulate ? *p : 0.f) + acc * a.scale;
}

// one partial (chunk 0 covers every token)
template <int D>
__global__ __launch_bounds__(D) void sel_dkbar_f32_kernel(SelArgs a) {
  const int m = blockIdx.x, g = blockIdx.y, b = blockIdx.z, d = threadIdx.x;
  const int G = a.Hq / a.Hkv, C = a.C, N = a.N;
  float acc = 0.f;
  for (int hh = 0; hh < G; ++hh) {
    const int h = g * G + hh;
    const float* q = reinterpret_cast<const float*>(a.q) + (size_t(b) * a.Hq + h) * size_t(N) * D;
    const float* ds = a.ds + (size_t(b) * a.Hq + h) * size_t(N) * C;
    for (int t = (m + 1) * a.block; t < N; ++t) acc = fmaf(ds[size_t(t) * C + m], q[size_t(t) * D + d], acc);
  }
  a.part[((size_t(b) * a.Hkv + g) * C + m) * D + d] = acc * a.scale;
}

// --------------------------------------------- dK̄ = sum of partials; dk ----
// Workgroup (m, g, b), thread d: the active chunks' partials in chunk order;
// block m's tokens get dK̄ / b.  Workgroup m == C clears (or keeps) the tail.
template <typename T, int D>
__global__ __launch_bounds__(D) void sel_pool_bwd_kernel(SelArgs a) {
  const int m = blockIdx.x, g = blockIdx.y, b = blockIdx.z, d = threadIdx.x;
  const int C = a.C, N = a.N;
  T* dk = reinterpret_cast<T*>(a.dk) + (size_t(b) * a.Hkv + g) * size_t(N) * D;
  if (m == C) {
    if (!a.accumulate)
      for (int j = C * a.block; j < N; ++j) dk[size_t(j) * D + d] = from_f32<T>(0.f);
    return;
  }
  const int bg = b * a.Hkv + g;
  const int m0 = (m / 128) * 128;  // the dK̄ kernel's block tile
  float s = 0.f;
  for (int ch = 0; ch < a.nch; ++ch)
    if (chunk_active(ch, a.tch, N, a.block, m0))
      s += a.part[((size_t(ch) * a.B * a.Hkv + bg) * C + m) * D + d];
  if (a.dkbar) a.dkbar[(size_t(bg) * C + m) * D + d] = s;
  const float v = s / float(a.block);
  for (int j = m * a.block; j < (m + 1) * a.block; ++j) {
    T* p = dk + size_t(j) * D + d;
    *p = add_out<T>(p, v, a.accumulate);
  }
}

template <int D>
hipError_t selector_bwd_t(SelArgs a, bool bf16, hipStream_t s) {
  if (bf16) {
    SAS_LAUNCH("sel_dq", (sel_dq_kernel<D>), dim3((a.N + 63) / 64, a.Hq, a.B), dim3(256), 0, s, a);
    if (a.C > 0)
      SAS_LAUNCH("sel_dkbar", (sel_dkbar_kernel<D>), dim3(a.nch, (a.C + 127) / 128, a.B * a.Hkv), dim3(256), 0, s, a);
    SAS_LAUNCH("sel_pool_bwd", (sel_pool_bwd_kernel<bf16_t, D>), dim3(a.C + 1, a.Hkv, a.B), dim3(D), 0, s, a);
  } else {
    SAS_LAUNCH("sel_dq", (sel_dq_f32_kernel<D>), dim3(a.N, a.Hq, a.B), dim3(D), 0, s, a);
    if (a.C > 0)
      SAS_LAUNCH("sel_dkbar", (sel_dkbar_f32_kernel<D>), dim3(a.C, a.Hkv, a.B), dim3(D), 0, s, a);
    SAS_LAUNCH("sel_pool_bwd", (sel_pool_bwd_kernel<float, D>), dim3(a.C + 1, a.Hkv, a.B), dim3(D), 0, s, a);
  }
  return hipGetLastError();
}

void sel_plan(int N, bool bf16, int* nch, int* tch) {
  if (bf16) {
    *tch = kSelTok;
    *nch = (N + kSelTok - 1) / kSelTok;
  } else {
    *tch = N > 0 ? N : 1;
    *nch = 1;
  }
}

}  // namespace

size_t selector_bwd_workspace(const Dims& d, bool bf16) {
  int nch, tch;
  sel_plan(d.N, bf16, &nch, &tch);
  return align_up(size_t(nch) * d.B * d.Hkv * size_t(d.C) * d.D * sizeof(float));
}

hipError_t launch_selector_bwd(const void* q, const void* kbar, const float* ds, void* dq, void* dk,
                               float* dkbar, const Dims& d, float scale, bool accumulate, bool bf16,
                               void* ws, hipStream_t s) {
  SelArgs a{};
  a.q = q;
  a.kbar = kbar;
  a.ds = ds;
  a.dq = dq;
  a.dk = dk;
  a.dkbar = dkbar;
  a.part = static_cast<float*>(ws);
  a.B = d.B;
  a.Hq = d.Hq;
  a.Hkv = d.Hkv;
  a.N = d.N;
  a.D = d.D;
  a.block = d.block;
  a.C = d.C;
  sel_plan(d.N, bf16, &a.nch, &a.tch);
  a.scale = scale;
  a.accumulate = accumulate ? 1 : 0;
  if (d.D == 64) return selector_bwd_t<64>(a, bf16, s);
  return selector_bwd_t<128>(a, bf16, s);
}

}  // namespace sas
