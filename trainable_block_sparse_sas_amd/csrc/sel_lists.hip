// Per-block lists of the tokens that select each history block: the transpose
// of the Top-K selection (each token's k chosen earlier blocks, the sparse
// branch of the method: jaehun.me review "Why the Four Design Choices Matter",
// the Top-K gate; the blog's 方法核心 section), used by the key-major kernels.
//
//   bits   per token, a bitmask of its valid selected blocks (m < own block;
//          entries out of range or repeated count once), and pre, the number of
//          set bits before each 32-block word (pre[MWB] = number selected).
//          Optionally also the log gates of the token's slots, so that the
//          forward reads one contiguous record per (token, slot) instead of
//          gathering a score and an LSE_s per query row.
//   count  per (KV head, word w, token segment): how many tokens of the segment
//          select each of the word's 32 blocks.
//   scan   per KV head: exclusive offsets over (block, segment), so each
//          block's list is its segments' tokens in ascending order, and the work
//          items in (token span, block) order: a block's own tokens, or a run of
//          at most `chunk` list entries whose tokens fall in one span of
//          ISEG segments (items that run together then share query rows).
//   fill   the lists, entry = token | (rank of the block among the token's
//          selected blocks) << 23, and per (token, rank) the entry's position.
// Every step is deterministic: the lists come out sorted by token.
#include "common.h"
#include "internal.h"

#include <algorithm>

namespace sas {
namespace {

constexpr int SEG = 512;           // tokens per segment of the count / fill passes
constexpr int kSegsPerSpan = 4;    // segments per token span of the work items (2048 tokens)

// One wave per token: lane e ORs its entry's bit into the wave's words in LDS
// (a repeated entry sets the same bit), then lane w takes word w.  With gates,
// lane e then writes the log gates of its entry's slot (the slot's rank from
// the words and their prefix counts; a repeated entry writes the same values
// to the same slot).
constexpr int kMaxWords = 512;  // 16384 blocks, the most a sparse-scope call accepts

__global__ __launch_bounds__(256) void selbits_kernel(const int32_t* __restrict__ idx,
                                                      uint32_t* __restrict__ bits,
                                                      uint16_t* __restrict__ pre, int N, int topk,
                                                      int block, int MWB, size_t tokens, SelGates sg) {
  __shared__ uint32_t wsh[4][kMaxWords];
  __shared__ uint16_t psh[4][kMaxWords];
  const size_t tok = size_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (tok >= tokens) return;
  const int t = int(tok % N);
  const int c = t / block;
  const int32_t* ir = idx + tok * topk;
  uint32_t* ws = wsh[wave];
  for (int w = lane; w < MWB; w += 64) ws[w] = 0u;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  for (int e = lane; e < topk; e += 64) {
    const int m = ir[e];
    if (m >= 0 && m < c) atomicOr(ws + (m >> 5), 1u << (m & 31));
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  int carry = 0;
  for (int w0 = 0; w0 < MWB; w0 += 64) {
    const int w = w0 + lane;
    const uint32_t word = w < MWB ? ws[w] : 0u;
    if (w < MWB) bits[tok * MWB + w] = word;
    const int cnt = __popc(word);
    int incl = cnt;
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (w < MWB) {
      pre[tok * (MWB + 1) + w] = uint16_t(carry + incl - cnt);
      psh[wave][w] = uint16_t(carry + incl - cnt);
    }
    carry += __shfl(incl, 63, 64);
  }
  if (lane == 0) pre[tok * (MWB + 1) + MWB] = uint16_t(carry);
  if (sg.out == nullptr) return;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // query row of head h of the group: (pair G + h) N + t
  const int G = sg.G;
  const size_t r0 = (tok / N) * size_t(G) * N + t;
  for (int e = lane; e < topk; e += 64) {
    const int m = ir[e];
    if (m < 0 || m >= c) continue;
    const int wd = m >> 5;
    const uint32_t slot = psh[wave][wd] + uint32_t(__popc(ws[wd] & ((1u << (m & 31)) - 1u)));
    // every load first (heads past G repeat head G - 1), so they go out
    // together rather than one head per round trip
    float sv[8], lv[8], x[8];
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      const size_t r = r0 + size_t(h < G ? h : G - 1) * N;
      sv[h] = sg.scores[r * sg.C + m];
      lv[h] = sg.lse_s[r];
    }
#pragma unroll
    for (int h = 0; h < 8; ++h) x[h] = (sv[h] - lv[h]) * kLog2e;
    float* op = sg.out + (tok * topk + slot) * G;
    if (G == 4) {
      *reinterpret_cast<float4*>(op) = make_float4(x[0], x[1], x[2], x[3]);
    } else {
#pragma unroll
      for (int h = 0; h < 8; ++h)
        if (h < G) op[h] = x[h];
    }
  }
}

// One wave per (KV head, word, segment).  FILL = false: counts; true: entries.
template <bool FILL>
__global__ __launch_bounds__(64) void sel_pass_kernel(SelLists L, int N, int C, int block) {
  const int lane = threadIdx.x;
  const int seg = blockIdx.x % L.nseg;
  const int w = (blockIdx.x / L.nseg) % L.MWB;
  const int pair = blockIdx.x / (L.nseg * L.MWB);
  const int MWB = L.MWB;
  // tokens that can select a block of word w start at block 32 w + 1
  const int t0 = max(seg * SEG, (32 * w + 1) * block);
  const int t1 = min(N, (seg + 1) * SEG);
  const size_t tok0 = size_t(pair) * N;
  const size_t cell = (size_t(pair) * L.NB + 32 * w) * L.nseg + seg;  // (pair, m = 32 w, seg)
  // running position per block b of the word: lane b holds it
  uint32_t run = 0;
  if (FILL && lane < 32 && 32 * w + lane < C) run = L.segoff[cell + size_t(lane) * L.nseg];
  uint32_t* ents = L.ents + size_t(pair) * L.ents_per_pair;
  const unsigned long long lt = lane ? (~0ull >> (64 - lane)) : 0ull;
  for (int tb = t0; tb < t1; tb += 64) {
    const int t = tb + lane;
    const bool ok = t < t1;
    const uint32_t word = ok ? L.bits[(tok0 + t) * MWB + w] : 0u;
    const int base = (FILL && ok) ? int(L.pre[(tok0 + t) * (MWB + 1) + w]) : 0;
#pragma unroll 4
    for (int b = 0; b < 32; ++b) {
      const bool sel = (word >> b) & 1u;
      const unsigned long long bal = __ballot(sel);
      if (bal == 0ull) continue;
      const uint32_t rb = uint32_t(__builtin_amdgcn_readlane(int(run), b));
      if (FILL && sel) {
        const uint32_t slot = uint32_t(base + __popc(word & ((1u << b) - 1u)));
        const uint32_t at = rb + uint32_t(__popcll(bal & lt));
        ents[at] = uint32_t(t) | (slot << 23);
        L.pos[(tok0 + t) * L.topk + slot] = at;
      }
      if (lane == b) run = rb + uint32_t(__popcll(bal));
    }
  }
  if (!FILL && lane < 32 && 32 * w + lane < C) L.cnt[cell + size_t(lane) * L.nseg] = run;
}

// Workgroup-wide exclusive scan of one value per thread (1024 threads).
__device__ uint32_t block_scan_excl(uint32_t v, uint32_t* sh, uint32_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t incl = v;
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    uint32_t x = lane < 16 ? sh[lane] : 0u;
    uint32_t xi = x;
    for (int off = 1; off < 16; off <<= 1) {
      const uint32_t y = __shfl_up(xi, off, 64);
      if (lane >= off) xi += y;
    }
    if (lane < 16) sh[16 + lane] = xi - x;
    if (lane == 15) sh[32] = xi;
  }
  __syncthreads();
  const uint32_t r = sh[16 + wave] + incl - v;
  *total = sh[32];
  __syncthreads();
  return r;
}

// One workgroup per KV head: block offsets, segment offsets and work items.
// Item = {m | own << 31, first entry, end entry, 0} (entries pair-relative).
__global__ __launch_bounds__(1024) void sel_scan_kernel(SelLists L, int N, int C, int block) {
  __shared__ uint32_t sh[40];
  const int pair = blockIdx.x;
  const int tid = threadIdx.x;
  const int NB = L.NB, nseg = L.nseg;
  uint32_t ecarry = 0;
  for (int m0 = 0; m0 < NB; m0 += 1024) {
    const int m = m0 + tid;
    // a block's segment counts are one contiguous row (16-byte pieces when
    // nseg is a multiple of 4)
    const bool vec = (nseg & 3) == 0;
    const size_t rowc = (size_t(pair) * NB + m) * nseg;
    uint32_t cm = 0;
    if (m < C) {
      if (vec)
        for (int sg = 0; sg < nseg; sg += 4) {
          const uint4 c4 = *reinterpret_cast<const uint4*>(L.cnt + rowc + sg);
          cm += c4.x + c4.y + c4.z + c4.w;
        }
      else
        for (int sg = 0; sg < nseg; ++sg) cm += L.cnt[rowc + sg];
    }
    uint32_t etot;
    const uint32_t eoff = ecarry + block_scan_excl(cm, sh, &etot);
    if (m < NB) {
      L.blkoff[size_t(pair) * (NB + 1) + m] = eoff;
      uint32_t run = eoff;
      if (m < C) {
        if (vec)
          for (int sg = 0; sg < nseg; sg += 4) {
            const uint4 c4 = *reinterpret_cast<const uint4*>(L.cnt + rowc + sg);
            uint4 o;
            o.x = run;
            o.y = o.x + c4.x;
            o.z = o.y + c4.y;
            o.w = o.z + c4.z;
            run = o.w + c4.w;
            *reinterpret_cast<uint4*>(L.segoff + rowc + sg) = o;
          }
        else
          for (int sg = 0; sg < nseg; ++sg) {
            const uint32_t c = L.cnt[rowc + sg];
            L.segoff[rowc + sg] = run;
            run += c;
          }
      }
    }
    ecarry += etot;
  }
  if (tid == 0) L.blkoff[size_t(pair) * (NB + 1) + NB] = ecarry;
  __syncthreads();  // segment offsets visible to the whole workgroup
  // work items over cells (span, block), span-major
  const int spi = kSegsPerSpan;
  const int nspan = (nseg + spi - 1) / spi;
  const int ncell = nspan * NB;
  uint32_t icarry = 0;
  uint32_t* items = L.items + size_t(pair) * L.maxitems * 4;
  for (int c0 = 0; c0 < ncell; c0 += 1024) {
    const int cell = c0 + tid;
    const int sp = cell / NB, m = cell % NB;
    uint32_t first = 0, cnt = 0, own = 0;
    if (cell < ncell) {
      own = (m * block) / (SEG * spi) == sp ? 1u : 0u;
      if (m < C) {
        const int s0 = sp * spi, s1 = min(nseg, s0 + spi);
        const size_t base = (size_t(pair) * NB + m) * nseg;
        first = L.segoff[base + s0];
        cnt = (s1 < nseg ? L.segoff[base + s1] : L.blkoff[size_t(pair) * (NB + 1) + m + 1]) - first;
      }
    }
    const uint32_t n = own + (cnt + L.chunk - 1) / L.chunk;
    uint32_t itot;
    const uint32_t ioff = icarry + block_scan_excl(n, sh, &itot);
    if (cell < ncell) {
      uint32_t* it = items + size_t(ioff) * 4;
      if (own) {
        it[0] = uint32_t(m) | 0x80000000u;
        it[1] = 0;
        it[2] = 0;
        it[3] = 0;
        it += 4;
      }
      for (uint32_t e = 0; e < cnt; e += L.chunk, it += 4) {
        it[0] = uint32_t(m);
        it[1] = first + e;
        it[2] = first + min(cnt, e + uint32_t(L.chunk));
        it[3] = 0;
      }
    }
    icarry += itot;
  }
  if (tid == 0) L.nitems[pair] = icarry;
}

}  // namespace

SelLists sel_lists_layout(int B, int Hkv, int N, int C, int topk, int block, int chunk, char* base,
                          size_t* bytes) {
  SelLists L{};
  const size_t pairs = size_t(B) * Hkv, tokens = pairs * N;
  L.MWB = C > 0 ? (C + 31) / 32 : 1;
  L.NB = (N + block - 1) / block;
  L.nseg = (N + SEG - 1) / SEG;
  L.chunk = chunk;
  L.ents_per_pair = size_t(N) * topk;
  {
    // own items + full runs + one partial run per nonempty (span, block) cell
    const size_t nspan = (L.nseg + kSegsPerSpan - 1) / kSegsPerSpan;
    const size_t ents = size_t(N) * topk;
    L.maxitems = int(L.NB + ents / chunk + std::min(ents, nspan * L.NB) + 1);
  }
  size_t at = 0;
  auto take = [&](size_t n) {
    const size_t o = at;
    at += align_up(n);
    return base ? base + o : nullptr;
  };
  L.bits = reinterpret_cast<uint32_t*>(take(tokens * L.MWB * 4));
  L.pre = reinterpret_cast<uint16_t*>(take(tokens * (L.MWB + 1) * 2));
  L.cnt = reinterpret_cast<uint32_t*>(take(pairs * L.NB * L.nseg * 4));
  L.segoff = reinterpret_cast<uint32_t*>(take(pairs * L.NB * L.nseg * 4));
  L.blkoff = reinterpret_cast<uint32_t*>(take(pairs * (L.NB + 1) * 4));
  L.nitems = reinterpret_cast<uint32_t*>(take(pairs * 4));
  L.items = reinterpret_cast<uint32_t*>(take(pairs * L.maxitems * 16));
  L.ents = reinterpret_cast<uint32_t*>(take(pairs * L.ents_per_pair * 4));
  L.pos = reinterpret_cast<uint32_t*>(take(tokens * size_t(topk > 0 ? topk : 1) * 4));
  L.topk = topk;
  if (bytes) *bytes = at;
  return L;
}

SparseCtx sparse_ctx_layout(const Dims& d, int topk, char* base, size_t* bytes) {
  SparseCtx c{};
  size_t lb = 0;
  c.L = sel_lists_layout(d.B, d.Hkv, d.N, d.C, topk, d.block, kListChunk, base, &lb);
  const size_t gb = size_t(d.B) * d.Hkv * c.L.ents_per_pair * d.G() * sizeof(float);
  c.lg2 = base ? reinterpret_cast<float*>(base + align_up(lb)) : nullptr;
  if (bytes) *bytes = align_up(lb) + align_up(gb);
  return c;
}

hipError_t launch_sel_lists(const int32_t* idx, const SelLists& L, int B, int Hkv, int N, int C,
                            int topk, int block, hipStream_t s, const SelGates* gates) {
  const size_t tokens = size_t(B) * Hkv * N;
  const int pairs = B * Hkv;
  if (L.MWB > kMaxWords) return hipErrorInvalidValue;  // more blocks than the entry points accept
  SelGates sg{};
  if (gates) {
    if (gates->G < 1 || gates->G > 8) return hipErrorInvalidValue;
    sg = *gates;
  }
  SAS_LAUNCH("selbits", selbits_kernel, dim3((tokens + 3) / 4), dim3(256), 0, s, idx, L.bits, L.pre, N,
             topk, block, L.MWB, tokens, sg);
  if (C > 0) {
    SAS_LAUNCH("sel_count", sel_pass_kernel<false>, dim3(pairs * L.MWB * L.nseg), dim3(64), 0, s, L, N, C,
               block);
  }
  SAS_LAUNCH("sel_scan", sel_scan_kernel, dim3(pairs), dim3(1024), 0, s, L, N, C, block);
  if (C > 0) {
    SAS_LAUNCH("sel_fill", sel_pass_kernel<true>, dim3(pairs * L.MWB * L.nseg), dim3(64), 0, s, L, N, C,
               block);
  }
  return hipGetLastError();
}

}  // namespace sas
