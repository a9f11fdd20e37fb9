// Tile layouts shared by the matrix-core attention kernels, and the direct
// global -> LDS load helpers (gfx950, wave64).
//
// A key tile is one 64-key block.  Row-major K (and V) tiles keep D bf16 per
// key with 16-byte chunks XOR-swizzled by k_swz(key), so 16 lanes reading one
// chunk column of 16 consecutive keys hit distinct banks.  Transposed tiles
// (V^T for P V, K^T for dS K) hold [D][64] with the keys permuted into the k
// order in which a lane's P^T (or dS^T) values leave the S^T accumulators of
// v_mfma_f32_16x16x32_bf16, and chunks swizzled by vt_swz(d).
#pragma once

#include "common.h"

namespace sas {
namespace tiles {

constexpr int KT = 64;  // keys per tile = block size of the matrix-core kernels

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Key position p (0..63) inside a 64-key tile of V^T -> key index.  Within each
// group of 32, position 8q + j holds key 4q + j (j < 4) or 16 + 4q + j - 4: the
// k order in which a lane's P^T values leave the S^T accumulators.
__device__ __forceinline__ int vt_key_of_pos(int p) {
  const int hh = p >> 5, q = (p >> 3) & 3, j = p & 7;
  return 32 * hh + (j < 4 ? 4 * q + j : 16 + 4 * q + j - 4);
}
// 16-byte chunk swizzles (conflict-free reads of 16 rows at one chunk column).
// (A swizzle that also separates the 32-byte chunk pairs of ds_read_b64_tr_b16
// was measured: it raised the bank-conflict count of the forward and the dQ
// kernel and left the dK/dV kernel's unchanged, so this one stays.)
template <int D>
__device__ __forceinline__ int k_swz(int key) {
  return D == 128 ? (key & 15) : ((key >> 1) & 7);
}
__device__ __forceinline__ int vt_swz(int d) { return (d >> 1) & 7; }

// Per 64-key block of a [N][D] tensor x (V, or K): x^T [D][64] with the keys in
// vt_key_of_pos order and row d's 16-byte chunk cc stored at chunk
// cc ^ vt_swz(d).  Keys beyond N are zero.
template <int D>
__global__ __launch_bounds__(256) void vt_kernel(const bf16_t* __restrict__ v, bf16_t* __restrict__ vt,
                                                 int Hkv, int N, int NB) {
  __shared__ uint16_t vs[KT][D + 2];
  const int m = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const bf16_t* src = v + ((size_t(b) * Hkv + g) * N + size_t(m) * KT) * D;
  for (int i = threadIdx.x; i < KT * D; i += 256) {
    const int key = i / D, d = i % D;
    vs[key][d] = (m * KT + key < N) ? src[size_t(key) * D + d] : 0;
  }
  __syncthreads();
  bf16_t* dst = vt + ((size_t(b) * Hkv + g) * NB + m) * size_t(KT) * D;
  for (int i = threadIdx.x; i < D * 8; i += 256) {
    const int d = i >> 3, pc = i & 7;
    const int cc = pc ^ vt_swz(d);
    uint32_t w[4];
    for (int j2 = 0; j2 < 4; ++j2) {
      const int p0 = cc * 8 + 2 * j2;
      w[j2] = uint32_t(vs[vt_key_of_pos(p0)][d]) | (uint32_t(vs[vt_key_of_pos(p0 + 1)][d]) << 16);
    }
    *reinterpret_cast<uint4*>(dst + size_t(d) * KT + pc * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// s_waitcnt vmcnt(n) (gfx9 encoding; expcnt and lgkmcnt left unconstrained).
template <int n>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((n & 15) | 0x70 | 0xF00 | (((n >> 4) & 3) << 14));
}

// One lane's share of a wave's direct global -> LDS copy: 16 bytes from src
// land at lds + 16 lane (lds is the wave-uniform base).
__device__ __forceinline__ void dma16_to_lds(const void* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds, 16, 0, 0);
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane 4a + c receives
// element c of the 4 x 16-bit values addressed by lanes a, a + 4, a + 8 and
// a + 12 of its group (checked on gfx950 with a standalone probe).  Pointing
// lane s of a group at (row_i, col0 + 4 (s % 4)) with i = s / 4 hands lane
// 4a + c the column col0 + 4a + c of rows row_0 .. row_3: four k values of an
// MFMA operand whose k runs over rows, read from a row-major tile.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p);
  return __builtin_bit_cast(uint2, v);
}

// Workgroup barrier of a load ring.  __syncthreads() carries a release fence,
// which waits for every outstanding global->LDS load (vmcnt(0)), including the
// tiles meant to stay in flight across the barrier.  Here each wave first waits
// for its own LDS reads (so no later load can overwrite a stage still being
// read), then meets the others; loads into LDS are waited for explicitly with
// wait_vm before the barrier of the step that consumes them.  The memory
// clobber keeps the compiler from moving LDS accesses across.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unconstrained
  asm volatile("s_barrier" ::: "memory");
}

}  // namespace tiles
}  // namespace sas
