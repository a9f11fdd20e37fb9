// Matrix-core helpers for gfx950 (CDNA4), wave64.
//
// v_mfma_f32_16x16x32_bf16: C[16x16] += A[16x32] * B[32x16].
// Lane l holds A row (l % 16), k = 8*(l/16) .. 8*(l/16)+7; B column (l % 16),
// the same 8 k; C column (l % 16), rows 4*(l/16) .. 4*(l/16)+3.
// (Lane layout checked on the hardware with a standalone probe.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sas {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

__device__ __forceinline__ f32x4 mfma16(const uint4& a, const uint4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Two fp32 -> packed bf16 pair (round to nearest even, hardware conversion).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2_t r;
  r.x = static_cast<__bf16>(lo);
  r.y = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// XCD-aware workgroup order.  Workgroups are handed to the 8 XCDs round-robin
// by linear id; when the number of (batch, KV head) pairs is a multiple of 8,
// every pair is pinned to one XCD so its K/V stream stays in that XCD's L2.
// Work items are visited heaviest first (highest tile index first).
__device__ __forceinline__ void xcd_order(int lin, int n_tiles, int n_pairs, int* tile, int* pair) {
  if ((n_pairs & 7) == 0) {
    const int x = lin & 7, j = lin >> 3;
    const int per = n_pairs >> 3;
    *tile = n_tiles - 1 - j / per;
    *pair = x + 8 * (j % per);
  } else {
    *tile = n_tiles - 1 - lin / n_pairs;
    *pair = lin % n_pairs;
  }
}

}  // namespace sas
