// Device-side helpers shared by the libsas kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sas {

typedef uint16_t bf16_t;  // bfloat16 stored as raw bits

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// float -> bfloat16 with round-to-nearest-even; NaN stays a quiet NaN.
// fp32 -> bf16, round to nearest even (one v_cvt_pk_bf16_f32 on gfx950; NaN
// stays NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return f32_to_bf16(x); }

// exp / log through the hardware base-2 instructions (v_exp_f32, v_log_f32).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float log_hw(float x) { return __builtin_amdgcn_logf(x) * kLn2; }

// Gate activations (the values of sas_gate).
constexpr int kGateSoftmax = 0, kGateSigmoid = 1, kGateRaw = 2, kGateOuter = 3, kGateSte = 4;

// ds of a history block from db (its dz sum when gated, else 0), x = s - LSE_s
// (for the sigmoid gate s is the rewritten score log sigmoid(s) and LSE_s = 0,
// so e^x = sigmoid(s)) and the row's dbeta total: the chain rule through log g
// of each gate activation.
//   softmax  db - e^x total   (log g = s - LSE(s))
//   sigmoid  db (1 - e^x)     (d log sigmoid(s) / ds = 1 - sigmoid(s))
//   raw      db               (log g = s)
// (the outer gate records g dg as db and takes the softmax rule)
__device__ __forceinline__ float gate_ds(int gate, float db, float x, float tot) {
  if (gate == kGateSigmoid) return -db * expm1f(x);
  if (gate == kGateRaw) return db;
  return db - exp_hw(x) * tot;
}

__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }
__device__ __forceinline__ int shfl_xor(int v, int mask) { return __shfl_xor(v, mask, 64); }

// Max / sum over the four lanes l, l^16, l^32, l^48 (one 16-lane column of an
// MFMA accumulator tile) with the gfx950 row swaps instead of LDS permutes.
__device__ __forceinline__ float max_xrows(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_xrows(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// x of lane (lane ^ mask) without LDS permutes: within a 16-lane row the
// xor is composed from DPP moves (row_half_mirror = xor 7, quad_perm = xor
// 1..3, row_ror:8 = xor 8), across rows from the gfx950 row swaps (after
// v_permlane16_swap(x, x) the first result holds row r ^ 1's x in the odd
// rows and the second in the even rows; likewise for halves with the 32-lane
// swap).  Every call site passes a mask that is constant after unrolling, so
// the branches fold away.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t x) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t lanes_xor(uint32_t x, int mask, int lane) {
  if (mask & 4) x = dpp<0x141>(x);
  const int q = (mask & 3) ^ ((mask & 4) ? 3 : 0);
  if (q == 1) x = dpp<0xB1>(x);       // quad_perm [1,0,3,2]
  else if (q == 2) x = dpp<0x4E>(x);  // quad_perm [2,3,0,1]
  else if (q == 3) x = dpp<0x1B>(x);  // quad_perm [3,2,1,0]
  if (mask & 8) x = dpp<0x128>(x);    // row_ror:8
  if (mask & 16) {
    const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = (lane & 16) ? a[0] : a[1];
  }
  if (mask & 32) {
    const auto a = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    x = (lane & 32) ? a[0] : a[1];
  }
  return x;
}

// Order-preserving map of an fp32 value to uint32 (larger float -> larger key).
// -0.0 is folded onto +0.0 and NaN onto -inf first.
__device__ __forceinline__ uint32_t score_key(float f) {
  if (f != f) f = kNegInf;
  if (f == 0.0f) f = 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace sas
