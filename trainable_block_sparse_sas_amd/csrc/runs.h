// Sorted runs of composite keys held in wave registers, for the Top-K
// kernels (gfx950, wave64).  Keys are unsigned integers (a 32-bit score key,
// or score key << 32 | ~block); larger sorts first.  A run of KP = R E keys
// lives in a group of R lanes, E keys per lane (element q E + r of a run:
// lane q of the group, register r).  Two sorted runs A and B reduce to the KP
// largest keys of their union by max(A[j], B[KP - 1 - j]), a bitonic sequence
// that the half-cleaners sort again.  All lane exchanges use DPP and the
// gfx950 row swaps (lanes_xor), not LDS permutes.
#pragma once

#include "common.h"

namespace sas {

__device__ __forceinline__ uint64_t shfl_xor_key(uint64_t v, int mask) {
  const int lane = threadIdx.x & 63;
  const uint32_t lo = lanes_xor(uint32_t(v), mask, lane);
  const uint32_t hi = lanes_xor(uint32_t(v >> 32), mask, lane);
  return (uint64_t(hi) << 32) | lo;
}
__device__ __forceinline__ uint32_t shfl_xor_key(uint32_t v, int mask) {
  return lanes_xor(v, mask, threadIdx.x & 63);
}

// Sorts the bitonic run held by each group of R lanes (E keys per lane)
// descending: half-cleaners at element distances KP/2 .. 1 (KP = R E).
constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

template <int E, int R, typename T>
__device__ __forceinline__ void bitonic_clean(T (&v)[E], int lane) {
  // distances as 1 << sh with a linear counter, so the loop fully unrolls and
  // every lane-exchange mask is a compile-time constant
#pragma unroll
  for (int sh = ilog2(R * E / 2); sh >= 0; --sh) {
    const int d = 1 << sh;
    if (d >= E) {
      const int dl = d / E;
      const bool lower = (lane & dl) == 0;
#pragma unroll
      for (int r = 0; r < E; ++r) {
        const T p = shfl_xor_key(v[r], dl);
        v[r] = lower ? (v[r] > p ? v[r] : p) : (v[r] < p ? v[r] : p);
      }
    } else {
#pragma unroll
      for (int r = 0; r < E; ++r)
        if ((r & d) == 0) {
          const T a = v[r], b = v[r + d];
          v[r] = a > b ? a : b;
          v[r + d] = a > b ? b : a;
        }
    }
  }
}

// Every group of R lanes holds a sorted run of R E keys; afterwards every
// group holds the R E largest keys of all 64 / R runs of the wave, sorted.
template <int E, int R, typename T>
__device__ __forceinline__ void merge_wave_runs(T (&v)[E], int lane) {
#pragma unroll
  for (int sh = ilog2(R); sh < 6; ++sh) {
    const int D = 1 << sh;
    T p[E];
#pragma unroll
    for (int r = 0; r < E; ++r) p[r] = shfl_xor_key(v[E - 1 - r], D | (R - 1));
#pragma unroll
    for (int r = 0; r < E; ++r) v[r] = v[r] > p[r] ? v[r] : p[r];
    bitonic_clean<E, R>(v, lane);
  }
}

// Sorted runs of ML E keys over groups of ML lanes from sorted runs of half
// that length (one bitonic merge per doubling), for ML = 2 .. R.
template <int E, int ML, int R, typename T>
__device__ __forceinline__ void build_runs(T (&v)[E], int lane) {
  if constexpr (ML <= R) {
    const bool lower = (lane & (ML - 1)) < ML / 2;
    T p[E];
#pragma unroll
    for (int r = 0; r < E; ++r) p[r] = shfl_xor_key(v[E - 1 - r], ML - 1);
#pragma unroll
    for (int r = 0; r < E; ++r) v[r] = lower ? (v[r] > p[r] ? v[r] : p[r]) : (v[r] < p[r] ? v[r] : p[r]);
    bitonic_clean<E, ML>(v, lane);
    build_runs<E, 2 * ML, R, T>(v, lane);
  }
}

// Merges the W wave runs in runs[0] (each R lanes x E keys, sorted) into
// one, GPW = 64 / R runs per merging wave per round; returns the buffer that
// holds the result in its row 0 (visible to every wave on return).
template <int E, int R, int KP, int W, typename T>
__device__ __forceinline__ int merge_block_runs(T (*runs)[W][KP], int w, int lane) {
  constexpr int GPW = 64 / R;
  static_assert(GPW >= 2, "a round must reduce the run count");
  int nruns = W, buf = 0;
  while (nruns > 1) {
    const int nw = (nruns + GPW - 1) / GPW;
    __syncthreads();
    if (w < nw) {
      const int src = w * GPW + lane / R;
      T v[E];
#pragma unroll
      for (int r = 0; r < E; ++r) v[r] = src < nruns ? runs[buf][src][(lane % R) * E + r] : T(0);
      merge_wave_runs<E, R, T>(v, lane);
      if (lane < R)
#pragma unroll
        for (int r = 0; r < E; ++r) runs[buf ^ 1][w][lane * E + r] = v[r];
    }
    buf ^= 1;
    nruns = nw;
  }
  __syncthreads();
  return buf;
}

// As merge_block_runs, for nruns (<= W) runs in runs[0] merged by the first
// `waves` waves of the workgroup, each taking every waves-th group of 64 / R
// runs in a round.  Every thread of the workgroup calls it.
template <int E, int R, int KP, int W, typename T>
__device__ __forceinline__ int merge_runs_n(T (*runs)[W][KP], int nruns, int waves, int w, int lane) {
  constexpr int GPW = 64 / R;
  static_assert(GPW >= 2, "a round must reduce the run count");
  int buf = 0;
  while (nruns > 1) {
    const int nw = (nruns + GPW - 1) / GPW;
    __syncthreads();
    for (int grp = w; grp < nw && w < waves; grp += waves) {
      const int src = grp * GPW + lane / R;
      T v[E];
#pragma unroll
      for (int r = 0; r < E; ++r) v[r] = src < nruns ? runs[buf][src][(lane % R) * E + r] : T(0);
      merge_wave_runs<E, R, T>(v, lane);
      if (lane < R)
#pragma unroll
        for (int r = 0; r < E; ++r) runs[buf ^ 1][grp][lane * E + r] = v[r];
    }
    buf ^= 1;
    nruns = nw;
  }
  __syncthreads();
  return buf;
}

}  // namespace sas
