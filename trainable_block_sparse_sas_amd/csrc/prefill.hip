// Prefill into a paged cache: the prompt's keys and values go to the pages of
// its blocks, and every complete block's pooled key (the mean of its keys) to
// the pooled-key page array, so that sparse decode can start from the pages
// (blog 方法核心, kernel paragraph: dense prefill, sparse decode; review
// "Our Perspective", Strengths: the paged KV cache of the serving backend, and
// Limitations: pooling-based block summaries).
//
// One workgroup per (block, KV head, sequence): it copies the block's rows
// below the sequence's length into the block's page with 16-byte loads and
// stores, and, when the block is complete, sums its keys per column in fp32
// (rows in order) and writes the mean rounded to the page dtype.
#include "common.h"
#include "internal.h"

namespace sas {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void prefill_pages_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                                            const int32_t* __restrict__ seq_len,
                                                            const int32_t* __restrict__ table,
                                                            T* __restrict__ k_pages, T* __restrict__ v_pages,
                                                            T* __restrict__ kbar_pages, int Hkv, int N, int D,
                                                            int block, int max_blocks) {
  constexpr int VEC = 16 / int(sizeof(T));
  const int m = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  int len = seq_len[b];
  len = len < N ? len : N;
  const int r0 = m * block;
  if (len <= 0 || r0 >= len) return;
  const int nr = min(block, len - r0);
  const size_t page = size_t(table[size_t(b) * max_blocks + m]);
  const size_t src = ((size_t(b) * Hkv + g) * N + r0) * D;
  const size_t dst = (page * Hkv + g) * size_t(block) * D;
  const int nvec = nr * D / VEC;
  for (int i = threadIdx.x; i < nvec; i += 256) {
    reinterpret_cast<uint4*>(k_pages + dst)[i] = reinterpret_cast<const uint4*>(k + src)[i];
    reinterpret_cast<uint4*>(v_pages + dst)[i] = reinterpret_cast<const uint4*>(v + src)[i];
  }
  if (nr == block) {
    for (int d = threadIdx.x; d < D; d += 256) {
      float acc = 0.f;
      for (int r = 0; r < block; ++r) acc += to_f32(k[src + size_t(r) * D + d]);
      kbar_pages[(page * Hkv + g) * D + d] = from_f32<T>(acc / float(block));
    }
  }
}

}  // namespace

hipError_t launch_prefill_pages(const void* k, const void* v, const int32_t* seq_len, const int32_t* table,
                                void* k_pages, void* v_pages, void* kbar_pages, int B, int Hkv, int N, int D,
                                int block, int max_blocks, bool bf16, hipStream_t s) {
  const int nblk = (N + block - 1) / block;
  if (B == 0 || nblk == 0) return hipSuccess;
  const dim3 grid(nblk, Hkv, B);
  if (bf16)
    SAS_LAUNCH("prefill_pages", prefill_pages_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)k,
               (const bf16_t*)v, seq_len, table, (bf16_t*)k_pages, (bf16_t*)v_pages, (bf16_t*)kbar_pages, Hkv, N,
               D, block, max_blocks);
  else
    SAS_LAUNCH("prefill_pages", prefill_pages_kernel<float>, grid, dim3(256), 0, s, (const float*)k,
               (const float*)v, seq_len, table, (float*)k_pages, (float*)v_pages, (float*)kbar_pages, Hkv, N, D,
               block, max_blocks);
  return hipGetLastError();
}

}  // namespace sas
