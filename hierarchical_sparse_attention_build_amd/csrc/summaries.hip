// Step 1 of HGA: RoPE-aware chunk and group key summaries.
// [HGA technical summary (it), Meccanismo Core, item 3].  bf16 post-RoPE keys
// with C <= 64: 16-byte row loads and one wave per group; otherwise the generic
// routine.  One workgroup per chunk of one (b, kv head).  See hga_summarize.hpp.
#include "hga_kernels.hpp"
#include "hga_summarize.hpp"

namespace hga {

constexpr int kSumThreads = 256;

template <typename T, int D>
__global__ __launch_bounds__(kSumThreads) void summaries_kernel(const T* __restrict__ K,
                                                                T* __restrict__ Krot,
                                                                float* __restrict__ chunk_sum,
                                                                float* __restrict__ group_sum,
                                                                int chunk_begin, int rotated,
                                                                KParams kp) {
  const int c = chunk_begin + blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int64_t row0 = bh * kp.n_cap + static_cast<int64_t>(c) * kp.C;
  summarize_chunk<T, D>(K + row0 * D, c, kp, rotated != 0, Krot ? Krot + row0 * D : nullptr,
                        chunk_sum + (bh * kp.n_chunks_cap + c) * D,
                        group_sum + (bh * kp.n_chunks_cap * kp.m + static_cast<int64_t>(c) * kp.m) * D);
}

// bf16 post-RoPE keys, C <= 64: the fast path of hga_summarize.hpp.
constexpr int kSumLdsFloats = 8448;  // 2 * (G + C/G) * d/2 + (C/G) * d for every C <= 64

template <int D, int MAXL>
__global__ __launch_bounds__(kSumThreads) void summaries_fast_kernel(const bf16* __restrict__ K,
                                                                     float* __restrict__ chunk_sum,
                                                                     float* __restrict__ group_sum, int chunk_begin,
                                                                     KParams kp) {
  extern __shared__ __align__(16) float lds[];  // summarize_lds_floats(kp)
  const int c = chunk_begin + blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int64_t row0 = bh * kp.n_cap + static_cast<int64_t>(c) * kp.C;
  summarize_chunk_fast<D, MAXL>(K + row0 * D, kp, lds, chunk_sum + (bh * kp.n_chunks_cap + c) * D,
                          group_sum + (bh * kp.n_chunks_cap * kp.m + static_cast<int64_t>(c) * kp.m) * D);
}

template <typename T, int D>
static hipError_t launch_summaries_t(const SummariesArgs& a, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    if (summarize_fast_ok<D>(a.kp, true, a.rotated != 0, kSumLdsFloats) && !a.Krot) {
      dim3 grid(a.chunk_end - a.chunk_begin, a.kp.B * a.kp.Hkv);
      const size_t lds_bytes = static_cast<size_t>(summarize_lds_floats(a.kp)) * sizeof(float);
      if (summarize_loads_per_group<D>(a.kp) == 4)
        summaries_fast_kernel<D, 4><<<grid, kSumThreads, lds_bytes, st>>>(static_cast<const bf16*>(a.K), a.chunk_sum,
                                                                  a.group_sum, a.chunk_begin, a.kp);
      else
        summaries_fast_kernel<D, 16><<<grid, kSumThreads, lds_bytes, st>>>(static_cast<const bf16*>(a.K), a.chunk_sum,
                                                                   a.group_sum, a.chunk_begin, a.kp);
      return hipGetLastError();
    }
  }
  dim3 grid(a.chunk_end - a.chunk_begin, a.kp.B * a.kp.Hkv);
  summaries_kernel<T, D><<<grid, kSumThreads, 0, st>>>(
      static_cast<const T*>(a.K), static_cast<T*>(a.Krot), a.chunk_sum, a.group_sum, a.chunk_begin,
      a.rotated, a.kp);
  return hipGetLastError();
}

hipError_t launch_summaries(const SummariesArgs& a, bool bf16_in, hipStream_t st) {
  if (a.chunk_end <= a.chunk_begin) return hipSuccess;
  if (bf16_in) return a.kp.d == 64 ? launch_summaries_t<bf16, 64>(a, st) : launch_summaries_t<bf16, 128>(a, st);
  return a.kp.d == 64 ? launch_summaries_t<float, 64>(a, st) : launch_summaries_t<float, 128>(a, st);
}

}  // namespace hga
