// Step 1 of HGA: RoPE-aware chunk and group key summaries.
// [HGA technical summary (it), Meccanismo Core, item 3].  bf16 post-RoPE keys
// with C <= 64: 8-byte row loads (both halves of each pair) and one wave per
// group; otherwise the generic
// routine.  One workgroup per chunk of one (b, kv head).  See hga_summarize.hpp.
#include "hga_kernels.hpp"
#include "hga_summarize.hpp"

#include <algorithm>

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

// bf16 post-RoPE keys, C <= 64: the fast path of hga_summarize.hpp.  A
// workgroup takes cpw consecutive chunks: the rotation tables (the same for
// every chunk) are built once, and each wave loads its group of the next chunk
// while the current chunk's group means are combined.  The group means of two
// consecutive chunks sit in two LDS buffers, so one barrier per chunk orders
// the means of a chunk before its combine and its combine before the same
// buffer is written again.
constexpr int kSumLdsFloats = 16384;  // 64 KB: tables and two sets of group means

__host__ __device__ inline int summaries_multi_lds_floats(const KParams& kp) {
  return summarize_lds_floats(kp) + kp.m * kp.d;
}

template <int D, int MAXL>
__global__ __launch_bounds__(kSumThreads) void summaries_fast_kernel(const bf16* __restrict__ K,
                                                                     float* __restrict__ chunk_sum,
                                                                     float* __restrict__ group_sum, int chunk_begin,
                                                                     int chunk_end, int cpw, KParams kp) {
  extern __shared__ __align__(16) float lds[];  // summaries_multi_lds_floats(kp)
  constexpr int P = D / 2;
  float2* rot = reinterpret_cast<float2*>(lds);
  float2* crot = rot + kp.G * P;
  float* gmean0 = reinterpret_cast<float*>(crot + kp.m * P);
  float* gmean1 = gmean0 + kp.m * D;
  const int64_t bh = blockIdx.y;
  const int c0 = chunk_begin + blockIdx.x * cpw;
  const int c1 = min(chunk_end, c0 + cpw);
  const int wid = wave_id(), nw = static_cast<int>(blockDim.x) / kWave;
  const bool one_group_per_wave = kp.m <= nw;
  auto rows_of = [&](int c) { return K + (bh * kp.n_cap + static_cast<int64_t>(c) * kp.C) * D; };
  GroupRows<D, MAXL> rows;
  if (wid < kp.m) load_group_rows<D, MAXL>(rows_of(c0), kp, wid, rows);
  build_summary_tables<D>(kp, rot, crot);
  for (int c = c0; c < c1; ++c) {
    float* gmean = ((c - c0) & 1) ? gmean1 : gmean0;
    float* gs_out = group_sum + (bh * kp.n_chunks_cap * kp.m + static_cast<int64_t>(c) * kp.m) * D;
    for (int g = wid; g < kp.m; g += nw) {
      if (g != wid) load_group_rows<D, MAXL>(rows_of(c), kp, g, rows);
      group_mean_wave<D, MAXL>(rows, kp, rot, g, gs_out, gmean);
    }
    // the next chunk's rows are on their way during the barrier and the combine
    if (one_group_per_wave && wid < kp.m && c + 1 < c1) load_group_rows<D, MAXL>(rows_of(c + 1), kp, wid, rows);
    __syncthreads();
    combine_chunk<D>(kp, crot, gmean, chunk_sum + (bh * kp.n_chunks_cap + c) * D);
  }
}

// chunks per workgroup: enough workgroups to fill the chip a few times over
static int summaries_cpw(int chunks, int bh) {
  const int64_t total = static_cast<int64_t>(chunks) * bh;
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(8, total / 1024)));
}

template <typename T, int D>
static hipError_t launch_summaries_t(const SummariesArgs& a, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    if (summarize_fast_ok<D>(a.kp, true, a.rotated != 0, kSumLdsFloats - a.kp.m * a.kp.d) && !a.Krot) {
      const int chunks = a.chunk_end - a.chunk_begin;
      const int bh = a.kp.B * a.kp.Hkv;
      const int cpw = summaries_cpw(chunks, bh);
      dim3 grid((chunks + cpw - 1) / cpw, bh);
      const size_t lds_bytes = static_cast<size_t>(summaries_multi_lds_floats(a.kp)) * sizeof(float);
      if (summarize_loads_per_group<D>(a.kp) == 4)
        summaries_fast_kernel<D, 4><<<grid, kSumThreads, lds_bytes, st>>>(static_cast<const bf16*>(a.K), a.chunk_sum,
                                                                  a.group_sum, a.chunk_begin, a.chunk_end, cpw,
                                                                  a.kp);
      else
        summaries_fast_kernel<D, 16><<<grid, kSumThreads, lds_bytes, st>>>(static_cast<const bf16*>(a.K), a.chunk_sum,
                                                                   a.group_sum, a.chunk_begin, a.chunk_end, cpw,
                                                                   a.kp);
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
