// Method parameters as the kernels see them (plain data, passed by value).
#pragma once

#include <stdint.h>

namespace hga {

constexpr int kMaxPairs = 64;  // head_dim <= 128

struct KParams {
  int32_t B, Hq, Hkv, d, C, G, m, gq;
  int32_t n_sink, n_local, top_k, top_g;
  int64_t n_cap;        // token capacity of K/V rows per (b, kv head)
  int32_t n_chunks_cap; // n_cap / C
  int32_t log2C, log2G; // log2 of C and G when they are powers of two, else -1
  float inv_sqrt_d;     // 1 / sqrt(d)
  float scale_log2;     // log2(e) / sqrt(d): attention scores are kept in base-2 units
  uint64_t hf_mask;     // bit i set: RoPE pair i is high-frequency
  float theta_f[kMaxPairs];   // theta_i (relative angles, small)
  double theta_d[kMaxPairs];  // theta_i (absolute angles, reduced in double)
};

// Forced (always-visible) chunks of query chunk j: sink chunks [0, a) and the
// window [lo, j].  When the two overlap the union is [0, j].
struct Forced {
  int32_t a, lo, n;  // n = number of distinct forced chunks
};

__host__ __device__ inline Forced forced_chunks(int32_t j, int32_t n_sink, int32_t n_local) {
  Forced f;
  f.a = n_sink < j + 1 ? n_sink : j + 1;
  f.lo = j - n_local > 0 ? j - n_local : 0;
  if (f.lo <= f.a) {
    f.lo = f.a;  // contiguous [0, j]
    f.n = j + 1;
  } else {
    f.n = f.a + (j - f.lo + 1);
  }
  return f;
}

// i-th forced chunk (ascending).
__host__ __device__ inline int32_t forced_chunk_at(const Forced& f, int32_t i) {
  return i < f.a ? i : f.lo + (i - f.a);
}

}  // namespace hga
