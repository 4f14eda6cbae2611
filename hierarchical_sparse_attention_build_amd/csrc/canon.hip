// Canonical form of caller-given group lists, for the attention kernels.
//
// The visible set of a query is the set union of its always-visible chunks
// (sink, local, current) and the tokens of its listed groups, up to the query
// [HGA technical summary (it), Meccanismo Core, item 2, third bullet, and
// item 4].  Routing only lists groups of candidate chunks, once each; a list a
// caller gives (route once, attend many; a backward pass) may repeat a group,
// name a group inside a forced chunk, after the query, or outside the cache.
// Every such entry adds no token to the set, so it is replaced by a hole (-1),
// and the attention kernels, which skip holes, then count every token once.
//
// A group g of query chunk j is kept iff 0 <= g < n_cap / G, its chunk
// c = g / m lies in [n_sink, j - n_local) (the chunks that are neither forced
// nor after j), and no earlier entry of the list names g.
#include "hga_device.hpp"
#include "hga_kernels.hpp"

namespace hga {

constexpr int kCanonThreads = 256;

__global__ __launch_bounds__(kCanonThreads) void canon_groups_kernel(CanonArgs a) {
  const KParams& kp = a.kp;
  const int64_t unit = blockIdx.x;  // (b, kv head, query chunk)
  const int u = static_cast<int>(unit % a.n_units);
  const int b = static_cast<int>(unit / a.n_units / kp.Hkv);
  const int32_t* in = a.in + unit * kp.top_g;
  int32_t* out = a.out + unit * kp.top_g;
  __shared__ int32_t g_s[kCanonMaxList];
  const int64_t t0 = (a.q_pos ? static_cast<int64_t>(a.q_pos[b]) : 0) + a.pos_bias;
  // query chunk of the unit; a position outside the cache keeps no entry (the
  // attention kernels write NaN for it)
  const int64_t j = t0 < 0 ? -1 : t0 / kp.C + (a.nq == 1 ? 0 : u);
  const int64_t n_groups_cap = kp.n_cap / kp.G;
  for (int e = threadIdx.x; e < kp.top_g; e += kCanonThreads) {
    const int32_t g = in[e];
    const int64_t c = g >= 0 ? g / kp.m : -1;
    const bool ok = g >= 0 && g < n_groups_cap && c >= kp.n_sink && c < j - kp.n_local;
    g_s[e] = ok ? g : -1;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < kp.top_g; e += kCanonThreads) {
    const int32_t g = g_s[e];
    bool first = g >= 0;
    for (int f = 0; first && f < e; ++f) first = g_s[f] != g;
    out[e] = first ? g : -1;
  }
}

hipError_t launch_canon_groups(const CanonArgs& a, hipStream_t st) {
  if (a.kp.top_g <= 0) return hipSuccess;
  if (a.kp.top_g > kCanonMaxList) return hipErrorInvalidValue;
  const int64_t units = static_cast<int64_t>(a.kp.B) * a.kp.Hkv * a.n_units;
  canon_groups_kernel<<<static_cast<unsigned>(units), kCanonThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace hga
