// Cold tier of HGA: fetch the routed K/V groups from pinned host memory.
// [HGA technical summary (it), Architettura della Memoria (hot / warm / cold
// tiers; the full K/V history can live in host RAM) and Meccanismo Core item 4
// (the router fetches the original token K/V of the selected chunks/groups
// from host memory into device memory)].
//
// A copy kernel reads the host buffers directly over the host link (the pinned
// allocation is mapped into the device address space) and writes the packed
// staging buffer [B*Hkv, top_g*G, d] that the attention kernel reads.  The
// group ids come straight from the routing kernel's output in device memory,
// so no host round trip is needed.  Bound by the host link, not by HBM.
#include "hga_kernels.hpp"
#include "hga_select.hpp"


namespace hga {

constexpr int kGatherThreads = 256;
constexpr int kGroupsPerBlock = 8;

__global__ __launch_bounds__(kGatherThreads) void gather_groups_kernel(GatherArgs a) {
  const KParams& kp = a.kp;
  const int64_t bh = blockIdx.y;
  const int g0 = blockIdx.x * kGroupsPerBlock;
  const int64_t vec_per_group = static_cast<int64_t>(kp.G) * kp.d * a.elem_bytes / 16;
  const int64_t vec_per_row = static_cast<int64_t>(kp.d) * a.elem_bytes / 16;
  const int32_t* gl = a.group_idx + bh * kp.top_g;
  const int64_t n_groups_cap = kp.n_cap / kp.G;
  const uint4* Kh = static_cast<const uint4*>(a.K_host);
  const uint4* Vh = static_cast<const uint4*>(a.V_host);
  uint4* Ks = static_cast<uint4*>(a.K_stage);
  uint4* Vs = static_cast<uint4*>(a.V_stage);
  const int64_t total = kGroupsPerBlock * vec_per_group;
  for (int64_t e = threadIdx.x; e < total; e += kGatherThreads) {
    const int gi = g0 + static_cast<int>(e / vec_per_group);
    if (gi >= kp.top_g) break;
    const int g = gl[gi];
    if (g < 0 || g >= n_groups_cap) continue;
    const int64_t w = e % vec_per_group;
    const int64_t src = (bh * kp.n_cap + static_cast<int64_t>(g) * kp.G) * vec_per_row + w;
    const int64_t dst = (bh * kp.top_g + gi) * vec_per_group + w;
    const uint4 kv = Kh[src];
    const uint4 vv = Vh[src];
    Ks[dst] = kv;
    Vs[dst] = vv;
  }
}

hipError_t launch_gather_groups(const GatherArgs& a, hipStream_t st) {
  if (a.kp.top_g <= 0) return hipSuccess;
  dim3 grid((a.kp.top_g + kGroupsPerBlock - 1) / kGroupsPerBlock, a.kp.B * a.kp.Hkv);
  gather_groups_kernel<<<grid, kGatherThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace hga
