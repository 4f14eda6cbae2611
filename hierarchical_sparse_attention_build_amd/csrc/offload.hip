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

static_assert(hga::kWarmMaxList <= hga::kSelMaxK, "victim selection limit");

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

// ---------------------------------------------------------------------------
// Warm tier [HGA technical summary (it), Architettura della Memoria: a bounded
// LRU cache in device memory holds the recently routed chunks].  The cached
// unit is the routed group.  One workgroup per (b, kv head):
//   * a routed group already cached keeps its slot (a hit; the lowest slot
//     holding it) and the slot's stamp is renewed to this step;
//   * the missing groups take the least recently used slots that this step
//     does not use: the largest keys ~stamp (an empty slot has stamp 0) by
//     the exact ballot selection, which breaks ties towards the lower slot and
//     emits the slots in ascending order; the j-th missing group in list order
//     gets the j-th of them;
//   * list entries outside [0, n_cap / G) are ignored.
constexpr int kWarmThreads = 256;
constexpr int kWarmMapGroups = 8192;  // contexts of up to this many groups per (b, kv head) use the LDS map

__global__ __launch_bounds__(kWarmThreads) void warm_lookup_kernel(WarmArgs a) {
  const KParams& kp = a.kp;
  const int64_t bh = blockIdx.x;
  const int S = a.slots;
  const int TG = kp.top_g;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = wave_id();
  const int n_groups_cap = static_cast<int>(kp.n_cap / kp.G);
  __shared__ int tags[kWarmMaxSlots];
  __shared__ int stamps[kWarmMaxSlots];
  __shared__ int entry[kWarmMaxList];   // routed group of each list entry (-1 ignored)
  __shared__ int slot[kWarmMaxList];    // its slot: >= 0 hit or assigned, -1 ignored, -2 missing
  __shared__ int victim[kWarmMaxList];  // slots taken by the missing groups, ascending
  __shared__ int n_hit, n_miss;
  __shared__ int gmap[kWarmMapGroups];  // lowest slot caching each group id (kWarmMaxSlots: none)

  int32_t* gtags = a.tags + bh * S;
  int32_t* gstamps = a.stamps + bh * S;
  const int now = a.clock[bh] + 1;
  for (int s = tid; s < S; s += kWarmThreads) {
    tags[s] = gtags[s];
    stamps[s] = gstamps[s];
  }
  for (int i = tid; i < TG; i += kWarmThreads) {
    const int g = a.group_idx[bh * TG + i];
    entry[i] = g >= 0 && g < n_groups_cap ? g : -1;
  }
  // ---- hits against the slots as they were before this step
  if (n_groups_cap <= kWarmMapGroups) {
    // indexed by group id: a map from group to its lowest caching slot,
    // built from the tags, then one read per entry
    for (int g = tid; g < n_groups_cap; g += kWarmThreads) gmap[g] = kWarmMaxSlots;
    __syncthreads();
    for (int s = tid; s < S; s += kWarmThreads) {
      const int t = tags[s];
      if (t >= 0 && t < n_groups_cap) atomicMin(&gmap[t], s);
    }
    __syncthreads();
    for (int i = tid; i < TG; i += kWarmThreads) {
      const int g = entry[i];
      slot[i] = g < 0 ? -1 : (gmap[g] < kWarmMaxSlots ? gmap[g] : -2);
    }
  } else {
    __syncthreads();
    // one wave per entry, its lanes comparing 64 slots at a time
    for (int i = wid; i < TG; i += kWarmThreads / kWave) {
      const int g = entry[i];
      int found = g < 0 ? -1 : -2;
      for (int s0 = 0; s0 < S && g >= 0; s0 += kWave) {
        const uint64_t m = __ballot(s0 + lane < S && tags[s0 + lane] == g);
        if (m) {
          found = s0 + __builtin_ctzll(m);
          break;
        }
      }
      if (lane == 0) slot[i] = found;
    }
  }
  __syncthreads();
  for (int i = tid; i < TG; i += kWarmThreads)
    if (slot[i] >= 0) stamps[slot[i]] = now;
  __syncthreads();
  // ---- wave 0: count, then take the least recently used free slots
  if (wid == 0) {
    int hits = 0, misses = 0;
    for (int i0 = 0; i0 < TG; i0 += kWave) {
      const int i = i0 + lane;
      const int sl = i < TG ? slot[i] : -1;
      hits += __popcll(__ballot(sl >= 0));
      misses += __popcll(__ballot(sl == -2));
    }
    if (misses > 0) {
      // key of slot s: ~stamp, or 0 (never taken) for a slot this step uses
      wave_topk_n<kSelMaxE>((S + kWave - 1) / kWave,
                  [&](int e) {
                    const int s = e * kWave + lane;
                    const int st = stamps[min(s, S - 1)];
                    return s < S && st != now ? ~static_cast<uint32_t>(st) : 0u;
                  },
                  misses, false, [&](int r, int e, uint32_t) { victim[r] = e * kWave + lane; });
    }
    if (lane == 0) {
      n_hit = hits;
      n_miss = misses;
    }
  }
  __syncthreads();
  // ---- wave 0: the j-th missing entry (list order) takes victim j
  if (wid == 0) {
    int base = 0;
    for (int i0 = 0; i0 < TG; i0 += kWave) {
      const int i = i0 + lane;
      const bool miss = i < TG && slot[i] == -2;
      const uint64_t m = __ballot(miss);
      if (miss) {
        const int j = base + bits_below(m);
        const int v = victim[j];
        slot[i] = -2 - v;  // missing: the attention reads host memory and fills slot v
        tags[v] = entry[i];
        stamps[v] = now;
      }
      base += __popcll(m);
    }
  }
  __syncthreads();
  for (int s = tid; s < S; s += kWarmThreads) {
    gtags[s] = tags[s];
    gstamps[s] = stamps[s];
  }
  for (int i = tid; i < TG; i += kWarmThreads) a.slot_of[bh * TG + i] = slot[i];
  if (tid == 0) {
    a.clock[bh] = now;
    if (a.hits) a.hits[bh] = n_hit;
    if (a.misses) a.misses[bh] = n_miss;
  }
}

hipError_t launch_warm_lookup(const WarmArgs& a, hipStream_t st) {
  if (a.kp.top_g <= 0) return hipSuccess;
  if (a.slots < a.kp.top_g || a.slots > kWarmMaxSlots || a.kp.top_g > kWarmMaxList) return hipErrorInvalidValue;
  warm_lookup_kernel<<<a.kp.B * a.kp.Hkv, kWarmThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace hga
