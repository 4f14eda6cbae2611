// Warm tier [HGA technical summary (it), Architettura della Memoria: a
// bounded LRU cache in device memory holds the recently routed chunks].  The
// cached unit is the routed group.  The lookup of one (b, kv head) unit, run
// by the workgroup of the routing launch that finishes the unit's lists:
//   * a routed group already cached keeps its slot (a hit; the lowest slot
//     holding it) and the slot's stamp is renewed to this step;
//   * the missing groups take the least recently used slots that this step
//     does not use: the largest keys ~stamp (an empty slot has stamp 0) by
//     the exact ballot selection, which breaks ties towards the lower slot and
//     emits the slots in ascending order; the j-th missing group in list order
//     gets the j-th of them;
//   * list entries outside [0, n_cap / G) are ignored.
// The slot list it writes holds a hit's slot, -2 - slot for a missing group
// (the attention reads its rows from host memory and writes them into that
// slot) and -1 for an ignored entry.
#pragma once

#include "hga_select.hpp"
#include "hga_warm_state.hpp"

namespace hga {

static_assert(kWarmMaxList <= kSelMaxK, "victim selection limit");

struct WarmSmem {
  int tags[kWarmMaxSlots];
  int stamps[kWarmMaxSlots];
  int entry[kWarmMaxList];   // routed group of each list entry (-1 ignored)
  int slot[kWarmMaxList];    // its slot: >= 0 hit or assigned, -1 ignored, -2 missing
  int victim[kWarmMaxList];  // slots taken by the missing groups, ascending
  int n_hit, n_miss;
  int gmap[kWarmMapGroups];  // lowest slot caching each group id (kWarmMaxSlots: none)
};

// Every thread of the workgroup (NT threads) calls this; list (TG entries)
// is readable by all of them.  Ends after its global writes are issued.
template <int NT>
__device__ void warm_lookup_unit(const WarmState w, int64_t bh, int TG, int n_groups_cap, const int* list,
                                 WarmSmem& sm) {
  const int S = w.slots;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = wave_id();
  int32_t* gtags = w.tags + bh * S;
  int32_t* gstamps = w.stamps + bh * S;
  const int now = w.clock[bh] + 1;
  for (int s = tid; s < S; s += NT) {
    sm.tags[s] = gtags[s];
    sm.stamps[s] = gstamps[s];
  }
  for (int i = tid; i < TG; i += NT) {
    const int g = list[i];
    sm.entry[i] = g >= 0 && g < n_groups_cap ? g : -1;
  }
  // ---- hits against the slots as they were before this step
  if (n_groups_cap <= kWarmMapGroups) {
    // indexed by group id: a map from group to its lowest caching slot,
    // built from the tags, then one read per entry
    for (int g = tid; g < n_groups_cap; g += NT) sm.gmap[g] = kWarmMaxSlots;
    __syncthreads();
    for (int s = tid; s < S; s += NT) {
      const int t = sm.tags[s];
      if (t >= 0 && t < n_groups_cap) atomicMin(&sm.gmap[t], s);
    }
    __syncthreads();
    for (int i = tid; i < TG; i += NT) {
      const int g = sm.entry[i];
      sm.slot[i] = g < 0 ? -1 : (sm.gmap[g] < kWarmMaxSlots ? sm.gmap[g] : -2);
    }
  } else {
    __syncthreads();
    // one wave per entry, its lanes comparing 64 slots at a time
    for (int i = wid; i < TG; i += NT / kWave) {
      const int g = sm.entry[i];
      int found = g < 0 ? -1 : -2;
      for (int s0 = 0; s0 < S && g >= 0; s0 += kWave) {
        const uint64_t m = __ballot(s0 + lane < S && sm.tags[s0 + lane] == g);
        if (m) {
          found = s0 + __builtin_ctzll(m);
          break;
        }
      }
      if (lane == 0) sm.slot[i] = found;
    }
  }
  __syncthreads();
  for (int i = tid; i < TG; i += NT)
    if (sm.slot[i] >= 0) sm.stamps[sm.slot[i]] = now;
  __syncthreads();
  // ---- wave 0: count, then take the least recently used free slots
  if (wid == 0) {
    int hits = 0, misses = 0;
    for (int i0 = 0; i0 < TG; i0 += kWave) {
      const int i = i0 + lane;
      const int sl = i < TG ? sm.slot[i] : -1;
      hits += __popcll(__ballot(sl >= 0));
      misses += __popcll(__ballot(sl == -2));
    }
    if (misses > 0) {
      // key of slot s: ~stamp, or 0 (never taken) for a slot this step uses
      wave_topk_n<kSelMaxE>((S + kWave - 1) / kWave,
                  [&](int e) {
                    const int s = e * kWave + lane;
                    const int st = sm.stamps[min(s, S - 1)];
                    return s < S && st != now ? ~static_cast<uint32_t>(st) : 0u;
                  },
                  misses, false, [&](int r, int e, uint32_t) { sm.victim[r] = e * kWave + lane; });
    }
    if (lane == 0) {
      sm.n_hit = hits;
      sm.n_miss = misses;
    }
  }
  __syncthreads();
  // ---- wave 0: the j-th missing entry (list order) takes victim j
  if (wid == 0) {
    int base = 0;
    for (int i0 = 0; i0 < TG; i0 += kWave) {
      const int i = i0 + lane;
      const bool miss = i < TG && sm.slot[i] == -2;
      const uint64_t m = __ballot(miss);
      if (miss) {
        const int j = base + bits_below(m);
        const int v = sm.victim[j];
        sm.slot[i] = -2 - v;  // missing: the attention reads host memory and fills slot v
        sm.tags[v] = sm.entry[i];
        sm.stamps[v] = now;
      }
      base += __popcll(m);
    }
  }
  __syncthreads();
  for (int s = tid; s < S; s += NT) {
    gtags[s] = sm.tags[s];
    gstamps[s] = sm.stamps[s];
  }
  for (int i = tid; i < TG; i += NT) w.slot_of[bh * TG + i] = sm.slot[i];
  if (tid == 0) {
    w.clock[bh] = now;
    if (w.hits) w.hits[bh] = sm.n_hit;
    if (w.misses) w.misses[bh] = sm.n_miss;
  }
}

}  // namespace hga
