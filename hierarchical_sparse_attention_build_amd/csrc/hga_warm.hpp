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
//
// The slots' tags and stamps are staged in LDS (warm_stage_load) while the
// routing still selects, so their loads share a round trip with the routing's
// own; the lookup itself then costs two barriers.
#pragma once

#include "hga_select.hpp"
#include "hga_warm_state.hpp"

namespace hga {

static_assert(kWarmMaxList <= kSelMaxK, "victim selection limit");
static_assert(kWarmMaxList <= kWarmMaxSlots, "a list fits the slots");

// LDS that lives through the routing tail: the unit's slots and its list
struct WarmStage {
  alignas(16) int tags[kWarmMaxSlots];
  int stamps[kWarmMaxSlots];
  int list[kWarmMaxList];  // routed group of each list entry (any value; validated here)
  int slot[kWarmMaxList];  // its slot: >= 0 hit, -1 ignored, -2 missing (then -2 - victim)
  int victim[kWarmMaxList];  // slots taken by the missing groups, ascending
  int now;                   // this step's stamp
};

// Every thread of the workgroup (NT threads) calls this; the stage is ready
// after the caller's next barrier.
template <int NT>
__device__ __forceinline__ void warm_stage_load(const WarmState& w, int64_t bh, WarmStage& st) {
  const int S = w.slots;
  const int32_t* gtags = w.tags + bh * S;
  const int32_t* gstamps = w.stamps + bh * S;
  for (int s = threadIdx.x; s < S; s += NT) {
    st.tags[s] = gtags[s];
    st.stamps[s] = gstamps[s];
  }
  if (threadIdx.x == 0) st.now = w.clock[bh] + 1;
}

// Every thread calls this after a barrier that follows warm_stage_load and
// the writes of st.list[0..TG).  Ends after its global writes are issued.
template <int NT>
__device__ void warm_lookup_unit(const WarmState w, int64_t bh, int TG, int n_groups_cap, WarmStage& st) {
  constexpr int NW = NT / kWave;
  const int S = w.slots;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = wave_id();
  const int now = st.now;
  // ---- hits against the slots as they were before this step: a row of 16
  // lanes per entry, lane r of the row reading tags 64 u + 4 r .. + 3 (16-byte
  // reads, four issued at once) for u = 0, 1, ...; the lowest matching slot is
  // the row's minimum
  {
    const int r = lane & 15;
    const int4* tags4 = reinterpret_cast<const int4*>(st.tags);
    for (int ib = wid * 4; ib < TG; ib += NW * 4) {
      const int i = ib + (lane >> 4);
      int g = -1;
      if (i < TG) {
        const int v = st.list[i];
        g = v >= 0 && v < n_groups_cap ? v : -1;
      }
      int best = kWarmMaxSlots;
      for (int t0 = 0; t0 < S; t0 += 256) {
        int4 t4[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int s0 = t0 + 64 * u + 4 * r;  // s0 + 3 < kWarmMaxSlots when s0 < S
          t4[u] = s0 < S ? tags4[s0 >> 2] : make_int4(-1, -1, -1, -1);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int s0 = t0 + 64 * u + 4 * r;
          int m = kWarmMaxSlots;
          if (t4[u].w == g && s0 + 3 < S) m = s0 + 3;
          if (t4[u].z == g && s0 + 2 < S) m = s0 + 2;
          if (t4[u].y == g && s0 + 1 < S) m = s0 + 1;
          if (t4[u].x == g) m = s0;
          best = min(best, m);
        }
      }
      best = min(best, dpp::movi<dpp::kRowRor8>(best));
      best = min(best, dpp::movi<dpp::kRowRor4>(best));
      best = min(best, dpp::movi<dpp::kQuad2301>(best));
      best = min(best, dpp::movi<dpp::kQuad1032>(best));
      if (r == 0 && i < TG) {
        const int sl = g < 0 ? -1 : (best < kWarmMaxSlots ? best : -2);
        st.slot[i] = sl;
        if (sl >= 0) st.stamps[sl] = now;
      }
    }
  }
  __syncthreads();
  // ---- wave 0: count, take the least recently used free slots, and give the
  // j-th missing entry (list order) victim j
  if (wid == 0) {
    int hits = 0, misses = 0;
    for (int i0 = 0; i0 < TG; i0 += kWave) {
      const int i = i0 + lane;
      const int sl = i < TG ? st.slot[i] : -1;
      hits += __popcll(__ballot(sl >= 0));
      misses += __popcll(__ballot(sl == -2));
    }
    if (misses > 0) {
      // key of slot s: ~stamp, or 0 (never taken) for a slot this step uses;
      // the keys share their top bits, so the search starts below them
      wave_topk_n<kSelMaxE, true>((S + kWave - 1) / kWave,
                  [&](int e) {
                    const int s = e * kWave + lane;
                    const int stv = st.stamps[min(s, S - 1)];
                    return s < S && stv != now ? ~static_cast<uint32_t>(stv) : 0u;
                  },
                  misses, false, [&](int r, int e, uint32_t) { st.victim[r] = e * kWave + lane; });
      int base = 0;
      for (int i0 = 0; i0 < TG; i0 += kWave) {
        const int i = i0 + lane;
        const int g = i < TG ? st.list[i] : -1;
        const bool miss = i < TG && st.slot[i] == -2;
        const uint64_t m = __ballot(miss);
        if (miss) {
          const int v = st.victim[base + bits_below(m)];
          st.slot[i] = -2 - v;  // missing: the attention reads host memory and fills slot v
          st.tags[v] = g;
          st.stamps[v] = now;
        }
        base += __popcll(m);
      }
    }
    if (lane == 0) {
      w.clock[bh] = now;
      if (w.hits) w.hits[bh] = hits;
      if (w.misses) w.misses[bh] = misses;
    }
  }
  __syncthreads();
  int32_t* gtags = w.tags + bh * S;
  int32_t* gstamps = w.stamps + bh * S;
  for (int s = tid; s < S; s += NT) {
    gtags[s] = st.tags[s];
    gstamps[s] = st.stamps[s];
  }
  for (int i = tid; i < TG; i += NT) w.slot_of[bh * TG + i] = st.slot[i];
}

}  // namespace hga
