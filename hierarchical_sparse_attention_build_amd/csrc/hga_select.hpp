// Exact top-k selection by a bitwise search on ordered keys, done by whole
// waves with ballots, without a barrier inside the search.
//
// Order of candidates: score descending, then position ascending (lower
// position wins a tie); NaN ranks with -inf.  The selected positions come out
// in ascending order, which is the order of the index lists the method hands
// from one routing level to the next and to the attention step
// [HGA technical summary (it), Meccanismo Core, item 2].
//
// A wave holds up to kSelMaxE keys per lane.  The k-th largest key T is found
// bit by bit from the top: a candidate prefix is kept when at least k keys are
// >= it (each count is a ballot and a population count per key slot, so the
// search runs on the scalar unit once the compares are done).  The
// selection is every key > T plus the lowest positions among the keys == T.
// A workgroup first lets each wave select the best min(k, its share) of a
// contiguous share of the list (a member of the overall top-k is in the
// top-k of its share), then one wave selects among those.
#pragma once

#include "hga_device.hpp"

namespace hga {

constexpr int kSelMaxE = 16;   // keys per lane in one wave search
constexpr int kSelMaxK = 256;  // largest k of the workgroup selection

// number of set bits of m at lanes below this one
__device__ __forceinline__ int bits_below(uint64_t m) {
  return static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                    __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u)));
}

__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

// OR and AND of v over the whole wave (every lane gets both)
__device__ __forceinline__ void wave_or_and(uint32_t& o, uint32_t& a) {
  using namespace dpp;
  o |= static_cast<uint32_t>(movi<kRowRor8>(static_cast<int>(o)));
  a &= static_cast<uint32_t>(movi<kRowRor8>(static_cast<int>(a)));
  o |= static_cast<uint32_t>(movi<kRowRor4>(static_cast<int>(o)));
  a &= static_cast<uint32_t>(movi<kRowRor4>(static_cast<int>(a)));
  o |= static_cast<uint32_t>(movi<kQuad2301>(static_cast<int>(o)));
  a &= static_cast<uint32_t>(movi<kQuad2301>(static_cast<int>(a)));
  o |= static_cast<uint32_t>(movi<kQuad1032>(static_cast<int>(o)));
  a &= static_cast<uint32_t>(movi<kQuad1032>(static_cast<int>(a)));
  auto r = __builtin_amdgcn_permlane16_swap(o, o, false, false);
  o = r[0] | r[1];
  r = __builtin_amdgcn_permlane16_swap(a, a, false, false);
  a = r[0] & r[1];
  r = __builtin_amdgcn_permlane32_swap(o, o, false, false);
  o = r[0] | r[1];
  r = __builtin_amdgcn_permlane32_swap(a, a, false, false);
  a = r[0] & r[1];
}

// Valid keys are order_key() values (always >= 0x007fffff); an empty slot holds 0.
// Returns the largest T with #{keys >= T} >= k, for 1 <= k <= number of valid keys
// (the k-th largest key, or a value with exactly k keys at or above it).
//
// With Prefix set, the search starts below the keys' common prefix: the bits
// above the highest bit in which two valid keys differ are the same in every
// valid key, and a greedy search from bit 31 would set exactly those of them
// that the keys have (each such step counts every valid key, or none).  The
// selection that follows (keys > T, then ties) is the same as the full
// search's.  It pays for keys that share many top bits (small integers under
// a complement); scores of mixed sign differ in bit 31 already.
template <int E, bool Prefix = false>
__device__ __forceinline__ uint32_t wave_kth_key(const uint32_t (&key)[E], int k) {
  uint32_t T = 0u;
  int top = 31;
  if constexpr (Prefix) {
    uint32_t o = 0u, a = ~0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      o |= key[e];
      a &= key[e] != 0u ? key[e] : ~0u;
    }
    wave_or_and(o, a);
    o = __builtin_amdgcn_readfirstlane(o);
    a = __builtin_amdgcn_readfirstlane(a);
    const uint32_t diff = o ^ a;  // no valid key holds a bit that the AND lacks above this
    if (diff == 0u) return a;     // every valid key is equal
    top = 31 - __builtin_clz(diff);
    T = top == 31 ? 0u : (a & ~((2u << top) - 1u));
  }
  for (int bit = top; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    int c = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) c += __popcll(ballot64(key[e] >= cand));
    if (c >= k) {
      T = cand;
      if (c == k) break;
    }
  }
  return T;
}

// Emit the k selected slots (keys > T, then the first keys == T in slot order)
// as out(rank, e, key) in ascending slot order, slot order being (e, lane).
template <int E, typename OutFn>
__device__ __forceinline__ void wave_emit(const uint32_t (&key)[E], int k, uint32_t T, OutFn out) {
  int n_gt = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) n_gt += __popcll(ballot64(key[e] > T));
  int need = k - n_gt;
  int base = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool is_eq = key[e] == T;
    const uint64_t eq = ballot64(is_eq);
    const bool take = key[e] > T || (is_eq && bits_below(eq) < need);
    const uint64_t tm = ballot64(take);
    if (take) out(base + bits_below(tm), e, key[e]);
    base += __popcll(tm);
    const int neq = __popcll(eq);
    need -= need < neq ? need : neq;
  }
}

// Emit every valid slot (key != 0) in slot order, as out(rank, e, key).
template <int E, typename OutFn>
__device__ __forceinline__ void wave_emit_all(const uint32_t (&key)[E], OutFn out) {
  int base = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool take = key[e] != 0u;
    const uint64_t tm = ballot64(take);
    if (take) out(base + bits_below(tm), e, key[e]);
    base += __popcll(tm);
  }
}

// One wave: keys key_of(e) for slots (e, lane), e < E; emit the best k
// (every valid key when all is set) through out(rank, e, key).
template <int E, bool Prefix = false, typename KeyFn, typename OutFn>
__device__ __forceinline__ void wave_topk(KeyFn key_of, int k, bool all, OutFn out) {
  uint32_t key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) key[e] = key_of(e);
  if (all) {
    wave_emit_all(key, out);
  } else if (k > 0) {
    const uint32_t T = wave_kth_key<E, Prefix>(key, k);
    wave_emit(key, k, T, out);
  }
}

// wave_topk with the slot count rounded up to 1, 2, 4, 8 or 16 (at most
// MaxE, a power of two <= kSelMaxE; slots <= MaxE).  Only the variants up to
// MaxE are compiled: a kernel that inlines the 8- and 16-slot ones needs more
// scalar registers at its peak, and the excess spills to vector lanes with
// reloads all over the kernel.
template <int MaxE, bool Prefix = false, typename KeyFn, typename OutFn>
__device__ __forceinline__ void wave_topk_n(int slots, KeyFn key_of, int k, bool all, OutFn out) {
  static_assert(MaxE >= 2 && MaxE <= kSelMaxE && (MaxE & (MaxE - 1)) == 0, "MaxE: 2, 4, 8 or 16");
  if (slots <= 0) return;
  if (slots <= 1) {
    wave_topk<1, Prefix>(key_of, k, all, out);
  } else if (MaxE == 2 || slots <= 2) {
    wave_topk<2, Prefix>(key_of, k, all, out);
  } else if constexpr (MaxE >= 4) {
    if (MaxE == 4 || slots <= 4) {
      wave_topk<4, Prefix>(key_of, k, all, out);
    } else if constexpr (MaxE >= 8) {
      if (MaxE == 8 || slots <= 8) wave_topk<8, Prefix>(key_of, k, all, out);
      else wave_topk<kSelMaxE, Prefix>(key_of, k, all, out);
    }
  }
}

template <int NT, int MK = kSelMaxK>
struct SelSmem {
  static constexpr int NW = NT / kWave;
  uint32_t key[NW * MK];
  int pos[NW * MK];
};

// True when block_select<NT, MaxE, MK> handles (n, k): k <= MK and at most
// MaxE keys per lane in either phase.  Monotone in n: it holds for every
// smaller n as well.
template <int NT, int MaxE = kSelMaxE, int MK = kSelMaxK>
__host__ __device__ constexpr bool block_select_fits(int n, int k) {
  constexpr int NW = NT / kWave;
  if (k > MK) return false;
  if (n <= k || n <= 2 * kWave) return true;  // nothing to select, or one wave with two keys per lane
  const int q = (n + NW - 1) / NW;
  return q <= kWave * MaxE && NW * (k < q ? k : q) <= kWave * MaxE;
}

// Exact selection of the min(n, k) best of sc(0..n) (sc reads LDS or memory);
// the chosen positions go to sel[] (LDS) in ascending order.  Every thread of
// the workgroup calls it; returns min(n, k) and ends with a barrier.
// Requires block_select_fits<NT, MaxE, MK>(n, k).
template <int NT, int MaxE = kSelMaxE, int MK = kSelMaxK, typename ScoreFn>
__device__ int block_select(ScoreFn sc, int n, int k, int* sel, SelSmem<NT, MK>& sm) {
  constexpr int NW = NT / kWave;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = wave_id();
  if (n <= k) {
    for (int i = tid; i < n; i += NT) sel[i] = i;
    __syncthreads();
    return n;
  }
  // key of position i (0 outside [0, hi)); the read index is clamped, so every
  // lane reads and no lane branches
  auto key_at = [&](int i, int hi) -> uint32_t {
    const uint32_t kk = order_key(sc(min(i, hi - 1)));
    return i < hi ? kk : 0u;
  };
  if (n <= 2 * kWave) {
    // one wave, at most two keys per lane
    if (wid == 0)
      wave_topk_n<MaxE>((n + kWave - 1) / kWave, [&](int e) { return key_at(e * kWave + lane, n); }, k, false,
                  [&](int r, int e, uint32_t) { sel[r] = e * kWave + lane; });
    __syncthreads();
    return k;
  }

  // phase 1: wave w selects min(k, its share) among positions [w*q, min(n, (w+1)*q))
  // and writes them, in ascending position order, after the earlier waves'
  // winners (their counts are known to every wave), so the winners lie end to end
  const int q = (n + NW - 1) / NW;
  const int lo = wid * q;
  const int hi = min(n, lo + q);
  const int nw = max(0, hi - lo);
  const int kw = min(k, nw);
  // with n > 128 and at most 16 waves, every wave but the last has a full share q
  const int start = min(k, q) * wid;
  wave_topk_n<MaxE>((nw + kWave - 1) / kWave, [&](int e) { return key_at(lo + e * kWave + lane, hi); }, kw, kw == nw,
              [&](int r, int e, uint32_t kk) {
                sm.key[start + r] = kk;
                sm.pos[start + r] = lo + e * kWave + lane;
              });
  __syncthreads();

  // phase 2: wave 0 selects k among the winners (ascending positions)
  if (wid == 0) {
    const int n2 = min(k, q) * (NW - 1) + min(k, max(0, n - (NW - 1) * q));
    wave_topk_n<MaxE>((n2 + kWave - 1) / kWave,
                [&](int e) {
                  const int jj = e * kWave + lane;
                  const uint32_t kk = sm.key[min(jj, n2 - 1)];
                  return jj < n2 ? kk : 0u;
                },
                k, n2 <= k, [&](int r, int e, uint32_t) { sel[r] = sm.pos[e * kWave + lane]; });
  }
  __syncthreads();
  return k;
}

}  // namespace hga
