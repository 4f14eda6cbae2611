// Device helpers shared by the HGA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hga_kparams.hpp"

namespace hga {

constexpr int kWave = 64;

// Index of the calling wave in its workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave); }

// ---------------------------------------------------------------- bf16 / f32
struct bf16 {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return static_cast<uint16_t>((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T> struct elem;
template <> struct elem<float> {
  static constexpr int bytes = 4;
  __device__ static float get(const float* p, int64_t i) { return p[i]; }
  __device__ static void put(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct elem<bf16> {
  static constexpr int bytes = 2;
  __device__ static float get(const bf16* p, int64_t i) { return bf16_to_f32(p[i].bits); }
  __device__ static void put(bf16* p, int64_t i, float v) { p[i].bits = f32_to_bf16(v); }
};

// Load `N` consecutive elements (N*bytes a multiple of 16, 16-byte aligned) as float.
template <typename T, int N>
__device__ __forceinline__ void load_row(const T* __restrict__ src, float (&dst)[N]) {
  if constexpr (sizeof(T) == 2) {
    static_assert(N % 8 == 0, "bf16 rows load in 16-byte pieces");
    const uint4* s = reinterpret_cast<const uint4*>(src);
#pragma unroll
    for (int v = 0; v < N / 8; ++v) {
      uint4 w = s[v];
      dst[8 * v + 0] = bf16lo(w.x); dst[8 * v + 1] = bf16hi(w.x);
      dst[8 * v + 2] = bf16lo(w.y); dst[8 * v + 3] = bf16hi(w.y);
      dst[8 * v + 4] = bf16lo(w.z); dst[8 * v + 5] = bf16hi(w.z);
      dst[8 * v + 6] = bf16lo(w.w); dst[8 * v + 7] = bf16hi(w.w);
    }
  } else {
    static_assert(N % 4 == 0, "f32 rows load in 16-byte pieces");
    const float4* s = reinterpret_cast<const float4*>(src);
#pragma unroll
    for (int v = 0; v < N / 4; ++v) {
      float4 w = s[v];
      dst[4 * v + 0] = w.x; dst[4 * v + 1] = w.y; dst[4 * v + 2] = w.z; dst[4 * v + 3] = w.w;
    }
  }
}

// Raw 16-byte pieces (kept packed until use).
template <int NV>
struct Raw16 {
  uint4 v[NV];
};

// ---------------------------------------------------------------- DPP lane ops
// Lane exchanges through DPP (within rows of 16 lanes) and the gfx950 permlane
// swaps (across rows), instead of LDS-routed shuffles.
namespace dpp {
constexpr int kRowRor4 = 0x124, kRowRor8 = 0x128;
constexpr int kQuad2301 = 0x4E, kQuad1032 = 0xB1;       // quad_perm [2,3,0,1], [1,0,3,2]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float movf(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int movi(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}
// value of lane n of this lane's row of 16 (DPP row_share, n a constant)
__device__ __forceinline__ float row_share(float v, int n) {
  switch (n & 15) {
    case 0: return movf<0x150>(v);
    case 1: return movf<0x151>(v);
    case 2: return movf<0x152>(v);
    case 3: return movf<0x153>(v);
    case 4: return movf<0x154>(v);
    case 5: return movf<0x155>(v);
    case 6: return movf<0x156>(v);
    case 7: return movf<0x157>(v);
    case 8: return movf<0x158>(v);
    case 9: return movf<0x159>(v);
    case 10: return movf<0x15A>(v);
    case 11: return movf<0x15B>(v);
    case 12: return movf<0x15C>(v);
    case 13: return movf<0x15D>(v);
    case 14: return movf<0x15E>(v);
    default: return movf<0x15F>(v);
  }
}
// value of the same lane in the paired row: xor 16 and xor 32 (results identical
// in both rows of a pair, so "a + other" is the pair's reduction)
__device__ __forceinline__ void swap16(float v, float& a, float& b) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float v, float& a, float& b) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
}  // namespace dpp

// all-reduce over each aligned group of 8 lanes
__device__ __forceinline__ float sum8(float v) {
  v += dpp::movf<dpp::kRowHalfMirror>(v);
  v += dpp::movf<dpp::kQuad2301>(v);
  v += dpp::movf<dpp::kQuad1032>(v);
  return v;
}
// all-reduce over each row of 16 lanes
__device__ __forceinline__ float sum16(float v) {
  v += dpp::movf<dpp::kRowRor8>(v);
  v += dpp::movf<dpp::kRowRor4>(v);
  v += dpp::movf<dpp::kQuad2301>(v);
  v += dpp::movf<dpp::kQuad1032>(v);
  return v;
}
// all-reduce over the 4 rows of the wave (lanes with equal lane%16)
__device__ __forceinline__ float sum_rows(float v) {
  float a, b;
  dpp::swap16(v, a, b);
  v = a + b;
  dpp::swap32(v, a, b);
  return a + b;
}
__device__ __forceinline__ float max_rows(float v) {
  float a, b;
  dpp::swap16(v, a, b);
  v = fmaxf(a, b);
  dpp::swap32(v, a, b);
  return fmaxf(a, b);
}
// all-reduce max / min over the whole wave
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp::movf<dpp::kRowRor8>(v));
  v = fmaxf(v, dpp::movf<dpp::kRowRor4>(v));
  v = fmaxf(v, dpp::movf<dpp::kQuad2301>(v));
  v = fmaxf(v, dpp::movf<dpp::kQuad1032>(v));
  return max_rows(v);
}
__device__ __forceinline__ float wave_min(float v) {
  v = fminf(v, dpp::movf<dpp::kRowRor8>(v));
  v = fminf(v, dpp::movf<dpp::kRowRor4>(v));
  v = fminf(v, dpp::movf<dpp::kQuad2301>(v));
  v = fminf(v, dpp::movf<dpp::kQuad1032>(v));
  float a, b;
  dpp::swap16(v, a, b);
  v = fminf(a, b);
  dpp::swap32(v, a, b);
  return fminf(a, b);
}

// all-reduce over the 32-lane halves (lane pairs of rows 0/1 and 2/3)
__device__ __forceinline__ float sum_rowpair(float v) {
  float a, b;
  dpp::swap16(v, a, b);
  return a + b;
}

// ---------------------------------------------------------------- wave ops
// Inclusive scan of ints across a wave (DPP row shifts, then row broadcasts).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp::movi<dpp::kRowShr1>(v);
  v += dpp::movi<dpp::kRowShr2>(v);
  v += dpp::movi<dpp::kRowShr4>(v);
  v += dpp::movi<dpp::kRowShr8>(v);
  v += dpp::movi<dpp::kRowBcast15, 0xA>(v);
  v += dpp::movi<dpp::kRowBcast31, 0xC>(v);
  return v;
}

// ---------------------------------------------------------------- block scan
// Exclusive prefix sum over the block (NT threads); also returns the total.
template <int NT>
struct BlockScanSmem {
  int wave_tot[NT / kWave];
};

template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int& total, BlockScanSmem<NT>& sm) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  int incl = wave_incl_scan(v);
  if (lane == kWave - 1) sm.wave_tot[wid] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) {
    int t = sm.wave_tot[w];
    before += (w < wid) ? t : 0;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return before + incl - v;
}

// ---------------------------------------------------------------- ordering
// Monotone map score -> u32 (bigger is better).  -0 equals +0; NaN ranks with -inf.
__device__ __forceinline__ uint32_t order_key(float s) {
  if (s != s) s = -__builtin_huge_valf();
  uint32_t b = __float_as_uint(s);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Key unique per candidate and ordered like (score desc, index asc).
__device__ __forceinline__ uint64_t composite_key(float v, int i) {
  return (static_cast<uint64_t>(order_key(v)) << 32) | static_cast<uint32_t>(~i);
}

// ---------------------------------------------------------------- top-k
// Exact selection of the min(k, n) best of sc(0..n) under (score desc, index
// asc).  Writes the selected candidate indices ascending to sel[0..cnt) (LDS or
// global) and returns cnt in every thread.  Every thread of the block must
// call it.
//
// Scores are first bucketed by value over [min, max] of the finite scores
// (the bucket map is monotone, so equal scores share a bucket); one histogram
// finds the bucket that holds the k-th best.  Buckets above it are taken
// whole; inside it the candidates are ranked exactly by (score, index).  When
// that bucket is large (many equal or near-equal scores) a radix select on the
// ordered 32-bit keys finishes the job instead.
template <int NT>
struct TopkSmem {
  unsigned hist[256];
  BlockScanSmem<NT> scan;
  float red[2][NT / kWave];
  float lo, scale;
  unsigned prefix;
  int krem, bucket, above, n_cand;
  uint64_t cand_key[1024];
};

__device__ __forceinline__ float sanitize_score(float s) { return s != s ? -__builtin_huge_valf() : s; }

// radix select on the ordered keys (slow path); returns the threshold key and,
// through krem, how many keys equal to it to take (lowest indices first)
template <int NT, typename ScoreFn>
__device__ unsigned radix_threshold(ScoreFn sc, int n, int k, int& krem_out, TopkSmem<NT>& sm) {
  const int tid = threadIdx.x;
  unsigned prefix = 0u, mask = 0u;
  int krem = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += NT) sm.hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      const unsigned key = order_key(sc(i));
      if ((key & mask) == prefix) atomicAdd(&sm.hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < kWave) {
      unsigned c[4];
      unsigned lsum = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        c[r] = sm.hist[255 - 4 * tid - r];
        lsum += c[r];
      }
      const int incl = wave_incl_scan(static_cast<int>(lsum));
      unsigned above = static_cast<unsigned>(incl) - lsum;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (above < static_cast<unsigned>(krem) && static_cast<unsigned>(krem) <= above + c[r]) {
          sm.prefix = prefix | (static_cast<unsigned>(255 - 4 * tid - r) << shift);
          sm.krem = krem - static_cast<int>(above);
        }
        above += c[r];
      }
    }
    __syncthreads();
    prefix = sm.prefix;
    krem = sm.krem;
    mask |= 255u << shift;
    __syncthreads();
  }
  krem_out = krem;
  return prefix;
}

template <int NT, typename ScoreFn>
__device__ int block_topk(ScoreFn sc_raw, int n, int k, int* sel, TopkSmem<NT>& sm) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  if (k <= 0 || n <= 0) return 0;
  if (n <= k) {
    for (int i = tid; i < n; i += NT) sel[i] = i;
    __syncthreads();
    return n;
  }
  auto sc = [&](int i) { return sanitize_score(sc_raw(i)); };
  // ---- range of the finite scores
  float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
  for (int i = tid; i < n; i += NT) {
    const float v = sc(i);
    if (v > -__builtin_huge_valf() && v < __builtin_huge_valf()) {
      lo = fminf(lo, v);
      hi = fmaxf(hi, v);
    }
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  if (lane == 0) {
    sm.red[0][wid] = lo;
    sm.red[1][wid] = hi;
  }
  for (int i = tid; i < 256; i += NT) sm.hist[i] = 0u;
  __syncthreads();
  if (tid == 0) {
    float l = sm.red[0][0], h = sm.red[1][0];
    for (int w = 1; w < NT / kWave; ++w) {
      l = fminf(l, sm.red[0][w]);
      h = fmaxf(h, sm.red[1][w]);
    }
    sm.lo = l;
    sm.scale = (h > l && h - l < __builtin_huge_valf()) ? 255.99f / (h - l) : 0.f;
    sm.n_cand = 0;
  }
  __syncthreads();
  const float blo = sm.lo, bscale = sm.scale;
  // bucket of a score: monotone non-decreasing in the score
  auto bucket = [&](float v) -> int {
    if (!(v > -__builtin_huge_valf())) return 0;
    const float f = (v - blo) * bscale;
    return f >= 255.f ? 255 : (f > 0.f ? static_cast<int>(f) : 0);
  };
  for (int i = tid; i < n; i += NT) atomicAdd(&sm.hist[bucket(sc(i))], 1u);
  __syncthreads();
  if (tid < kWave) {
    unsigned c[4];
    unsigned lsum = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      c[r] = sm.hist[255 - 4 * tid - r];
      lsum += c[r];
    }
    const int incl = wave_incl_scan(static_cast<int>(lsum));
    unsigned above = static_cast<unsigned>(incl) - lsum;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (above < static_cast<unsigned>(k) && static_cast<unsigned>(k) <= above + c[r]) {
        sm.bucket = 255 - 4 * tid - r;
        sm.above = static_cast<int>(above);
      }
      above += c[r];
    }
  }
  __syncthreads();
  const int bt = sm.bucket;
  const int need = k - sm.above;
  const int n_bt = static_cast<int>(sm.hist[bt]);
  bool fast = n_bt <= 1024;
  unsigned T = 0u;
  int krem = 0;
  if (fast) {
    // candidates of the boundary bucket, ranked exactly
    for (int i = tid; i < n; i += NT) {
      const float v = sc(i);
      if (bucket(v) == bt) sm.cand_key[atomicAdd(&sm.n_cand, 1)] = composite_key(v, i);
    }
    __syncthreads();
  } else {
    T = radix_threshold<NT>(sc, n, k, krem, sm);
  }
  // ---- flags in index order (contiguous ranges per thread), then positions
  const int per = (n + NT - 1) / NT;
  const int b0 = min(n, tid * per), b1 = min(n, b0 + per);
  auto selected = [&](int i, int& eq_seen) -> bool {
    const float v = sc(i);
    if (fast) {
      const int bi = bucket(v);
      if (bi != bt) return bi > bt;
      const uint64_t mine = composite_key(v, i);
      int rank = 0;
      int c = 0;
      for (; c + 16 <= n_bt; c += 16) {
        uint64_t w[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) w[r] = sm.cand_key[c + r];
#pragma unroll
        for (int r = 0; r < 16; ++r) rank += w[r] > mine;
      }
      for (; c < n_bt; ++c) rank += sm.cand_key[c] > mine;
      return rank < need;
    }
    const unsigned key = order_key(v);
    if (key != T) return key > T;
    return eq_seen++ < krem;
  };
  int eq_before = 0;
  if (!fast) {
    int n_eq = 0;
    for (int i = b0; i < b1; ++i) n_eq += order_key(sc(i)) == T;
    int tot;
    eq_before = block_excl_scan<NT>(n_eq, tot, sm.scan);
  }
  int cnt_local = 0;
  {
    int eq_seen = eq_before;
    for (int i = b0; i < b1; ++i) cnt_local += selected(i, eq_seen);
  }
  int tot;
  int pos = block_excl_scan<NT>(cnt_local, tot, sm.scan);
  {
    int eq_seen = eq_before;
    for (int i = b0; i < b1; ++i)
      if (selected(i, eq_seen)) sel[pos++] = i;
  }
  __syncthreads();
  return k;
}

// ---------------------------------------------------------------- cross-workgroup hand-off
// Data that the last workgroup of a unit reads is written and read with
// device-scope (agent) atomic stores/loads, which go past the per-XCD L2 to the
// coherent memory side, so no L2 write-back or invalidate is needed.  Each
// wave waits for its stores to complete before the arrival is counted.
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// s_waitcnt vmcnt(0): this wave's vector memory operations (stores included)
// have completed.  GFX9 encoding: vmcnt = 0, expcnt = 7, lgkmcnt = 15.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Every thread of a workgroup calls this after its st_agent() writes.  One
// thread counts the arrival; the last arriver resets the counter and
// invalidates its caches.  Returns true in every thread of the last
// workgroup, which may then read the others' data with plain loads.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t expected, int* flag_lds) {
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == expected - 1u;
    if (last) {
      __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // drop this CU's and this XCD's cached copies, so that plain loads of the
      // other workgroups' data see memory
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    *flag_lds = last;
  }
  __syncthreads();
  return *flag_lds != 0;
}

// ---------------------------------------------------------------- RoPE helpers
// Rotate (a, b) by angle phi given as (cos, sin).
__device__ __forceinline__ void rot2(float a, float b, float c, float s, float& ra, float& rb) {
  ra = a * c - b * s;
  rb = a * s + b * c;
}

// cos/sin of theta * t for large t, with the angle reduced in double precision.
__device__ __forceinline__ void sincos_abs(double theta, double t, float& s, float& c) {
  const double two_pi = 6.283185307179586476925286766559;
  double ph = theta * t;
  ph -= two_pi * rint(ph / two_pi);
  sincosf(static_cast<float>(ph), &s, &c);
}

}  // namespace hga
