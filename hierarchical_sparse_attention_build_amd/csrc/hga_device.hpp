// Device helpers shared by the HGA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hga_kparams.hpp"

namespace hga {

constexpr int kWave = 64;

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

// ---------------------------------------------------------------- top-k
// Exact selection of the min(k, n) best of sc[0..n) under (score desc, index
// asc), by radix select on the ordered 32-bit key followed by an index-ordered
// tie fill.  Writes the selected candidate indices ascending to sel[0..cnt)
// (sel may be LDS or global) and returns cnt to every thread.  sc may live in
// LDS or global memory.  Every thread of the block must call it.
template <int NT>
struct TopkSmem {
  unsigned hist[256];
  BlockScanSmem<NT> scan;
  unsigned prefix;
  int krem;
};

template <int NT, typename ScoreFn>
__device__ int block_topk(ScoreFn sc, int n, int k, int* sel, TopkSmem<NT>& sm) {
  const int tid = threadIdx.x;
  if (k <= 0 || n <= 0) return 0;
  if (n <= k) {
    for (int i = tid; i < n; i += NT) sel[i] = i;
    __syncthreads();
    return n;
  }
  // ---- radix select: threshold key T and how many keys equal to T to take
  unsigned prefix = 0u, mask = 0u;
  int krem = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += NT) sm.hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      unsigned key = order_key(sc(i));
      if ((key & mask) == prefix) atomicAdd(&sm.hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < kWave) {
      // lane l owns digits 255-4l .. 252-4l (descending)
      unsigned c[4];
      unsigned lsum = 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        c[r] = sm.hist[255 - 4 * tid - r];
        lsum += c[r];
      }
      int incl = wave_incl_scan(static_cast<int>(lsum));
      unsigned above = static_cast<unsigned>(incl) - lsum;  // keys with a larger digit
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
  const unsigned T = prefix;
  // ---- index-ordered fill: contiguous ranges per thread
  const int per = (n + NT - 1) / NT;
  const int b0 = min(n, tid * per), b1 = min(n, b0 + per);
  int n_gt = 0, n_eq = 0;
  for (int i = b0; i < b1; ++i) {
    unsigned key = order_key(sc(i));
    n_gt += key > T;
    n_eq += key == T;
  }
  int tot;
  int eq_before = block_excl_scan<NT>(n_eq, tot, sm.scan);
  int take_eq = max(0, min(n_eq, krem - eq_before));
  int out_before = block_excl_scan<NT>(n_gt + take_eq, tot, sm.scan);
  int pos = out_before, eq_seen = eq_before;
  for (int i = b0; i < b1; ++i) {
    unsigned key = order_key(sc(i));
    bool s = key > T;
    if (key == T) {
      s = eq_seen < krem;
      ++eq_seen;
    }
    if (s) sel[pos++] = i;
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
