// Device routine that summarises one chunk; used by the summary kernel and by
// the decode routing kernel (which keeps the tables current as chunks complete).
//
// [HGA technical summary (it), Meccanismo Core, item 3]: high-frequency RoPE
// pairs are rotated per token before the mean; low-frequency pairs are averaged
// in raw key space and rotated to the span's representative position (its
// centre).  Built from the existing projected keys only.
//
// Work item (pair i, group g) sums the G tokens of group g for pair i, giving
// the group summary; the chunk summary is combined from the m group sums in LDS:
//   high-frequency pair: chunk mean = mean of the group means;
//   low-frequency pair:  chunk = mean over groups of the group summary turned by
//                        theta_i * (p_chunk - p_group)  (rotations compose).
// The same combine holds for post-RoPE and raw keys.
#pragma once

#include "hga_device.hpp"

namespace hga {

// Summaries of chunk `c` whose C rows start at `Kc` (row stride d elements).
// rotated: rows are post-RoPE keys (relative-angle form, small angles only);
// otherwise raw keys (absolute angles reduced in double); krot (nullable, raw
// mode only) receives the RoPE'd rows.
template <typename T, int D>
__device__ void summarize_chunk(const T* __restrict__ Kc, int c, const KParams& kp, bool rotated,
                                T* __restrict__ krot, float* __restrict__ cs_out,
                                float* gs_out) {
  constexpr int P = D / 2;
  const int C = kp.C, G = kp.G, m = kp.m;
  const float invG = 1.0f / static_cast<float>(G);
  const float gcen = 0.5f * static_cast<float>(G - 1);
  for (int w = threadIdx.x; w < P * m; w += blockDim.x) {
    const int i = w % P;
    const int g = w / P;
    const bool hf = (kp.hf_mask >> i) & 1ull;
    const float th = kp.theta_f[i];
    float sa = 0.f, sb = 0.f;
    for (int r = 0; r < G; ++r) {
      const int row = g * G + r;
      const float a = elem<T>::get(Kc, static_cast<int64_t>(row) * D + i);
      const float b = elem<T>::get(Kc, static_cast<int64_t>(row) * D + i + P);
      if (rotated) {
        if (hf) {
          sa += a;
          sb += b;
        } else {
          float s, co;
          sincosf(th * (gcen - static_cast<float>(r)), &s, &co);
          float ra, rb;
          rot2(a, b, co, s, ra, rb);
          sa += ra;
          sb += rb;
        }
      } else {
        const double t = static_cast<double>(c) * C + row;
        float ra = a, rb = b;
        if (hf || krot) {
          float s, co;
          sincos_abs(kp.theta_d[i], t, s, co);
          rot2(a, b, co, s, ra, rb);
          if (krot) {
            elem<T>::put(krot, static_cast<int64_t>(row) * D + i, ra);
            elem<T>::put(krot, static_cast<int64_t>(row) * D + i + P, rb);
          }
        }
        if (hf) {
          sa += ra;
          sb += rb;
        } else {
          sa += a;
          sb += b;
        }
      }
    }
    sa *= invG;
    sb *= invG;
    if (!rotated && !hf) {  // raw mean -> representative position of the group
      float s, co;
      const double pg = static_cast<double>(c) * C + g * G + 0.5 * (G - 1);
      sincos_abs(kp.theta_d[i], pg, s, co);
      float ra, rb;
      rot2(sa, sb, co, s, ra, rb);
      sa = ra;
      sb = rb;
    }
    gs_out[static_cast<int64_t>(g) * D + i] = sa;
    gs_out[static_cast<int64_t>(g) * D + i + P] = sb;
  }
  __threadfence_block();
  __syncthreads();
  const float invm = 1.0f / static_cast<float>(m);
  const float ccen = 0.5f * static_cast<float>(C - 1);
  for (int i = threadIdx.x; i < P; i += blockDim.x) {
    const bool hf = (kp.hf_mask >> i) & 1ull;
    const float th = kp.theta_f[i];
    float sa = 0.f, sb = 0.f;
    for (int g = 0; g < m; ++g) {
      const float a = gs_out[g * D + i], b = gs_out[g * D + i + P];
      if (hf) {
        sa += a;
        sb += b;
      } else {
        float s, co;
        sincosf(th * (ccen - (static_cast<float>(g * G) + gcen)), &s, &co);
        float ra, rb;
        rot2(a, b, co, s, ra, rb);
        sa += ra;
        sb += rb;
      }
    }
    cs_out[i] = sa * invm;
    cs_out[i + P] = sb * invm;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Fast path for bf16 post-RoPE keys (C <= 64, G a multiple of the rows that
// one 64-lane load covers): the same arithmetic as above, with 8-byte row
// loads, one wave per group, and the rotation angles read from tables:
//   rot[r * P + i]  = (cos, sin) of theta_i * (gcen - r)         for r < G,
//   crot[g * P + i] = (cos, sin) of theta_i * (ccen - gcen_g)     for g < m,
// the identity for high-frequency pairs.  A lane loads both halves of four
// pairs of a row (dimensions 4 q .. 4 q + 3 and the same plus P, two 8-byte
// loads), so it rotates them with no exchange between lanes.

template <int D>
__host__ __device__ constexpr int summarize_rows_per_load() { return kWave / (D / 8); }

// LDS floats the fast path needs: both tables (float2) and the group means
__host__ __device__ inline int summarize_lds_floats(const KParams& kp) {
  return 2 * (kp.G + kp.m) * (kp.d / 2) + kp.m * kp.d;
}

template <int D>
__host__ __device__ inline bool summarize_fast_ok(const KParams& kp, bool bf16_in, bool rotated, int lds_floats) {
  return bf16_in && rotated && kp.d == D && kp.C <= 64 && kp.G % summarize_rows_per_load<D>() == 0 &&
         summarize_lds_floats(kp) <= lds_floats;
}

// All threads of the workgroup build the tables (ends with a barrier).  The
// offsets are symmetric: gcen - r and gcen - (G - 1 - r) are exact negatives
// (small multiples of 1/2), and so are the chunk offsets of groups g and
// m - 1 - g, so one sincos serves both entries (the sine changes sign).
template <int D>
__device__ void build_summary_tables(const KParams& kp, float2* rot, float2* crot) {
  constexpr int P = D / 2;
  const float gcen = 0.5f * static_cast<float>(kp.G - 1);
  const float ccen = 0.5f * static_cast<float>(kp.C - 1);
  const int hr = (kp.G + 1) / 2, hg = (kp.m + 1) / 2;
  for (int x = threadIdx.x; x < hr * P; x += blockDim.x) {
    const int r = x / P, i = x % P;
    float sn = 0.f, cn = 1.f;
    if (!((kp.hf_mask >> i) & 1ull)) sincosf(kp.theta_f[i] * (gcen - static_cast<float>(r)), &sn, &cn);
    rot[r * P + i] = make_float2(cn, sn);
    const int rm = kp.G - 1 - r;
    if (rm != r) rot[rm * P + i] = make_float2(cn, -sn);
  }
  for (int x = threadIdx.x; x < hg * P; x += blockDim.x) {
    const int g = x / P, i = x % P;
    float sn = 0.f, cn = 1.f;
    if (!((kp.hf_mask >> i) & 1ull))
      sincosf(kp.theta_f[i] * (ccen - (static_cast<float>(g * kp.G) + gcen)), &sn, &cn);
    crot[g * P + i] = make_float2(cn, sn);
    const int gm = kp.m - 1 - g;
    if (gm != g) crot[gm * P + i] = make_float2(cn, -sn);
  }
  __syncthreads();
}

// Sum over the lanes that hold the same columns (different rows).
template <int D>
__device__ __forceinline__ float sum_row_lanes(float v) {
  if constexpr (D == 64) v += dpp::movf<dpp::kRowRor8>(v);
  return sum_rows(v);
}

// The rows of one group that this lane loads, MAXL rows at most (G <= MAXL
// rows per load): four values of the first half and the same four of the
// second half of each row.
template <int D, int MAXL>
struct GroupRows {
  uint2 lo[MAXL];
  uint2 hi[MAXL];
};

template <int D, int MAXL>
__device__ __forceinline__ void load_group_rows(const bf16* __restrict__ Kc, const KParams& kp, int g,
                                                GroupRows<D, MAXL>& rows) {
  constexpr int P = D / 2;
  constexpr int LR = D / 8;  // lanes per row, four pairs each
  constexpr int RPI = summarize_rows_per_load<D>();
  const int lane = threadIdx.x & (kWave - 1);
  const int pc = lane % LR, ro = lane / LR;
  const int spg = kp.G / RPI;
#pragma unroll
  for (int s = 0; s < MAXL; ++s) {
    if (s < spg) {
      const bf16* r = Kc + static_cast<int64_t>(g * kp.G + s * RPI + ro) * D + 4 * pc;
      rows.lo[s] = *reinterpret_cast<const uint2*>(r);
      rows.hi[s] = *reinterpret_cast<const uint2*>(r + P);
    }
  }
}

// One wave: group g's mean from its loaded rows, into gs_out (global) and
// gmean (LDS, [m][D]).  Pair i = 4 pc + j of a row with offset r becomes
// (a c - b s, a s + b c), (c, s) = rot[r * P + i].
template <int D, int MAXL>
__device__ __forceinline__ void group_mean_wave(const GroupRows<D, MAXL>& rows, const KParams& kp, const float2* rot,
                                                int g, float* __restrict__ gs_out, float* gmean) {
  constexpr int P = D / 2;
  constexpr int LR = D / 8;
  constexpr int RPI = summarize_rows_per_load<D>();
  const int lane = threadIdx.x & (kWave - 1);
  const int pc = lane % LR, ro = lane / LR;
  const int i0 = 4 * pc;
  const int spg = kp.G / RPI;
  float ra[4], rb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) ra[j] = rb[j] = 0.f;
#pragma unroll
  for (int s = 0; s < MAXL; ++s) {
    if (s < spg) {
      const float4* tr = reinterpret_cast<const float4*>(rot + (s * RPI + ro) * P + i0);
      const float4 t01 = tr[0], t23 = tr[1];  // (c, s) of pairs i0 .. i0 + 3
      const float a[4] = {bf16lo(rows.lo[s].x), bf16hi(rows.lo[s].x), bf16lo(rows.lo[s].y), bf16hi(rows.lo[s].y)};
      const float b[4] = {bf16lo(rows.hi[s].x), bf16hi(rows.hi[s].x), bf16lo(rows.hi[s].y), bf16hi(rows.hi[s].y)};
      const float c[4] = {t01.x, t01.z, t23.x, t23.z};
      const float sn[4] = {t01.y, t01.w, t23.y, t23.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ra[j] = fmaf(a[j], c[j], fmaf(-b[j], sn[j], ra[j]));
        rb[j] = fmaf(b[j], c[j], fmaf(a[j], sn[j], rb[j]));
      }
    }
  }
  const float invG = 1.0f / static_cast<float>(kp.G);
  float ga[4], gb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ga[j] = sum_row_lanes<D>(ra[j]) * invG;
    gb[j] = sum_row_lanes<D>(rb[j]) * invG;
  }
  if (ro == 0) {
    const float4 va = make_float4(ga[0], ga[1], ga[2], ga[3]), vb = make_float4(gb[0], gb[1], gb[2], gb[3]);
    float* go = gs_out + static_cast<int64_t>(g) * D + i0;
    *reinterpret_cast<float4*>(go) = va;
    *reinterpret_cast<float4*>(go + P) = vb;
    float* gl = gmean + g * D + i0;
    *reinterpret_cast<float4*>(gl) = va;
    *reinterpret_cast<float4*>(gl + P) = vb;
  }
}

// The chunk summary from the group means in LDS (after a barrier): the mean
// over groups of each group's mean turned to the chunk centre.
template <int D>
__device__ void combine_chunk(const KParams& kp, const float2* crot, const float* gmean, float* __restrict__ cs_out) {
  constexpr int P = D / 2;
  const float invm = 1.0f / static_cast<float>(kp.m);
  for (int i = threadIdx.x; i < P; i += blockDim.x) {
    float sa = 0.f, sb = 0.f;
    for (int g = 0; g < kp.m; ++g) {
      const float a = gmean[g * D + i], b = gmean[g * D + i + P];
      const float2 t = crot[g * P + i];
      float ra, rb;
      rot2(a, b, t.x, t.y, ra, rb);
      sa += ra;
      sb += rb;
    }
    cs_out[i] = sa * invm;
    cs_out[i + P] = sb * invm;
  }
}

// Loads per lane of one group on the fast path: 4 covers G <= 16 (d = 128) and
// G <= 32 (d = 64); 16 covers every G <= 64.
template <int D>
__host__ __device__ inline int summarize_loads_per_group(const KParams& kp) {
  return kp.G / summarize_rows_per_load<D>() <= 4 ? 4 : 16;
}

// The whole workgroup: chunk and group summaries of the chunk at Kc, with the
// LDS area lds (summarize_lds_floats(kp) floats, 16-byte aligned).  Each wave
// issues the loads of its first group before the tables are built.  Ends with
// the summaries written (no barrier after the last store).
template <int D, int MAXL>
__device__ void summarize_chunk_fast(const bf16* __restrict__ Kc, const KParams& kp, float* lds,
                                     float* __restrict__ cs_out, float* __restrict__ gs_out) {
  float2* rot = reinterpret_cast<float2*>(lds);
  float2* crot = rot + kp.G * (D / 2);
  float* gmean = reinterpret_cast<float*>(crot + kp.m * (D / 2));
  const int wid = wave_id(), nw = static_cast<int>(blockDim.x) / kWave;
  GroupRows<D, MAXL> rows;
  if (wid < kp.m) load_group_rows<D, MAXL>(Kc, kp, wid, rows);
  build_summary_tables<D>(kp, rot, crot);
  for (int g = wid; g < kp.m; g += nw) {
    if (g != wid) load_group_rows<D, MAXL>(Kc, kp, g, rows);
    group_mean_wave<D, MAXL>(rows, kp, rot, g, gs_out, gmean);
  }
  __syncthreads();
  combine_chunk<D>(kp, crot, gmean, cs_out);
}

}  // namespace hga
