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

}  // namespace hga
