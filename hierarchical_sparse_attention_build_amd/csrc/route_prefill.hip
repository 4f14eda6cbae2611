// Steps 2-3 of HGA for prefill on the matrix cores: two-level routing of one
// unit (a query chunk of C = 64 positions x the query heads of a KV head).
// [HGA technical summary (it), Meccanismo Core, item 2, first two bullets].
//
// Scores are a dense contraction: for every candidate chunk c,
//   score(c) = max over the unit's query rows of q . s_c / sqrt(d).
// With 32x32x16 MFMAs a wave computes D = Q_w S^T for its 32 query rows
// against a tile of 32 summaries: lane = summary column, the 16 accumulators
// of a lane are 16 query rows, so the max over queries is lane-local (plus the
// partner half-wave and the other waves through LDS).  Q is exact in bf16;
// the fp32 summaries are split as s = hi + lo with hi = bf16(s) and
// lo = bf16(s - hi) and both products accumulate in fp32 (relative error of
// the split about 2^-17).  Summary tiles are converted once per workgroup
// into LDS.  Top-k on the chunk scores, then the same contraction over the
// C/G groups of every routed chunk and a top-g.
#include "hga_device.hpp"
#include "hga_kernels.hpp"

namespace hga {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kRTile = 32;  // summaries per tile

template <int D, int NW>
struct RoutePrefillSmem {
  static constexpr int ROW = D * 2 + 16;  // bytes per bf16 row (padded)
  alignas(16) unsigned char hi[2][kRTile * ROW];
  alignas(16) unsigned char lo[2][kRTile * ROW];
  float wmax[NW][kRTile];
  float scores[1024 * 4];   // chunk scores of the unit, then group scores
  int sel_chunks[1024];
  int sel_groups[1024];
  RankSmem<NW * 64> rank;
  TopkSmem<NW * 64> topk;
};

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void route_prefill_mfma_kernel(RouteArgs a) {
  constexpr int NT = NW * 64;
  constexpr int KSTEPS = D / 16;
  constexpr int F4 = D / 4;                     // float4 per summary row
  constexpr int FPT = kRTile * F4 / NT;         // float4 per thread per tile
  static_assert(FPT >= 1 && kRTile * F4 % NT == 0, "tile split");
  using Smem = RoutePrefillSmem<D, NW>;
  const KParams& kp = a.kp;

  int x = blockIdx.x;
  const int h = x % kp.Hkv;
  x /= kp.Hkv;
  const int b = x % kp.B;
  x /= kp.B;
  const int u = a.n_units - 1 - x;
  const int bh = b * kp.Hkv + h;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int ql = lane & 31;
  const int hb = lane >> 5;
  const int hh = wid / 2;
  const int pos0 = (wid & 1) * 32;
  const int t0 = (a.q_pos ? a.q_pos[b] : 0) + a.pos_bias;
  const int64_t unit = static_cast<int64_t>(bh) * a.n_units + u;

  __shared__ Smem sm;

  if (t0 < 0 || static_cast<int64_t>(t0) + a.nq - 1 >= kp.n_cap || t0 % kp.C != 0) {
    for (int i = tid; i < kp.top_k; i += NT) a.chunk_idx[unit * kp.top_k + i] = -1;
    for (int i = tid; i < kp.top_g; i += NT) a.group_idx[unit * kp.top_g + i] = -1;
    return;
  }
  const int j = t0 / kp.C + u;
  const int nM = max(0, j - kp.n_local - kp.n_sink);

  // ---- the wave's 32 query rows as the A operand
  bf16x8_t qa[KSTEPS];
  {
    const int64_t qrow = (static_cast<int64_t>(b) * kp.Hq + static_cast<int64_t>(h) * kp.gq + hh) * a.nq +
                         static_cast<int64_t>(u) * kp.C + pos0 + ql;
    const uint4* qp = reinterpret_cast<const uint4*>(static_cast<const bf16*>(a.Q) + qrow * D);
#pragma unroll
    for (int d = 0; d < KSTEPS; ++d) qa[d] = __builtin_bit_cast(bf16x8_t, qp[2 * d + hb]);
  }

  // scores of n rows (row(i) -> float32 summary row) into out[0..n)
  auto score_tiles = [&](int n, auto row, float* out) {
    const int n_tiles = (n + kRTile - 1) / kRTile;
    float4 reg[FPT];
    auto fetch = [&](int tt) {
#pragma unroll
      for (int i = 0; i < FPT; ++i) {
        const int f = tid + i * NT;
        const int r = f / F4, c = f % F4;
        const int idx = tt * kRTile + r;
        reg[i] = idx < n ? reinterpret_cast<const float4*>(row(idx))[c] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    };
    auto stage = [&](int buf) {
#pragma unroll
      for (int i = 0; i < FPT; ++i) {
        const int f = tid + i * NT;
        const int r = f / F4, c = f % F4;
        const float4 v = reg[i];
        const float hx = bf16_to_f32(f32_to_bf16(v.x)), hy = bf16_to_f32(f32_to_bf16(v.y));
        const float hz = bf16_to_f32(f32_to_bf16(v.z)), hw = bf16_to_f32(f32_to_bf16(v.w));
        *reinterpret_cast<uint2*>(&sm.hi[buf][r * Smem::ROW + c * 8]) =
            make_uint2(pack_bf16x2(hx, hy), pack_bf16x2(hz, hw));
        *reinterpret_cast<uint2*>(&sm.lo[buf][r * Smem::ROW + c * 8]) =
            make_uint2(pack_bf16x2(v.x - hx, v.y - hy), pack_bf16x2(v.z - hz, v.w - hw));
      }
    };
    if (n_tiles == 0) return;
    fetch(0);
    stage(0);
    __syncthreads();
    for (int tt = 0; tt < n_tiles; ++tt) {
      const int buf = tt & 1;
      if (tt + 1 < n_tiles) fetch(tt + 1);
      f32x16_t acc = f32x16_t{};
#pragma unroll
      for (int d = 0; d < KSTEPS; ++d) {
        const int off = ql * Smem::ROW + (16 * d + 8 * hb) * 2;
        const bf16x8_t bh_ = *reinterpret_cast<const bf16x8_t*>(&sm.hi[buf][off]);
        const bf16x8_t bl_ = *reinterpret_cast<const bf16x8_t*>(&sm.lo[buf][off]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[d], bh_, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[d], bl_, acc, 0, 0, 0);
      }
      float mx = acc[0];
#pragma unroll
      for (int v = 1; v < 16; ++v) mx = fmaxf(mx, acc[v]);
      {
        float pa, pb;
        dpp::swap32(mx, pa, pb);
        mx = fmaxf(pa, pb);
      }
      if (hb == 0) sm.wmax[wid][ql] = mx;
      if (tt + 1 < n_tiles) stage(buf ^ 1);
      __syncthreads();
      if (tid < kRTile) {
        const int idx = tt * kRTile + tid;
        float m = sm.wmax[0][tid];
#pragma unroll
        for (int w = 1; w < NW; ++w) m = fmaxf(m, sm.wmax[w][tid]);
        if (idx < n) out[idx] = m * kp.inv_sqrt_d;
      }
      __syncthreads();
    }
  };

  // ---- level 1: chunk scores and top-k
  const float* ctab = a.chunk_sum + static_cast<int64_t>(bh) * kp.n_chunks_cap * D;
  score_tiles(nM, [&](int i) { return ctab + static_cast<int64_t>(kp.n_sink + i) * D; }, sm.scores);
  int cnt;
  if (nM <= NT)
    cnt = rank_select<NT>(tid < nM ? sm.scores[tid] : 0.f, nM, kp.top_k, sm.sel_chunks, sm.rank);
  else
    cnt = block_topk<NT>([&](int i) { return sm.scores[i]; }, nM, kp.top_k, sm.sel_chunks, sm.topk);
  int32_t* ci = a.chunk_idx + unit * kp.top_k;
  for (int i = tid; i < kp.top_k; i += NT) ci[i] = i < cnt ? kp.n_sink + sm.sel_chunks[i] : -1;

  // ---- level 2: group scores of the routed chunks and top-g
  const int m = kp.m;
  const int nG = cnt * m;
  const float* gtab = a.group_sum + static_cast<int64_t>(bh) * kp.n_chunks_cap * kp.m * D;
  score_tiles(nG,
              [&](int i) {
                const int64_t gid = static_cast<int64_t>(kp.n_sink + sm.sel_chunks[i / m]) * m + i % m;
                return gtab + gid * D;
              },
              sm.scores);
  int gcnt;
  if (nG <= NT)
    gcnt = rank_select<NT>(tid < nG ? sm.scores[tid] : 0.f, nG, kp.top_g, sm.sel_groups, sm.rank);
  else
    gcnt = block_topk<NT>([&](int i) { return sm.scores[i]; }, nG, kp.top_g, sm.sel_groups, sm.topk);
  int32_t* gi = a.group_idx + unit * kp.top_g;
  for (int i = tid; i < kp.top_g; i += NT) {
    int32_t v = -1;
    if (i < gcnt) {
      const int sg = sm.sel_groups[i];
      v = (kp.n_sink + sm.sel_chunks[sg / m]) * m + sg % m;
    }
    gi[i] = v;
  }
}

bool route_prefill_mfma_supported(const KParams& kp, bool bf16_in, int64_t nq) {
  return bf16_in && nq > 1 && kp.C == 64 && (kp.d == 64 || kp.d == 128) &&
         (kp.gq == 1 || kp.gq == 2 || kp.gq == 4) && kp.n_chunks_cap <= 4096 &&
         static_cast<int64_t>(kp.top_k) * kp.m <= 4096;
}

template <int D, int NW>
static hipError_t launch_t(const RouteArgs& a, hipStream_t st) {
  const unsigned n_wg = static_cast<unsigned>(a.kp.B) * a.kp.Hkv * a.n_units;
  route_prefill_mfma_kernel<D, NW><<<n_wg, NW * 64, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_route_prefill_mfma(const RouteArgs& a, hipStream_t st) {
  const int nw = 2 * a.kp.gq;
  if (a.kp.d == 128) {
    if (nw == 2) return launch_t<128, 2>(a, st);
    if (nw == 4) return launch_t<128, 4>(a, st);
    if (nw == 8) return launch_t<128, 8>(a, st);
  } else {
    if (nw == 2) return launch_t<64, 2>(a, st);
    if (nw == 4) return launch_t<64, 4>(a, st);
    if (nw == 8) return launch_t<64, 8>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace hga
