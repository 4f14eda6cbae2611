// The first launch of an HGA decode step: routing (steps 2-3) and attention
// over the always-visible chunks (part of steps 4-5), plus the summary update
// of the chunk the query completes (step 1).  The routed rows are attended by
// the second launch, which also merges in this launch's partial results.
// [HGA technical summary (it), Meccanismo Core, items 1-4].
//
// Work of one (batch, KV head) unit, all on one XCD so that its summaries and
// K/V rows are shared through that XCD's L2:
//   * One routing workgroup scores every candidate chunk summary (all rows in
//     flight at once), selects the top-k chunks, scores their groups and
//     selects the top-g groups, and writes the index lists.
//   * F forced workgroups attend shares of the sink, local and current chunks
//     (known before routing) while the routing workgroup works and store their
//     partial softmax (max, sum, output).  Forced workgroup 0 then summarises
//     the chunk that the query completes.
// No workgroup waits for another.
//
// The score of a chunk or group is the max over the unit's query heads of
// q . s / sqrt(d); selection is exact (score descending, index ascending).
#include "hga_attend_core.hpp"
#include "hga_kernels.hpp"
#include "hga_select.hpp"
#include "hga_summarize.hpp"

#include <algorithm>

namespace hga {

constexpr int kDecThreads = 512;
constexpr int kDecWaves = kDecThreads / kWave;
constexpr int kForcedPF = 2;  // forced blocks in flight per wave
constexpr int kRoutedPF = 4;  // routed blocks in flight per wave
#ifndef HGA_DECODE_HEADS_PER_WG
#define HGA_DECODE_HEADS_PER_WG 1  // query heads per routed-attention workgroup (of 4)
#endif

template <int GQ, int D>
struct DecodeSmem {
  float qs[GQ * D];             // query rows of the unit (fp32) for the scans
  float sc[kDecMaxScores];      // chunk scores, then group scores
  int selc[kSelMaxK];           // selected chunk positions (ascending)
  int selg[kSelMaxK];           // selected group positions (ascending)
  SelSmem<kDecThreads> sel;
  AttnMergeSmem<GQ, D, kDecWaves> mg;
};

// out[i] = max over the GQ query rows in qs of q . row(i) * scale, i in [0, n).
// Eight lanes share one fp32 summary row (each holds D/8 values of it and of
// every query row); a batch of 8 rounds x 64 rows is loaded at once and each
// round is computed as soon as it arrives.
template <int D, int GQ, typename RowFn>
__device__ __forceinline__ void scan_scores(const float* qs, int n, float scale, RowFn row, float* out) {
  constexpr int L = 8;                       // lanes per row
  constexpr int NV = D / 32;                 // float4 pieces per lane per row
  constexpr int RPR = kDecThreads / L;       // rows per round
  constexpr int KR = 8;                      // rounds per batch
  constexpr int BATCH = RPR * KR;
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int piece = lane % L;
  const int rw = wid * (kWave / L) + lane / L;
  float4 q[GQ][NV];
#pragma unroll
  for (int qh = 0; qh < GQ; ++qh)
#pragma unroll
    for (int v = 0; v < NV; ++v) q[qh][v] = *reinterpret_cast<const float4*>(qs + qh * D + v * 32 + piece * 4);
  for (int base = 0; base < n; base += BATCH) {
    float4 cur[KR][NV];
#pragma unroll
    for (int k = 0; k < KR; ++k) {
      const int i = base + k * RPR + rw;
      const float4* r = i < n ? reinterpret_cast<const float4*>(row(i)) : nullptr;
#pragma unroll
      for (int v = 0; v < NV; ++v) cur[k][v] = r ? r[v * L + piece] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // rounds in load order, so that each is computed as soon as it arrives;
    // rounds past the last row are skipped (a wave-uniform branch)
#pragma unroll
    for (int k = 0; k < KR; ++k) {
      if (base + k * RPR >= n) break;
      float mx = -__builtin_huge_valf();
#pragma unroll
      for (int qh = 0; qh < GQ; ++qh) {
        float acc = 0.f;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          acc = fmaf(q[qh][v].x, cur[k][v].x, acc);
          acc = fmaf(q[qh][v].y, cur[k][v].y, acc);
          acc = fmaf(q[qh][v].z, cur[k][v].z, acc);
          acc = fmaf(q[qh][v].w, cur[k][v].w, acc);
        }
        mx = fmaxf(mx, sum8(acc));
      }
      const int i = base + k * RPR + rw;
      if (i < n && piece == 0) out[i] = mx * scale;
    }
  }
}

template <typename T, int D, int GQ>
__global__ __launch_bounds__(kDecThreads) void decode_route_kernel(DecodeArgs a) {
  const KParams& kp = a.kp;
  const int F = a.forced_wgs;
  // Placement: consecutive workgroups go to consecutive XCDs, so all
  // workgroups of unit bh carry the same blockIdx.x % 8; the forced roles
  // (0 .. F-1) come before the routing role (F) in blockIdx order.
  const int x = blockIdx.x;
  const int xcd = x % kXcds;
  const int slot = x / kXcds;
  const int role = slot / a.units_per_xcd;
  const int bh = (slot % a.units_per_xcd) * kXcds + xcd;
  if (bh >= kp.B * kp.Hkv || role > F) return;
  const int b = bh / kp.Hkv;
  const int h = bh % kp.Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = wave_id();
  const bool routing = role == F;
  const int t = a.seq_len[b] - 1;
  constexpr int stride = attn_part_stride<D, GQ>();
  float* parts = a.partials + static_cast<int64_t>(bh) * F * stride;

  __shared__ DecodeSmem<GQ, D> sm;

  // a position outside the cache: empty index lists and NaN output (the
  // attention launch then does nothing for this unit)
  if (t < 0 || t >= kp.n_cap) {
    if (routing) {
      for (int i = tid; i < kp.top_k; i += kDecThreads) a.chunk_idx[static_cast<int64_t>(bh) * kp.top_k + i] = -1;
      for (int i = tid; i < kp.top_g; i += kDecThreads) a.group_idx[static_cast<int64_t>(bh) * kp.top_g + i] = -1;
      const AttnOut out{a.O, nullptr, a.out_bf16, static_cast<int64_t>(b) * kp.Hq + h * GQ, 1, 0};
      out.put_nan<D, kDecThreads>(GQ);
    }
    return;
  }
  const int j = t / kp.C;
  const T* Qb = static_cast<const T*>(a.Q) + (static_cast<int64_t>(b) * kp.Hq + h * GQ) * D;
  const T* Kb = static_cast<const T*>(a.K) + static_cast<int64_t>(bh) * kp.n_cap * D;
  const T* Vb = static_cast<const T*>(a.V) + static_cast<int64_t>(bh) * kp.n_cap * D;

  AttnLaneFor<T, D, GQ> st;
  auto init_q = [&]() { st.init([&](int hh) { return Qb + static_cast<int64_t>(hh) * D; }, lane & 15); };

  if (!routing) {
    // ---- a share of the forced (sink, local, current) chunk rows
    const int f = role;
    init_q();
    const Forced fc = forced_chunks(j, kp.n_sink, kp.n_local);
    const int nF = fc.n * kp.C;
    const int nblk = (nF + kAttnBlock - 1) / kAttnBlock;
    const int bb = min(nblk, f * a.forced_bpw);
    const int be = min(nblk, bb + a.forced_bpw);
    // masked slots point at the query's own row
    auto row = [&](int s, const T*& kr, const T*& vr) -> bool {
      const int fi = s >> kp.log2C;
      const int off = s & (kp.C - 1);
      const int64_t tok = s < nF ? static_cast<int64_t>(forced_chunk_at(fc, fi)) * kp.C + off : t;
      const bool ok = s < nF && tok <= t;
      kr = Kb + (ok ? tok : t) * D;
      vr = Vb + (ok ? tok : t) * D;
      return ok;
    };
    st.template run<kForcedPF>(0, bb + wid, be, kDecWaves, kp.scale_log2, row);
    attn_merge_waves(st, sm.mg);
    // publish [o | m | l]; the attention launch that follows reads it
    float* mine = parts + static_cast<int64_t>(f) * stride;
    for (int e = tid; e < GQ * D; e += kDecThreads) mine[e] = attn_wg_value<D, GQ, kDecWaves>(sm.mg, e);
    if (tid < GQ) {
      mine[GQ * D + tid] = sm.mg.M[tid];
      mine[GQ * D + GQ + tid] = sm.mg.L[tid];
    }

    // ---- the query completes chunk j: summarise it for the next steps' routing
    if (f == 0 && a.build_summary && (t + 1) % kp.C == 0) {
      summarize_chunk<T, D>(Kb + static_cast<int64_t>(j) * kp.C * D, j, kp, true, nullptr,
                            a.chunk_sum_w + (static_cast<int64_t>(bh) * kp.n_chunks_cap + j) * D,
                            a.group_sum_w + (static_cast<int64_t>(bh) * kp.n_chunks_cap * kp.m +
                                             static_cast<int64_t>(j) * kp.m) * D);
    }
    return;
  }

  // ---- level 1: score every candidate chunk, keep the top-k
  for (int e = tid; e < GQ * D; e += kDecThreads) sm.qs[e] = elem<T>::get(Qb, e);
  __syncthreads();
  const int nM = max(0, j - kp.n_local - kp.n_sink);
  const float* ctab = a.chunk_sum + (static_cast<int64_t>(bh) * kp.n_chunks_cap + kp.n_sink) * D;
  scan_scores<D, GQ>(sm.qs, nM, kp.inv_sqrt_d, [&](int i) { return ctab + static_cast<int64_t>(i) * D; }, sm.sc);
  __syncthreads();
  const int cnt = block_select<kDecThreads>([&](int i) { return sm.sc[i]; }, nM, kp.top_k, sm.selc, sm.sel);
  int32_t* ci = a.chunk_idx + static_cast<int64_t>(bh) * kp.top_k;
  for (int i = tid; i < kp.top_k; i += kDecThreads) ci[i] = i < cnt ? kp.n_sink + sm.selc[i] : -1;

  // ---- level 2: score the groups of the routed chunks, keep the top-g
  const int m = kp.m;
  const int nG = cnt * m;
  const float* gtab = a.group_sum + static_cast<int64_t>(bh) * kp.n_chunks_cap * m * D;
  scan_scores<D, GQ>(sm.qs, nG, kp.inv_sqrt_d,
                     [&](int i) {
                       const int64_t gid = static_cast<int64_t>(kp.n_sink + sm.selc[i / m]) * m + i % m;
                       return gtab + gid * D;
                     },
                     sm.sc);
  __syncthreads();
  const int gcnt = block_select<kDecThreads>([&](int i) { return sm.sc[i]; }, nG, kp.top_g, sm.selg, sm.sel);
  for (int i = tid; i < kp.top_g; i += kDecThreads) {
    int32_t v = -1;
    if (i < gcnt) {
      const int sg = sm.selg[i];
      v = (kp.n_sink + sm.selc[sg / m]) * m + sg % m;
    }
    a.group_idx[static_cast<int64_t>(bh) * kp.top_g + i] = v;
  }
}

// ---------------------------------------------------------------------------
// Second launch: workgroup (unit, hg) attends every routed group row of the
// unit for query heads hg*HG .. hg*HG+HG-1 and merges the result with those
// heads' forced-window partials from the first launch into the output.  The
// GQ/HG workgroups of a unit read the same K/V rows, on the same XCD, so the
// repeats are served by that XCD's L2.
template <int GQ, int HG, int D>
struct DecodeAttendSmem {
  int gl[kSelMaxK];
  AttnMergeSmem<HG, D, kDecWaves> mg;
};

template <typename T, int D, int GQ, int HG>
__global__ __launch_bounds__(kDecThreads) void decode_attend_kernel(DecodeArgs a) {
  constexpr int NHG = GQ / HG;
  const KParams& kp = a.kp;
  const int F = a.forced_wgs;
  // placement: the NHG workgroups of unit bh share blockIdx.x % 8 (one XCD)
  const int x = blockIdx.x;
  const int xcd = x % kXcds;
  const int slot = x / kXcds;
  const int hg = slot / a.units_per_xcd;
  const int bh = (slot % a.units_per_xcd) * kXcds + xcd;
  if (bh >= kp.B * kp.Hkv || hg >= NHG) return;
  const int b = bh / kp.Hkv;
  const int h = bh % kp.Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = wave_id();
  const int t = a.seq_len[b] - 1;
  if (t < 0 || t >= kp.n_cap) return;  // NaN output written by the routing launch
  const int head0 = h * GQ + hg * HG;   // first query head of this workgroup
  const T* Qb = static_cast<const T*>(a.Q) + (static_cast<int64_t>(b) * kp.Hq + head0) * D;
  const T* Kb = static_cast<const T*>(a.K) + static_cast<int64_t>(bh) * kp.n_cap * D;
  const T* Vb = static_cast<const T*>(a.V) + static_cast<int64_t>(bh) * kp.n_cap * D;
  constexpr int stride = attn_part_stride<D, GQ>();
  const float* parts = a.partials + static_cast<int64_t>(bh) * F * stride;

  __shared__ DecodeAttendSmem<GQ, HG, D> sm;
  for (int i = tid; i < kp.top_g; i += kDecThreads) sm.gl[i] = a.group_idx[static_cast<int64_t>(bh) * kp.top_g + i];
  AttnLaneFor<T, D, HG> st;
  st.init([&](int hh) { return Qb + static_cast<int64_t>(hh) * D; }, lane & 15);
  __syncthreads();

  const int nR = kp.top_g * kp.G;
  const int nblk = (nR + kAttnBlock - 1) / kAttnBlock;
  // masked slots point at the query's own row
  auto row = [&](int s, const T*& kr, const T*& vr) -> bool {
    const int e = s >> kp.log2G;
    const int g = s < nR ? sm.gl[e] : -1;
    const int64_t tok = (static_cast<int64_t>(g) << kp.log2G) + (s & (kp.G - 1));
    const bool ok = g >= 0 && tok <= t;
    kr = Kb + (ok ? tok : t) * D;
    vr = Vb + (ok ? tok : t) * D;
    return ok;
  };
  st.template run<kRoutedPF>(0, wid, nblk, kDecWaves, kp.scale_log2, row);
  attn_merge_waves(st, sm.mg);

  const AttnOut out{a.O, nullptr, a.out_bf16, static_cast<int64_t>(b) * kp.Hq + head0, 1, 0};
  constexpr int kOut = (HG * D + kDecThreads - 1) / kDecThreads;
#pragma unroll
  for (int r = 0; r < kOut; ++r) {
    const int e = tid + r * kDecThreads;
    if (e >= HG * D) continue;
    const int hh = e / D;               // head within this workgroup
    const int gh = hg * HG + hh;        // head within the unit (forced partial layout)
    float mp[kDecMaxParts], lp[kDecMaxParts], op[kDecMaxParts];
#pragma unroll
    for (int p = 0; p < kDecMaxParts; ++p) {
      const bool in = p < F;
      const float* q = parts + (in ? p : 0) * stride;
      mp[p] = in ? q[GQ * D + gh] : -__builtin_huge_valf();
      lp[p] = q[GQ * D + GQ + gh];
      op[p] = q[gh * D + e % D];
    }
    float M = sm.mg.M[hh];
#pragma unroll
    for (int p = 0; p < kDecMaxParts; ++p) M = fmaxf(M, mp[p]);
    const float wo = sm.mg.M[hh] == -__builtin_huge_valf() ? 0.f : exp2f(sm.mg.M[hh] - M);
    float num = attn_wg_value<D, HG, kDecWaves>(sm.mg, e) * wo;
    float den = sm.mg.L[hh] * wo;
#pragma unroll
    for (int p = 0; p < kDecMaxParts; ++p) {
      const float w = mp[p] == -__builtin_huge_valf() ? 0.f : exp2f(mp[p] - M);
      num += w * op[p];
      den += w * lp[p];
    }
    out.put<D>(hh, e % D, num / den);
  }
}

bool decode_fused_supported(const KParams& kp) {
  const int64_t max_cand = std::max<int64_t>(0, kp.n_chunks_cap - 1 - kp.n_local - kp.n_sink);
  return (kp.gq == 1 || kp.gq == 2 || kp.gq == 4) && (kp.d == 64 || kp.d == 128) && kp.log2C >= 0 &&
         kp.log2G >= 0 &&
         max_cand <= kDecMaxScores && block_select_fits<kDecThreads>(static_cast<int>(max_cand), kp.top_k) &&
         static_cast<int64_t>(kp.top_k) * kp.m <= kDecMaxScores &&
         block_select_fits<kDecThreads>(kp.top_k * kp.m, kp.top_g) && kp.top_g <= kSelMaxK;
}

template <typename T, int D, int GQ>
static hipError_t launch_t(const DecodeArgs& a, hipStream_t st) {
  const unsigned n_wg = static_cast<unsigned>(kXcds) * a.units_per_xcd * (a.forced_wgs + 1);
  decode_route_kernel<T, D, GQ><<<n_wg, kDecThreads, 0, st>>>(a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_gq(const DecodeArgs& a, hipStream_t st) {
  switch (a.kp.gq) {
    case 1: return launch_t<T, D, 1>(a, st);
    case 2: return launch_t<T, D, 2>(a, st);
    case 4: return launch_t<T, D, 4>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_route(const DecodeArgs& a, bool bf16_in, hipStream_t st) {
  if (bf16_in) return a.kp.d == 64 ? launch_gq<bf16, 64>(a, st) : launch_gq<bf16, 128>(a, st);
  return a.kp.d == 64 ? launch_gq<float, 64>(a, st) : launch_gq<float, 128>(a, st);
}

template <typename T, int D, int GQ, int HG>
static hipError_t launch_att_t(const DecodeArgs& a, hipStream_t st) {
  const unsigned n_wg = static_cast<unsigned>(kXcds) * a.units_per_xcd * (GQ / HG);
  decode_attend_kernel<T, D, GQ, HG><<<n_wg, kDecThreads, 0, st>>>(a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_att_gq(const DecodeArgs& a, hipStream_t st) {
  switch (a.kp.gq) {
    case 1: return launch_att_t<T, D, 1, 1>(a, st);
    case 2: return launch_att_t<T, D, 2, 1>(a, st);
    case 4: return launch_att_t<T, D, 4, HGA_DECODE_HEADS_PER_WG>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_attend(const DecodeArgs& a, bool bf16_in, hipStream_t st) {
  if (bf16_in) return a.kp.d == 64 ? launch_att_gq<bf16, 64>(a, st) : launch_att_gq<bf16, 128>(a, st);
  return a.kp.d == 64 ? launch_att_gq<float, 64>(a, st) : launch_att_gq<float, 128>(a, st);
}

}  // namespace hga
