// Steps 2-3 of HGA: two-level routing on the vector ALUs.
// [HGA technical summary (it), Meccanismo Core, item 2, first two bullets]:
// the current chunk (or decode query) scores the compact chunk-summary table and
// keeps the top-k chunks; inside them it scores the group summaries and keeps
// the top-g groups.
//
// Layout of the work: each (b, kv head, unit) has its candidate chunks
// [n_sink, j - n_local) split over `slices` workgroups.  A workgroup streams
// its slice of the fp32 summary table once.  Eight lanes share one summary row
// and every load instruction of a wave covers eight whole 128-byte pieces of
// eight rows; a lane keeps D/8 values of its row and of every query vector,
// the dot products are reduced over the eight lanes with DPP.  The score of a
// row is the max over the unit's query vectors of q.s / sqrt(d).  Every
// workgroup keeps the top-k of its own slice (a chunk of the global top-k is
// in the top-k of its slice) and publishes those (score, chunk) pairs with
// device-coherent stores; the last workgroup of the unit to finish
// (device-scope counter) selects the top-k among them, scores the groups of
// the routed chunks and selects the top-g.  The scan is bound by HBM
// bandwidth in decode.
//
// In a decode step one extra workgroup per (b, kv head) summarises the chunk
// that the query completes, so a decode loop keeps the tables current.  With
// the warm tier, the workgroup that finishes a unit's lists also runs the
// unit's LRU lookup (hga_warm.hpp) on them.
#include "hga_kernels.hpp"
#include "hga_select.hpp"
#include "hga_summarize.hpp"
#include "hga_warm.hpp"

#include <type_traits>

namespace hga {

// Workgroup shapes: NT threads, eight lanes per summary row, kRounds rows in
// flight per lane.  Prefill units use 256 threads; a decode unit uses 512, so
// a unit has half as many slices and slice winners, and the last workgroup
// scores the group rows of the routed chunks in one round of loads.
constexpr int kRouteThreads = 256;     // prefill
constexpr int kRouteDecThreads = 512;  // decode (one query per sequence)
constexpr int kRowLanes = 8;           // lanes per summary row
constexpr int kRounds = 4;             // rounds in flight per lane
template <int NT>
struct RouteShape {
  static constexpr int kRowsPerRound = NT / kRowLanes;            // rows per block round
  static constexpr int kSliceRows = kRowsPerRound * kRounds;      // candidate chunks per workgroup
  // query vectors per register batch; the wide shape holds fewer, so that it
  // stays within 128 registers and two workgroups fit on a CU
  static constexpr int kQB = NT > 256 ? 2 : 4;
  static constexpr int kWavesPerSimd = NT > 256 ? 4 : 1;          // occupancy asked of the compiler
};
constexpr int kLdsCand = 2048;         // candidates staged in LDS for the selections
constexpr int kRouteQs = 16 * 128;     // query elements staged in LDS (one query per sequence)

template <int NT>
struct RouteSmem {
  union {  // scratch of the selection in use
    TopkSmem<NT> topk;
    SelSmem<NT> sel;
  };
  float loc[RouteShape<NT>::kSliceRows];
  int loc_sel[RouteShape<NT>::kSliceRows];
  int sel_chunks[1024];
  int sel_groups[1024];
  float cand_s[kLdsCand];
  int cand_i[kLdsCand];
  float qs[kRouteQs];  // the unit's query vectors in fp32, when they fit (one query per sequence)
  int is_last;
};

// number of slice-local winners published by slice x (and, summed, the offset
// of slice x's entries): min(k, rows of the slice)
__device__ __forceinline__ int slice_count(int x, int nM, int cps, int k) {
  const int rows = max(0, min(cps, nM - x * cps));
  return min(k, rows);
}

// put(i, max over the unit's query vectors of q . row(i) / sqrt(d)) for i in
// [0, n); only lanes with lane % 8 == 0 call put.  row(i) is a float32 row.
// The query vectors come from qs (LDS, fp32, vector v at qs + v * D) when it
// is set, else from global memory at qbase.
template <typename T, int D, int NT, typename RowFn, typename PutFn>
__device__ __forceinline__ void score_rows(const T* __restrict__ qbase, int64_t head_stride,
                                           int rows_per_head, int nqv, const float* qs, const KParams& kp,
                                           int n, RowFn row, PutFn put) {
  constexpr int NV = D / 32;  // float4 pieces per lane per row
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  const int piece = lane % kRowLanes;
  const int rw = wid * (kWave / kRowLanes) + lane / kRowLanes;  // row within a round
  constexpr int kRowsPerRound = RouteShape<NT>::kRowsPerRound;
  constexpr int kQB = RouteShape<NT>::kQB;
  for (int base = 0; base < n; base += kRowsPerRound * kRounds) {
    float4 s[kRounds][NV];
#pragma unroll
    for (int k = 0; k < kRounds; ++k) {
      const int i = base + k * kRowsPerRound + rw;
      const float4* r = i < n ? reinterpret_cast<const float4*>(row(i)) : nullptr;
#pragma unroll
      for (int v = 0; v < NV; ++v)
        s[k][v] = r ? r[v * kRowLanes + piece] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float mx[kRounds];
#pragma unroll
    for (int k = 0; k < kRounds; ++k) mx[k] = -__builtin_huge_valf();
    for (int v0 = 0; v0 < nqv; v0 += kQB) {
      float4 q[kQB][NV];
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb) {
        const int vv = v0 + qb < nqv ? v0 + qb : nqv - 1;
        if (qs) {
#pragma unroll
          for (int v = 0; v < NV; ++v) q[qb][v] = *reinterpret_cast<const float4*>(qs + vv * D + v * 32 + piece * 4);
        } else {
          const T* qr = qbase + (vv / rows_per_head) * head_stride + static_cast<int64_t>(vv % rows_per_head) * D;
#pragma unroll
          for (int v = 0; v < NV; ++v) {
            const int d0 = v * 32 + piece * 4;
            q[qb][v] = make_float4(elem<T>::get(qr, d0), elem<T>::get(qr, d0 + 1), elem<T>::get(qr, d0 + 2),
                                   elem<T>::get(qr, d0 + 3));
          }
        }
      }
#pragma unroll
      for (int k = 0; k < kRounds; ++k) {
#pragma unroll
        for (int qb = 0; qb < kQB; ++qb) {
          float acc = 0.f;
#pragma unroll
          for (int v = 0; v < NV; ++v) {
            acc = fmaf(q[qb][v].x, s[k][v].x, acc);
            acc = fmaf(q[qb][v].y, s[k][v].y, acc);
            acc = fmaf(q[qb][v].z, s[k][v].z, acc);
            acc = fmaf(q[qb][v].w, s[k][v].w, acc);
          }
          mx[k] = fmaxf(mx[k], sum8(acc));
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kRounds; ++k) {
      const int i = base + k * kRowsPerRound + rw;
      if (i < n && piece == 0) put(i, mx[k] * kp.inv_sqrt_d);
    }
  }
}

template <typename T, int D, int NT>
__global__ __launch_bounds__(NT, RouteShape<NT>::kWavesPerSimd) void route_scan_kernel(RouteArgs a) {
  const KParams& kp = a.kp;
  const int bh = blockIdx.z;
  const int u = blockIdx.y;
  const int x = blockIdx.x;
  const int b = bh / kp.Hkv;
  const int h = bh % kp.Hkv;
  const int t0 = (a.q_pos ? a.q_pos[b] : 0) + a.pos_bias;
  const bool prefill = a.nq > 1;
  const int j = t0 / kp.C + (prefill ? u : 0);

  __shared__ RouteSmem<NT> sm;
  // the warm tier's stage (decode shape only; a prefill launch never has it)
  constexpr bool kWarm = NT == kRouteDecThreads;
  __shared__ std::conditional_t<kWarm, WarmStage, char> wst;
  const int n_groups_cap = static_cast<int>(kp.n_cap / kp.G);

  // positions outside the cache (or a prefill block not aligned to C): the unit
  // gets empty index lists and nothing else happens
  const int64_t t_last = static_cast<int64_t>(t0) + (prefill ? a.nq - 1 : 0);
  if (t0 < 0 || t_last >= kp.n_cap || (prefill && t0 % kp.C != 0)) {
    if (x == 0) {
      const int64_t unit = static_cast<int64_t>(bh) * a.n_units + u;
      for (int i = threadIdx.x; i < kp.top_k; i += NT) a.chunk_idx[unit * kp.top_k + i] = -1;
      for (int i = threadIdx.x; i < kp.top_g; i += NT) a.group_idx[unit * kp.top_g + i] = -1;
      if constexpr (kWarm) {
        if (a.warm.tags) {  // the step still counts
          warm_stage_load<NT>(a.warm, unit, wst);
          for (int i = threadIdx.x; i < kp.top_g; i += NT) wst.list[i] = -1;
          __syncthreads();
          warm_lookup_unit<NT>(a.warm, unit, kp.top_g, n_groups_cap, wst);
        }
      }
    }
    return;
  }

  if (x == a.slices) {
    // fused summary update: this decode query completes chunk j
    if (!a.build_summary || (t0 + 1) % kp.C != 0) return;
    const int c = j;
    int64_t slot = c;
    if (a.ksrc.ring && c >= kp.n_sink) slot = kp.n_sink + (c - kp.n_sink) % (kp.n_local + 1);
    const T* rows = static_cast<const T*>(a.ksrc.base) +
                    (static_cast<int64_t>(bh) * a.ksrc.bh_rows + slot * kp.C) * D;
    summarize_chunk<T, D>(rows, c, kp, true, nullptr,
                          a.chunk_sum_w + (static_cast<int64_t>(bh) * kp.n_chunks_cap + c) * D,
                          a.group_sum_w + (static_cast<int64_t>(bh) * kp.n_chunks_cap * kp.m +
                                           static_cast<int64_t>(c) * kp.m) * D);
    return;
  }

  const int64_t unit = static_cast<int64_t>(bh) * a.n_units + u;
  const int nM = max(0, j - kp.n_local - kp.n_sink);
  const int c_lo = kp.n_sink + x * a.chunks_per_slice;
  const int n_here = max(0, min(kp.n_sink + nM, c_lo + a.chunks_per_slice) - c_lo);

  const int rows_per_head = prefill ? kp.C : 1;
  const int nqv = kp.gq * rows_per_head;
  const T* qbase = static_cast<const T*>(a.Q) +
                   ((static_cast<int64_t>(b) * kp.Hq + static_cast<int64_t>(h) * kp.gq) * a.nq +
                    (prefill ? static_cast<int64_t>(u) * kp.C : 0)) * D;
  const int64_t head_stride = a.nq * D;
  // one query per sequence: its vectors once into LDS (fp32), instead of 2-byte
  // global loads of each vector for every batch of rows in both scans
  const float* qs = !prefill && nqv * D <= kRouteQs ? sm.qs : nullptr;
  if (qs)
    for (int e = threadIdx.x; e < nqv * D; e += NT) sm.qs[e] = elem<T>::get(qbase, e);
  __syncthreads();

  float* cand_s = a.scores + unit * kp.n_chunks_cap;   // published (score, chunk) pairs
  int* cand_i = a.cand_ids + unit * kp.n_chunks_cap;
  const float* ctab = a.chunk_sum + static_cast<int64_t>(bh) * kp.n_chunks_cap * D;
  float* sc_out = a.scores_out ? a.scores_out + static_cast<int64_t>(bh) * kp.n_chunks_cap : nullptr;
  if (n_here > 0) {
    score_rows<T, D, NT>(qbase, head_stride, rows_per_head, nqv, qs, kp, n_here,
                     [&](int i) { return ctab + static_cast<int64_t>(c_lo + i) * D; },
                     [&](int i, float v) {
                       sm.loc[i] = v;
                       if (sc_out) sc_out[c_lo + i] = v;
                     });
  }
  __syncthreads();
  // ---- top-k of this slice, published in ascending chunk order
  {
    int off = 0;
    for (int xx = 0; xx < x; ++xx) off += slice_count(xx, nM, a.chunks_per_slice, kp.top_k);
    const int kk = slice_count(x, nM, a.chunks_per_slice, kp.top_k);
    if (kk > 0) {
      if (kk < n_here) {
        block_select<NT>([&](int i) { return sm.loc[i]; }, n_here, kk, sm.loc_sel, sm.sel);
        for (int r = threadIdx.x; r < kk; r += NT) {
          const int i = sm.loc_sel[r];
          st_agent(cand_s + off + r, sm.loc[i]);
          st_agent(cand_i + off + r, c_lo + i);
        }
      } else {
        for (int r = threadIdx.x; r < kk; r += NT) {
          st_agent(cand_s + off + r, sm.loc[r]);
          st_agent(cand_i + off + r, c_lo + r);
        }
      }
    }
  }

  // ---- last workgroup of the unit does the selections
  if (!arrive_last(&a.counters[unit], static_cast<uint32_t>(a.slices), &sm.is_last)) return;

  // the warm slots' loads share the round trip of the winners' loads
  if constexpr (kWarm) {
    if (a.warm.tags) warm_stage_load<NT>(a.warm, unit, wst);
  }
  int n_c = 0;
  for (int xx = 0; xx < a.slices; ++xx) n_c += slice_count(xx, nM, a.chunks_per_slice, kp.top_k);
  const bool in_lds = n_c <= kLdsCand;
  if (in_lds) {
    for (int i = threadIdx.x; i < n_c; i += NT) {
      sm.cand_s[i] = cand_s[i];
      sm.cand_i[i] = cand_i[i];
    }
  }
  __syncthreads();
  // candidates are in ascending chunk order, so position order breaks ties
  int cnt;
  if (in_lds && block_select_fits<NT>(n_c, kp.top_k)) {
    cnt = block_select<NT>([&](int i) { return sm.cand_s[i]; }, n_c, kp.top_k, sm.sel_chunks, sm.sel);
  } else if (in_lds) {
    cnt = block_topk<NT>([&](int i) { return sm.cand_s[i]; }, n_c, kp.top_k, sm.sel_chunks, sm.topk);
  } else {
    cnt = block_topk<NT>([&](int i) { return cand_s[i]; }, n_c, kp.top_k, sm.sel_chunks, sm.topk);
  }
  // selected positions -> chunk ids (ascending)
  for (int i = threadIdx.x; i < cnt; i += NT) {
    const int pos = sm.sel_chunks[i];
    sm.sel_chunks[i] = in_lds ? sm.cand_i[pos] : cand_i[pos];
  }
  __syncthreads();
  int32_t* ci = a.chunk_idx + unit * kp.top_k;
  for (int i = threadIdx.x; i < kp.top_k; i += NT) ci[i] = i < cnt ? sm.sel_chunks[i] : -1;

  const int nG = cnt * kp.m;
  const int m = kp.m;
  const float* gtab = a.group_sum + static_cast<int64_t>(bh) * kp.n_chunks_cap * kp.m * D;
  float* gsc = nG <= kLdsCand ? sm.cand_s : a.gscores + unit * static_cast<int64_t>(kp.top_k) * kp.m;
  if (nG > 0) {
    score_rows<T, D, NT>(qbase, head_stride, rows_per_head, nqv, qs, kp, nG,
                     [&](int i) {
                       const int64_t gid = static_cast<int64_t>(sm.sel_chunks[i / m]) * m + i % m;
                       return gtab + gid * D;
                     },
                     [&](int i, float v) { gsc[i] = v; });
  }
  __threadfence_block();
  __syncthreads();
  int gcnt;
  if (block_select_fits<NT>(nG, kp.top_g))
    gcnt = block_select<NT>([&](int i) { return gsc[i]; }, nG, kp.top_g, sm.sel_groups, sm.sel);
  else
    gcnt = block_topk<NT>([&](int i) { return gsc[i]; }, nG, kp.top_g, sm.sel_groups, sm.topk);
  int32_t* gi = a.group_idx + unit * kp.top_g;
  for (int i = threadIdx.x; i < kp.top_g; i += NT) {
    int32_t v = -1;
    if (i < gcnt) {
      const int sg = sm.sel_groups[i];
      v = sm.sel_chunks[sg / m] * m + sg % m;
    }
    gi[i] = v;
    if constexpr (kWarm) {
      if (a.warm.tags) wst.list[i] = v;
    }
  }
  if constexpr (kWarm) {
    if (a.warm.tags) {
      __syncthreads();
      warm_lookup_unit<NT>(a.warm, unit, kp.top_g, n_groups_cap, wst);
    }
  }
}

int route_chunks_per_slice(const KParams& kp, int64_t nq) {
  (void)kp;
  return nq == 1 ? RouteShape<kRouteDecThreads>::kSliceRows : RouteShape<kRouteThreads>::kSliceRows;
}

template <typename T, int D>
static hipError_t launch_t(const RouteArgs& a, hipStream_t st) {
  dim3 grid(a.slices + (a.build_summary ? 1 : 0), a.n_units, a.kp.B * a.kp.Hkv);
  if (a.nq == 1)
    route_scan_kernel<T, D, kRouteDecThreads><<<grid, kRouteDecThreads, 0, st>>>(a);
  else
    route_scan_kernel<T, D, kRouteThreads><<<grid, kRouteThreads, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_route_scan(const RouteArgs& a, bool bf16_q, bool /*bf16_k*/, hipStream_t st) {
  if (bf16_q) return a.kp.d == 64 ? launch_t<bf16, 64>(a, st) : launch_t<bf16, 128>(a, st);
  return a.kp.d == 64 ? launch_t<float, 64>(a, st) : launch_t<float, 128>(a, st);
}

}  // namespace hga
