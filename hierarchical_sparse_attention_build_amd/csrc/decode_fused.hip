// An HGA decode step in one launch: routing (steps 2-3), attention over the
// union of the routed groups with the sink, local and current chunks (steps
// 4-5), and the summary update of the chunk the query completes (step 1)
// [HGA technical summary (it), Meccanismo Core, items 1-4].
//
// Work of one (batch, KV head) unit, all on one XCD so that its summaries and
// K/V rows are shared through that XCD's L2:
//   * R routing workgroups (R = 1 or 2) each score every candidate chunk
//     summary, select the top-k chunks, score their groups and select the
//     top-g groups; they compute the same lists (the same arithmetic on the
//     same data), routing workgroup 0 writes them, and each attends the unit's
//     query heads over its share of the routed groups' rows.  A second one
//     costs no hand-off: it repeats the routing (its summary reads hit the
//     XCD's L2) to halve the routed attention, which follows the routing on
//     the critical path.
//   * F forced workgroups attend shares of the sink, local and current chunks
//     (known before routing) while the routing workgroups work.  Forced
//     workgroup 0 then summarises the chunk that the query completes.
//   * When the grid leaves compute units idle, one more workgroup per unit
//     reads the candidate summaries at launch, in the scans' order, so that
//     the routing scans find much of the table in the XCD's L2 (it computes
//     nothing and takes no part in the merge).
// The F + R partial softmax results (max, sum, output) are merged by the last
// of them to finish; no workgroup waits for another.
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
constexpr int kRoutedPF = 2;  // routed blocks in flight per wave
// Widest selection compiled in: 4 keys per lane covers 2048 candidate chunks
// and k <= 32 (wider selections go to the separate routing kernel); the 8-
// and 16-key variants would push the kernel's scalar registers into spills.
constexpr int kDecSelE = 4;

template <int GQ, int D>
struct DecodeSmem {
  float qs[GQ * D];             // query rows of the unit (fp32) for the scans
  alignas(16) float sc[kDecMaxScores];  // chunk scores, then group scores
  int selc[kSelMaxK];           // selected chunk positions (ascending)
  int selg[kSelMaxK];           // selected group positions (ascending)
  int gl[kSelMaxK];             // routed group ids
  int early;                    // the routing workgroup arrived early (given lists: their length)
  SelSmem<kDecThreads> sel;
  AttnMergeSmem<GQ, D, kDecWaves> mg;
  alignas(16) unsigned char ktile[kDecWaves * attn_ktile_bytes<D>()];
};

// Scans: out[i] = max over the GQ query rows in qs of q . row(i) * scale, i in
// [0, n).  Eight lanes share one fp32 summary row (each holds D/8 values of it
// and of every query row).  Rows go in batches of 2 rounds x 64 rows, two
// batches in flight: a CU with more loads outstanding streams slower here.
constexpr int kScanL = 8;                         // lanes per row
constexpr int kScanKR = 2;                        // rounds per batch (more in flight is slower)
constexpr int kScanRPR = kDecThreads / kScanL;    // rows per round
constexpr int kScanBatch = kScanRPR * kScanKR;

template <int D>
struct ScanBatch {
  float4 v[kScanKR][D / 32];
};

// This lane's pieces of rows base + k * kScanRPR + (its row), those < n.
template <int D, typename RowFn>
__device__ __forceinline__ void scan_load(int base, int n, RowFn row, ScanBatch<D>& b) {
  constexpr int NV = D / 32;
  const int lane = threadIdx.x & (kWave - 1);
  const int piece = lane % kScanL;
  const int rw = wave_id() * (kWave / kScanL) + lane / kScanL;
#pragma unroll
  for (int k = 0; k < kScanKR; ++k) {
    const int i = base + k * kScanRPR + rw;
    const float4* r = i < n ? reinterpret_cast<const float4*>(row(i)) : nullptr;
#pragma unroll
    for (int v = 0; v < NV; ++v) b.v[k][v] = r ? r[v * kScanL + piece] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// With FIRST, the batch at 0 was loaded beforehand (scan_load(0, n0, ...) with
// n0 >= min(n, kScanBatch)) and is passed in `first`.
template <int D, int GQ, bool FIRST = false, typename RowFn>
__device__ __forceinline__ void scan_scores(const float* qs, int n, float scale, RowFn row, float* out,
                                            const ScanBatch<D>& first = ScanBatch<D>{}) {
  constexpr int NV = D / 32;
  const int lane = threadIdx.x & (kWave - 1);
  const int piece = lane % kScanL;
  const int rw = wave_id() * (kWave / kScanL) + lane / kScanL;
  float4 q[GQ][NV];
#pragma unroll
  for (int qh = 0; qh < GQ; ++qh)
#pragma unroll
    for (int v = 0; v < NV; ++v) q[qh][v] = *reinterpret_cast<const float4*>(qs + qh * D + v * 32 + piece * 4);
  // rounds in load order, so that each is computed as soon as it arrives;
  // rounds past the last row are skipped (a wave-uniform branch)
  auto compute = [&](int base, const ScanBatch<D>& cur) {
#pragma unroll
    for (int k = 0; k < kScanKR; ++k) {
      if (base + k * kScanRPR >= n) break;
      float mx = -__builtin_huge_valf();
#pragma unroll
      for (int qh = 0; qh < GQ; ++qh) {
        float acc = 0.f;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          acc = fmaf(q[qh][v].x, cur.v[k][v].x, acc);
          acc = fmaf(q[qh][v].y, cur.v[k][v].y, acc);
          acc = fmaf(q[qh][v].z, cur.v[k][v].z, acc);
          acc = fmaf(q[qh][v].w, cur.v[k][v].w, acc);
        }
        mx = fmaxf(mx, sum8(acc));
      }
      const int i = base + k * kScanRPR + rw;
      if (i < n && piece == 0) out[i] = mx * scale;
    }
  };
  // two batches in flight: the next batch's loads go out before the current
  // batch is computed
  ScanBatch<D> cur;
  if (FIRST) cur = first;
  else scan_load<D>(0, n, row, cur);
  for (int base = 0; base < n; base += kScanBatch) {
    ScanBatch<D> nxt;
    if (base + kScanBatch < n) scan_load<D>(base + kScanBatch, n, row, nxt);
    compute(base, cur);
    cur = nxt;
  }
}

// ---------------------------------------------------------------------------
// Forced-window partials and the final merge.  Part slots of a unit: forced
// workgroup f in slot f, routing workgroup r in slot F + r.  Every workgroup
// of a unit counts its arrival once its slot is written; the last arriver
// merges the other slots with its own result (still in LDS) into O.  A lone
// routing workgroup normally arrives last: it checks the count early, and
// when every forced workgroup has arrived it arrives at once and prefetches
// their slots while it still routes and attends.  Nobody waits for anybody.

// This thread's output element e = threadIdx.x (GQ * D <= kDecThreads) of the
// part slots in `want` (bit p: slot p), loaded with plain loads.
struct PartRegs {
  float m[kDecMaxParts], l[kDecMaxParts], o[kDecMaxParts];
};

template <int D, int GQ>
__device__ __forceinline__ void load_parts(const float* parts, uint32_t want, PartRegs& r) {
  constexpr int stride = attn_part_stride<D, GQ>();
  const int e = min(static_cast<int>(threadIdx.x), GQ * D - 1);
  const int hh = e / D;
#pragma unroll
  for (int p = 0; p < kDecMaxParts; ++p) {
    const bool in = (want >> p) & 1u;
    const float* q = parts + (in ? p : 0) * stride;
    r.m[p] = in ? q[GQ * D + hh] : -__builtin_huge_valf();
    r.l[p] = q[GQ * D + GQ + hh];
    r.o[p] = q[e];
  }
}

// Park this thread's loaded forced slots in LDS (stash[kDecMaxForced * 3 *
// kDecThreads] floats) and take them back; slots p >= n come back empty.
template <int D, int GQ>
__device__ __forceinline__ void stash_parts(const PartRegs& r, float* stash) {
  const int t = threadIdx.x;
#pragma unroll
  for (int p = 0; p < kDecMaxForced; ++p) {
    stash[(3 * p) * kDecThreads + t] = r.m[p];
    stash[(3 * p + 1) * kDecThreads + t] = r.l[p];
    stash[(3 * p + 2) * kDecThreads + t] = r.o[p];
  }
}
template <int D, int GQ>
__device__ __forceinline__ void unstash_parts(const float* stash, int n, PartRegs& r) {
  const int t = threadIdx.x;
#pragma unroll
  for (int p = 0; p < kDecMaxForced; ++p) {
    r.m[p] = p < n ? stash[(3 * p) * kDecThreads + t] : -__builtin_huge_valf();
    r.l[p] = stash[(3 * p + 1) * kDecThreads + t];
    r.o[p] = stash[(3 * p + 2) * kDecThreads + t];
  }
#pragma unroll
  for (int p = kDecMaxForced; p < kDecMaxParts; ++p) {
    r.m[p] = -__builtin_huge_valf();
    r.l[p] = 0.f;
    r.o[p] = 0.f;
  }
}
static_assert(kDecMaxForced * 3 * kDecThreads <= kDecMaxScores, "stash fits the score array");

// O[e] from the unit's part slots, merged in slot order: slot `own` is this
// workgroup's merged waves (mg, the values it publishes), the others were
// loaded into r (an empty slot has m = -inf).  The order does not depend on
// which workgroup arrives last, so a call's output does not either.
template <int D, int GQ>
__device__ __forceinline__ void merge_store(const AttnMergeSmem<GQ, D, kDecWaves>& mg, const PartRegs& r, int own,
                                            const AttnOut& out) {
  const int e = threadIdx.x;
  if (e >= GQ * D) return;
  const int hh = e / D;
  float m[kDecMaxParts], l[kDecMaxParts], o[kDecMaxParts];
  const float om = mg.M[hh], ol = mg.L[hh], oo = attn_wg_value<D, GQ, kDecWaves>(mg, e);
#pragma unroll
  for (int p = 0; p < kDecMaxParts; ++p) {
    m[p] = p == own ? om : r.m[p];
    l[p] = p == own ? ol : r.l[p];
    o[p] = p == own ? oo : r.o[p];
  }
  float M = -__builtin_huge_valf();
#pragma unroll
  for (int p = 0; p < kDecMaxParts; ++p) M = fmaxf(M, m[p]);
  float num = 0.f, den = 0.f;
#pragma unroll
  for (int p = 0; p < kDecMaxParts; ++p) {
    if (m[p] != -__builtin_huge_valf()) {
      const float w = exp2f(m[p] - M);
      num = fmaf(w, o[p], num);
      den = fmaf(w, l[p], den);
    }
  }
  out.put<D>(hh, e % D, num / den);
}

// Part slots per unit.
__device__ __forceinline__ int unit_parts(const DecodeArgs& a) { return a.forced_wgs + a.routing_wgs; }

// Write this workgroup's merged waves into part slot `slot` (device-coherent
// stores), count the arrival and return true in every thread of the last
// arriver of the unit's F + R workgroups.
template <int D, int GQ>
__device__ __forceinline__ bool publish_arrive(const DecodeArgs& a, int bh, int slot, AttnMergeSmem<GQ, D, kDecWaves>& mg) {
  constexpr int stride = attn_part_stride<D, GQ>();
  const int tid = threadIdx.x;
  float* mine = a.partials + (static_cast<int64_t>(bh) * unit_parts(a) + slot) * stride;
  for (int e = tid; e < GQ * D; e += kDecThreads) st_agent(mine + e, attn_wg_value<D, GQ, kDecWaves>(mg, e));
  if (tid < GQ) {
    st_agent(mine + GQ * D + tid, mg.M[tid]);
    st_agent(mine + GQ * D + GQ + tid, mg.L[tid]);
  }
  return arrive_last(a.sync + 4 * static_cast<int64_t>(bh), static_cast<uint32_t>(unit_parts(a)), &mg.is_last);
}

__device__ __forceinline__ AttnOut unit_out(const DecodeArgs& a, int bh, int gq) {
  const KParams& kp = a.kp;
  return AttnOut{a.O, nullptr, a.out_bf16, static_cast<int64_t>(bh / kp.Hkv) * kp.Hq + (bh % kp.Hkv) * gq, 1, 0};
}

// Attention of the unit's GQ query heads over the sink, local and current
// chunks, blocks [f * bpw, (f + 1) * bpw) of them.
template <typename T, int D, int GQ>
__device__ __forceinline__ void forced_role(const DecodeArgs& a, int bh, int f, int t, DecodeSmem<GQ, D>& sm) {
  const KParams& kp = a.kp;
  const int b = bh / kp.Hkv, h = bh % kp.Hkv;
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = wave_id();
  const int j = t / kp.C;
  const T* Qb = static_cast<const T*>(a.Q) + (static_cast<int64_t>(b) * kp.Hq + h * GQ) * D;
  const T* Kb = static_cast<const T*>(a.K) + static_cast<int64_t>(bh) * kp.n_cap * D;
  const T* Vb = static_cast<const T*>(a.V) + static_cast<int64_t>(bh) * kp.n_cap * D;
  AttnLaneFor<T, D, GQ> st;
  st.init([&](int hh) { return Qb + static_cast<int64_t>(hh) * D; }, lane & 15);
  st.set_tile(sm.ktile);
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
  if (publish_arrive<D, GQ>(a, bh, f, sm.mg)) {
    // last arriver (rare): merge the other slots, the routing ones included
    PartRegs r;
    const uint32_t all = (1u << unit_parts(a)) - 1u;
    load_parts<D, GQ>(a.partials + static_cast<int64_t>(bh) * unit_parts(a) * attn_part_stride<D, GQ>(),
                      all & ~(1u << f), r);
    merge_store<D, GQ>(sm.mg, r, f, unit_out(a, bh, GQ));
  }
  // ---- the query completes chunk j: summarise it for the next steps' routing
  if (f == 0 && a.build_summary && (t + 1) % kp.C == 0) {
    float* cs = a.chunk_sum_w + (static_cast<int64_t>(bh) * kp.n_chunks_cap + j) * D;
    float* gs = a.group_sum_w + (static_cast<int64_t>(bh) * kp.n_chunks_cap * kp.m + static_cast<int64_t>(j) * kp.m) * D;
    bool done = false;
    if constexpr (sizeof(T) == 2) {
      if (summarize_fast_ok<D>(kp, true, true, kDecMaxScores) && summarize_loads_per_group<D>(kp) == 4) {
        // the tables and group means in the score array, which this role does
        // not use (only the 4-load variant is compiled in: the kernel stays
        // within its registers)
        summarize_chunk_fast<D, 4>(reinterpret_cast<const bf16*>(Kb) + static_cast<int64_t>(j) * kp.C * D, kp,
                                   sm.sc, cs, gs);
        done = true;
      }
    }
    if (!done) summarize_chunk<T, D>(Kb + static_cast<int64_t>(j) * kp.C * D, j, kp, true, nullptr, cs, gs);
  }
}

// Routing of the unit (chunk top-k, then group top-g) and attention of its GQ
// query heads over share r of the routed groups' rows (routed blocks r, r + R,
// ... of the 16-row blocks), merged with the other partials.
template <typename T, int D, int GQ>
__device__ __forceinline__ void routing_role(const DecodeArgs& a, int bh, int r, DecodeSmem<GQ, D>& sm) {
  const KParams& kp = a.kp;
  const int F = a.forced_wgs;
  const int R = a.routing_wgs;
  const bool writer = r == 0;  // the one routing workgroup that writes the lists
  const int b = bh / kp.Hkv, h = bh % kp.Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = wave_id();
  const T* Qb = static_cast<const T*>(a.Q) + (static_cast<int64_t>(b) * kp.Hq + h * GQ) * D;
  const T* Kb = static_cast<const T*>(a.K) + static_cast<int64_t>(bh) * kp.n_cap * D;
  const T* Vb = static_cast<const T*>(a.V) + static_cast<int64_t>(bh) * kp.n_cap * D;
  const float* parts = a.partials + static_cast<int64_t>(bh) * (F + R) * attn_part_stride<D, GQ>();
  const uint32_t others = ((1u << (F + R)) - 1u) & ~(1u << (F + r));
  uint32_t* counter = a.sync + 4 * static_cast<int64_t>(bh);
  const float* ctab = a.chunk_sum + (static_cast<int64_t>(bh) * kp.n_chunks_cap + kp.n_sink) * D;
  auto crow = [&](int i) { return ctab + static_cast<int64_t>(i) * D; };
  const bool given = a.routes_in != nullptr;  // the group list is an input (no routing)
  // ---- loads that do not depend on the position go out together with it:
  // the query rows and the first batch of candidate summaries (bounded by
  // the table, masked once the candidate count is known)
  ScanBatch<D> first;
  if (!given && kp.top_k > 0) {
    scan_load<D>(0, min(kScanBatch, kp.n_chunks_cap - kp.n_sink), crow, first);
    for (int e = tid; e < GQ * D; e += kDecThreads) sm.qs[e] = elem<T>::get(Qb, e);
  }
  const int t = a.seq_len[b] + a.pos_offset;
  if (t < 0 || t >= kp.n_cap) {
    // a position outside the cache: empty index lists and NaN output
    if (!writer) return;
    if (a.chunk_idx)
      for (int i = tid; i < kp.top_k; i += kDecThreads) a.chunk_idx[static_cast<int64_t>(bh) * kp.top_k + i] = -1;
    if (a.group_idx)
      for (int i = tid; i < kp.top_g; i += kDecThreads) a.group_idx[static_cast<int64_t>(bh) * kp.top_g + i] = -1;
    unit_out(a, bh, GQ).put_nan<D, kDecThreads>(GQ);
    return;
  }
  const int j = t / kp.C;
  int gcnt = 0;
  bool early = false;
  PartRegs pr;
  if (given) {
    // ---- the given list in canonical form: an entry outside the cache, in a
    // forced chunk, after the query's chunk, or repeating an earlier entry
    // adds no token to the visible set and is dropped; the others keep their
    // order, without holes
    const int32_t* gin = a.routes_in + static_cast<int64_t>(bh) * kp.top_g;
    const int64_t n_groups_cap = kp.n_cap / kp.G;
    int* raw = sm.selc;   // top_g <= kSelMaxK entries
    int* keep = sm.selg;
    for (int e = tid; e < kp.top_g; e += kDecThreads) {
      const int g = gin[e];
      const int c = g >= 0 ? g / kp.m : -1;
      raw[e] = g >= 0 && g < n_groups_cap && c >= kp.n_sink && c < j - kp.n_local ? g : -1;
    }
    __syncthreads();
    for (int e = tid; e < kp.top_g; e += kDecThreads) {
      const int g = raw[e];
      bool first = g >= 0;
      for (int f = 0; first && f < e; ++f) first = raw[f] != g;
      keep[e] = first;
    }
    __syncthreads();
    if (wid == 0) {
      int base = 0;
      for (int i0 = 0; i0 < kp.top_g; i0 += kWave) {
        const bool ok = i0 + lane < kp.top_g && keep[i0 + lane];
        const uint64_t mk = __ballot(ok);
        if (ok) sm.gl[base + bits_below(mk)] = raw[i0 + lane];
        base += __popcll(mk);
      }
      if (lane == 0) sm.early = base;
    }
    __syncthreads();
    gcnt = sm.early;
  } else {
  __syncthreads();
  // ---- level 1: score every candidate chunk, keep the top-k (none to score
  // when top_k = 0: a streaming head sees its sink and local windows only)
  const int nM = kp.top_k > 0 ? max(0, j - kp.n_local - kp.n_sink) : 0;
  scan_scores<D, GQ, true>(sm.qs, nM, kp.inv_sqrt_d, crow, sm.sc, first);
  __syncthreads();
  const int cnt = block_select<kDecThreads, kDecSelE>([&](int i) { return sm.sc[i]; }, nM, kp.top_k, sm.selc, sm.sel);
  // ---- a lone routing workgroup: have all forced workgroups arrived?  Then
  // this one is the last: it arrives now (resetting the count) and prefetches
  // their slots below.
  if (tid == 0) {
    int early = 0;
    if (R == 1 && __hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == static_cast<uint32_t>(F)) {
      __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      early = 1;
    }
    sm.early = early;
  }
  int32_t* ci = a.chunk_idx + static_cast<int64_t>(bh) * kp.top_k;
  if (writer)
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
  early = sm.early != 0;
  if (early) load_parts<D, GQ>(parts, (1u << F) - 1u, pr);
  gcnt = block_select<kDecThreads, kDecSelE>([&](int i) { return sm.sc[i]; }, nG, kp.top_g, sm.selg, sm.sel);
  // the prefetched slots wait in LDS (the scores are no longer needed)
  if (early) stash_parts<D, GQ>(pr, sm.sc);
  for (int i = tid; i < kp.top_g; i += kDecThreads) {
    int32_t v = -1;
    if (i < gcnt) {
      const int sg = sm.selg[i];
      v = (kp.n_sink + sm.selc[sg / m]) * m + sg % m;
      sm.gl[i] = v;
    }
    if (writer) a.group_idx[static_cast<int64_t>(bh) * kp.top_g + i] = v;
  }
  __syncthreads();
  }  // routing
  // ---- attention over the routed groups' rows (routed chunks end before the
  // local window, so all their rows are visible)
  AttnLaneFor<T, D, GQ> st;
  st.init([&](int hh) { return Qb + static_cast<int64_t>(hh) * D; }, lane & 15);
  st.set_tile(sm.ktile);
  const int nR = gcnt * kp.G;
  const int nblk = (nR + kAttnBlock - 1) / kAttnBlock;
  if (kp.log2G >= 4 && !given) {
    // groups of whole blocks: every fetched slot is a routed row, so no slot is
    // masked (and the list reads of a block have no branch around them)
    auto row = [&](int s, const T*& kr, const T*& vr) -> bool {
      const int64_t tok = (static_cast<int64_t>(sm.gl[s >> kp.log2G]) << kp.log2G) + (s & (kp.G - 1));
      kr = Kb + tok * D;
      vr = Vb + tok * D;
      return true;
    };
    st.template run<kRoutedPF>(0, r * kDecWaves + wid, nblk, R * kDecWaves, kp.scale_log2, row);
  } else {
    // slots past the list and rows after the query are masked and point at
    // the query's own row
    auto row = [&](int s, const T*& kr, const T*& vr) -> bool {
      const int64_t tok =
          (static_cast<int64_t>(sm.gl[min(s >> kp.log2G, kSelMaxK - 1)]) << kp.log2G) + (s & (kp.G - 1));
      const bool ok = s < nR && tok <= t;
      kr = Kb + (ok ? tok : t) * D;
      vr = Vb + (ok ? tok : t) * D;
      return ok;
    };
    st.template run<kRoutedPF>(0, r * kDecWaves + wid, nblk, R * kDecWaves, kp.scale_log2, row);
  }
  attn_waves_to_lds(st, sm.mg);
  attn_merge_waves_rest(sm.mg);
  if (early) {
    unstash_parts<D, GQ>(sm.sc, F, pr);
    merge_store<D, GQ>(sm.mg, pr, F, unit_out(a, bh, GQ));
    return;
  }
  if (publish_arrive<D, GQ>(a, bh, F + r, sm.mg)) {
    load_parts<D, GQ>(parts, others, pr);
    merge_store<D, GQ>(sm.mg, pr, F + r, unit_out(a, bh, GQ));
  }
}

// Warm-up role: read candidate summary rows [0, nM) of unit bh (every 16-byte
// piece, in the scans' order, eight loads of a thread in flight: more or fewer
// were slower) and discard the values.
template <int D>
__device__ __forceinline__ void warm_summaries(const DecodeArgs& a, int bh) {
  const KParams& kp = a.kp;
  const int t = a.seq_len[bh / kp.Hkv] + a.pos_offset;
  if (t < 0 || t >= kp.n_cap) return;
  const int nM = max(0, t / kp.C - kp.n_local - kp.n_sink);
  const float4* tab = reinterpret_cast<const float4*>(a.chunk_sum + (static_cast<int64_t>(bh) * kp.n_chunks_cap + kp.n_sink) * D);
  const int end = nM * (D / 4);
  float acc = 0.f;
#pragma unroll 8
  for (int i = static_cast<int>(threadIdx.x); i < end; i += kDecThreads) {
    const float4 v = tab[i];
    acc = fmaxf(acc, fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w)));
  }
  asm volatile("" ::"v"(acc));  // keeps the loads; nothing is written
}

// Unit bh of the workgroup at blockIdx.x: consecutive workgroups go to
// consecutive XCDs, so all workgroups of a unit share blockIdx.x % 8 and its
// summaries and rows are shared through one L2; roles in blockIdx order.
__device__ __forceinline__ void unit_of(const DecodeArgs& a, int& bh, int& role) {
  const int x = blockIdx.x;
  const int slot = x / kXcds;
  role = slot / a.units_per_xcd;
  bh = (slot % a.units_per_xcd) * kXcds + x % kXcds;
}

// One launch per step.  Roles: 0..R-1 routing and routed attention, R..R+F-1
// forced, R+F the summary warm-up (when present).
template <typename T, int D, int GQ>
__global__ __launch_bounds__(kDecThreads) void decode_step_kernel(DecodeArgs a) {
  int bh, role;
  unit_of(a, bh, role);
  const KParams& kp = a.kp;
  if (bh >= kp.B * kp.Hkv || role >= a.routing_wgs + a.forced_wgs + a.warm_wgs) return;
  if (role >= a.routing_wgs + a.forced_wgs) {
    warm_summaries<D>(a, bh);
    return;
  }
  __shared__ DecodeSmem<GQ, D> sm;
  if (role < a.routing_wgs) {
    routing_role<T, D, GQ>(a, bh, role, sm);
  } else {
    const int t = a.seq_len[bh / kp.Hkv] + a.pos_offset;
    if (t < 0 || t >= kp.n_cap) return;  // NaN output written by routing workgroup 0
    forced_role<T, D, GQ>(a, bh, role - a.routing_wgs, t, sm);
  }
}

bool decode_fused_supported(const KParams& kp) {
  const int64_t max_cand = std::max<int64_t>(0, kp.n_chunks_cap - 1 - kp.n_local - kp.n_sink);
  return (kp.gq == 1 || kp.gq == 2 || kp.gq == 4) && (kp.d == 64 || kp.d == 128) && kp.log2C >= 0 &&
         kp.log2G >= 0 &&
         max_cand <= kDecMaxScores && block_select_fits<kDecThreads, kDecSelE>(static_cast<int>(max_cand), kp.top_k) &&
         static_cast<int64_t>(kp.top_k) * kp.m <= kDecMaxScores &&
         block_select_fits<kDecThreads, kDecSelE>(kp.top_k * kp.m, kp.top_g) && kp.top_g <= kSelMaxK;
}

template <typename T, int D, int GQ>
static hipError_t launch_t(const DecodeArgs& a, hipStream_t st) {
  const unsigned per_role = static_cast<unsigned>(kXcds) * a.units_per_xcd;
  decode_step_kernel<T, D, GQ><<<per_role * (a.routing_wgs + a.forced_wgs + a.warm_wgs), kDecThreads, 0, st>>>(a);
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

hipError_t launch_decode_step(const DecodeArgs& a, bool bf16_in, hipStream_t st) {
  if (a.forced_wgs < 1 || a.forced_wgs > kDecMaxForced || a.routing_wgs < 1 || a.routing_wgs > kDecMaxRouting ||
      a.warm_wgs < 0 || a.warm_wgs > 1 || (a.warm_wgs && a.routes_in))
    return hipErrorInvalidValue;
  if (bf16_in) return a.kp.d == 64 ? launch_gq<bf16, 64>(a, st) : launch_gq<bf16, 128>(a, st);
  return a.kp.d == 64 ? launch_gq<float, 64>(a, st) : launch_gq<float, 128>(a, st);
}

}  // namespace hga
