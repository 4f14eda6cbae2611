// Steps 4-5 of HGA on the vector ALUs: visibility union + exact softmax
// attention over the gathered original K/V rows, split over workgroups.
// [HGA technical summary (it), Meccanismo Core, item 2 third bullet (current,
// sink and recent local chunks always visible) and item 4 (standard softmax
// over the bounded exact token set; no summary enters the output)].
//
// Token slots of a query at position t in chunk j: first the forced chunks
// (sink + local + current, C slots each; tokens after t masked), then the
// routed groups (G slots each; -1 entries masked).  Slots are cut into blocks
// of 16 rows.  A workgroup takes a contiguous range of blocks; its four waves
// take every fourth block and run independently (the per-wave loop is in
// hga_attend_core.hpp).  All query heads that share the KV head are served by
// the same loads.  With several workgroups per query the partial (max, sum,
// output) goes to the workspace and the last workgroup merges.  In decode the
// kernel is bound by HBM bandwidth.
#include "hga_attend_core.hpp"
#include "hga_kernels.hpp"

namespace hga {

constexpr int kAttThreads = 256;
constexpr int kAttWaves = kAttThreads / kWave;
static_assert(kAttnBlock == kAttBlockRows && kAttnMaxParts == kAttMaxParts, "block and part limits");

template <int GQ, int D>
struct AttSmem {
  int gl[1024];
  int sl[1024];  // staged slot of each routed entry (warm tier)
  AttnMergeSmem<GQ, D, kAttWaves> mg;
  alignas(16) unsigned char ktile[kAttWaves * attn_ktile_bytes<D>()];
};

template <typename T, int D, int GQ>
__global__ __launch_bounds__(kAttThreads) void attend_splitk_kernel(AttendArgs a) {
  const KParams& kp = a.kp;
  const int bh = blockIdx.z;
  const int qi = blockIdx.y;
  const int x = blockIdx.x;
  const int b = bh / kp.Hkv;
  const int h = bh % kp.Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = wave_id();
  const int t_row0 = (a.q_pos ? a.q_pos[b] : 0) + a.pos_bias;
  const int t = t_row0 + qi;
  const int j = t / kp.C;
  const int u = a.nq == 1 ? 0 : j - t_row0 / kp.C;
  const AttnOut out{a.O, a.lse, a.out_bf16, static_cast<int64_t>(b) * kp.Hq + h * GQ, a.nq, qi};

  __shared__ AttSmem<GQ, D> sm;

  // a position outside the cache (or a prefill block not aligned to C) yields NaN
  if (t_row0 < 0 || static_cast<int64_t>(t_row0) + a.nq - 1 >= kp.n_cap ||
      (a.nq > 1 && t_row0 % kp.C != 0) || u < 0 || u >= a.n_units) {
    if (x == 0 && a.part_offset == 0) out.put_nan<D, kAttThreads>(GQ);
    return;
  }

  // ---- routed group list of the unit (entries outside [0, n_cap/G) are masked)
  const int32_t* glg = a.group_idx + (static_cast<int64_t>(bh) * a.n_units + u) * kp.top_g;
  for (int e = tid; e < kp.top_g; e += kAttThreads) sm.gl[e] = glg[e];
  if (a.stage_slot)
    for (int e = tid; e < kp.top_g; e += kAttThreads)
      sm.sl[e] = a.stage_slot[(static_cast<int64_t>(bh) * a.n_units + u) * kp.top_g + e];

  const T* Qb = static_cast<const T*>(a.Q);
  AttnLaneFor<T, D, GQ> st;
  st.init([&](int hh) { return Qb + ((static_cast<int64_t>(b) * kp.Hq + h * GQ + hh) * a.nq + qi) * D; },
          lane & 15);
  st.set_tile(sm.ktile);
  __syncthreads();

  const Forced fc = forced_chunks(j, kp.n_sink, kp.n_local);
  const int nF = fc.n * kp.C;
  const int n_slots = nF + kp.top_g * kp.G;
  // part 3: both parts in one grid, workgroups [0, part1_splits) on the forced
  // slots and the rest on the routed ones, with the block ranges and partial
  // slots of two launches (part 1, then part 2 at part_offset part1_splits)
  const int part = a.part == 3 ? (x < a.part1_splits ? 1 : 2) : a.part;
  const int xs = a.part == 3 && part == 2 ? x - a.part1_splits : x;  // index within the part
  int R0 = 0, R1 = n_slots;
  if (part == 1) R1 = nF;
  if (part == 2) R0 = nF;
  const int nblocks = (R1 - R0 + kAttnBlock - 1) / kAttnBlock;
  const int bb = min(nblocks, xs * a.tiles_per_split);
  const int be = min(nblocks, bb + a.tiles_per_split);
  const int n_groups_cap = static_cast<int>(kp.n_cap / kp.G);

  const T* Kb = static_cast<const T*>(a.K);
  const T* Vb = static_cast<const T*>(a.V);
  const T* Ks = static_cast<const T*>(a.K_stage);
  const T* Vs = static_cast<const T*>(a.V_stage);
  const bool staged_routed = Ks != nullptr;

  // the query's own row (always written): what masked slots point at
  int64_t own;
  {
    int64_t hs = j;
    if (a.kv.ring && j >= kp.n_sink) hs = kp.n_sink + (j - kp.n_sink) % (kp.n_local + 1);
    own = (static_cast<int64_t>(bh) * a.kv.bh_rows + hs * kp.C + (t - j * kp.C)) * D;
  }
  // K and V rows of slot s, or false (pointing at the own row) when the slot is masked
  auto row = [&](int s, const T*& kr, const T*& vr) -> bool {
    kr = Kb + own;
    vr = Vb + own;
    if (s >= R1) return false;
    int64_t ro;
    if (s < nF) {
      const int fi = kp.log2C >= 0 ? s >> kp.log2C : s / kp.C;
      const int off = s - fi * kp.C;
      const int c = forced_chunk_at(fc, fi);
      const int64_t tok = static_cast<int64_t>(c) * kp.C + off;
      if (tok > t) return false;
      int64_t hs = c;
      if (a.kv.ring && c >= kp.n_sink) hs = kp.n_sink + (c - kp.n_sink) % (kp.n_local + 1);
      ro = (static_cast<int64_t>(bh) * a.kv.bh_rows + hs * kp.C + off) * D;
      kr = Kb + ro;
      vr = Vb + ro;
      return true;
    }
    const int rs = s - nF;
    const int e = kp.log2G >= 0 ? rs >> kp.log2G : rs / kp.G;
    const int g = sm.gl[e];
    if (g < 0 || g >= n_groups_cap) return false;
    const int64_t tok = static_cast<int64_t>(g) * kp.G + (rs - e * kp.G);
    if (tok > t) return false;
    if (staged_routed && a.stage_slot) {
      const int sl = sm.sl[e];
      if (sl >= 0) {  // cached: the slot's rows
        ro = ((static_cast<int64_t>(bh) * a.stage_slots + sl) * kp.G + (rs - e * kp.G)) * D;
        kr = Ks + ro;
        vr = Vs + ro;
      } else {  // missing (-2 - slot): the rows in host memory (written back to the slot)
        ro = (static_cast<int64_t>(bh) * kp.n_cap + tok) * D;
        kr = static_cast<const T*>(a.K_host) + ro;
        vr = static_cast<const T*>(a.V_host) + ro;
      }
    } else if (staged_routed) {
      ro = (static_cast<int64_t>(bh) * kp.top_g * kp.G + rs) * D;
      kr = Ks + ro;
      vr = Vs + ro;
    } else {
      ro = (static_cast<int64_t>(bh) * a.kv.bh_rows + tok) * D;
      kr = Kb + ro;
      vr = Vb + ro;
    }
    return true;
  };

  if (a.stage_slot && a.K_host) {
    // warm tier: a missing group's rows, read from host memory, also go into
    // the slot the lookup gave it (-2 - slot in the slot list)
    T* Kw = static_cast<T*>(const_cast<void*>(a.K_stage));
    T* Vw = static_cast<T*>(const_cast<void*>(a.V_stage));
    auto wb = [&](int s, T*& kd, T*& vd) -> bool {
      if (s < nF || s >= R1) return false;
      const int rs = s - nF;
      const int e = kp.log2G >= 0 ? rs >> kp.log2G : rs / kp.G;
      const int g = sm.gl[e];
      const int sl = sm.sl[e];
      if (g < 0 || g >= n_groups_cap || sl > -2) return false;
      const int64_t wo = ((static_cast<int64_t>(bh) * a.stage_slots + (-2 - sl)) * kp.G + (rs - e * kp.G)) * D;
      kd = Kw + wo;
      vd = Vw + wo;
      return true;
    };
    st.run(R0, bb + wid, be, kAttWaves, kp.scale_log2, row, wb);
  } else {
    st.run(R0, bb + wid, be, kAttWaves, kp.scale_log2, row);
  }
  attn_merge_waves(st, sm.mg);

  if (a.parts_total == 1) {
    attn_write_final<D, GQ, kAttWaves, kAttThreads>(sm.mg, out);
    return;
  }
  const int64_t row_id = static_cast<int64_t>(bh) * a.nq + qi;  // (b, kv head, query row)
  constexpr int stride = attn_part_stride<D, GQ>();
  attn_publish_and_merge<D, GQ, kAttWaves, kAttThreads>(sm.mg, a.partials + row_id * a.parts_total * stride,
                                                        a.part_offset + x, a.parts_total, &a.counters[row_id], out);
}

int attend_max_slots(const KParams& kp) {
  return (kp.n_sink + kp.n_local + 1) * kp.C + kp.top_g * kp.G;
}

template <typename T, int D, int GQ>
static hipError_t launch_t(const AttendArgs& a, hipStream_t st) {
  dim3 grid(a.splits, static_cast<unsigned>(a.nq), a.kp.B * a.kp.Hkv);
  attend_splitk_kernel<T, D, GQ><<<grid, kAttThreads, 0, st>>>(a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_gq(const AttendArgs& a, hipStream_t st) {
  switch (a.kp.gq) {
    case 1: return launch_t<T, D, 1>(a, st);
    case 2: return launch_t<T, D, 2>(a, st);
    case 4: return launch_t<T, D, 4>(a, st);
    case 8: return launch_t<T, D, 8>(a, st);
    case 16: return launch_t<T, D, 16>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attend_splitk(const AttendArgs& a, bool bf16_in, hipStream_t st) {
  if (bf16_in) return a.kp.d == 64 ? launch_gq<bf16, 64>(a, st) : launch_gq<bf16, 128>(a, st);
  return a.kp.d == 64 ? launch_gq<float, 64>(a, st) : launch_gq<float, 128>(a, st);
}

}  // namespace hga
