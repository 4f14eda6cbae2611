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
// take every fourth block and run independently (online softmax in base 2, no
// LDS and no barrier inside the loop).  Within a block, lane (g, c) holds rows
// g, g+4, g+8, g+12 and the c-th sixteenth of each row, so one load
// instruction fetches four whole rows; QK^T reduces over the 16 lanes of a
// row with DPP, the block max and sum over the 4 row groups with permlane
// swaps, and PV accumulates per lane into its sixteenth of the output.  The
// next block's loads are issued before the current block is computed.  All
// query heads that share the KV head are served by the same loads.  With
// several workgroups per query the partial (max, sum, output) goes to the
// workspace and the last workgroup merges.  In decode the kernel is bound by
// HBM bandwidth.
#include "hga_device.hpp"
#include "hga_kernels.hpp"

namespace hga {

constexpr int kAttThreads = 256;
constexpr int kAttWaves = kAttThreads / kWave;
constexpr int kBlockRows = kAttBlockRows;
constexpr int kMaxParts = kAttMaxParts;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int BYTES> struct RawVec;
template <> struct RawVec<8> { uint2 v; };
template <> struct RawVec<16> { uint4 v; };
template <> struct RawVec<32> { uint4 v0, v1; };

template <int BYTES>
__device__ __forceinline__ RawVec<BYTES> load_raw(const void* p) {
  RawVec<BYTES> r;
  if constexpr (BYTES == 8) r.v = *reinterpret_cast<const uint2*>(p);
  else if constexpr (BYTES == 16) r.v = *reinterpret_cast<const uint4*>(p);
  else {
    r.v0 = reinterpret_cast<const uint4*>(p)[0];
    r.v1 = reinterpret_cast<const uint4*>(p)[1];
  }
  return r;
}

template <int BYTES>
__device__ __forceinline__ RawVec<BYTES> zero_raw() {
  RawVec<BYTES> r;
  if constexpr (BYTES == 8) r.v = make_uint2(0u, 0u);
  else if constexpr (BYTES == 16) r.v = make_uint4(0u, 0u, 0u, 0u);
  else {
    r.v0 = make_uint4(0u, 0u, 0u, 0u);
    r.v1 = r.v0;
  }
  return r;
}

// the 32-bit words of a raw vector
template <int BYTES>
__device__ __forceinline__ uint32_t word(const RawVec<BYTES>& r, int i) {
  if constexpr (BYTES == 8) return i == 0 ? r.v.x : r.v.y;
  else if constexpr (BYTES == 16) return i == 0 ? r.v.x : i == 1 ? r.v.y : i == 2 ? r.v.z : r.v.w;
  else {
    const uint4& hv = i < 4 ? r.v0 : r.v1;
    const int k = i & 3;
    return k == 0 ? hv.x : k == 1 ? hv.y : k == 2 ? hv.z : hv.w;
  }
}

template <int GQ, int D>
struct AttSmem {
  int gl[1024];
  float wm[kAttWaves][GQ];
  float wl[kAttWaves][GQ];
  float wgt[kAttWaves][GQ];
  float L[GQ];
  float M[GQ];
  float ow[kAttWaves][GQ * D];
  float pm[kMaxParts * GQ];  // merge: per-part max, then weight
  float pl[kMaxParts * GQ];
  int is_last;
};

template <typename T, int D, int GQ>
__global__ __launch_bounds__(kAttThreads) void attend_splitk_kernel(AttendArgs a) {
  constexpr int EPL = D / 16;                            // elements of a row per lane
  constexpr int RB = EPL * static_cast<int>(sizeof(T));  // bytes of a row per lane
  constexpr bool kBF = sizeof(T) == 2;
  const KParams& kp = a.kp;
  const int bh = blockIdx.z;
  const int qi = blockIdx.y;
  const int x = blockIdx.x;
  const int b = bh / kp.Hkv;
  const int h = bh % kp.Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int rg = lane >> 4;  // row group within a block
  const int cc = lane & 15;  // sixteenth of the row
  const int t_row0 = (a.q_pos ? a.q_pos[b] : 0) + a.pos_bias;
  const int t = t_row0 + qi;
  const int j = t / kp.C;
  const int u = a.nq == 1 ? 0 : j - t_row0 / kp.C;

  __shared__ AttSmem<GQ, D> sm;

  // a position outside the cache (or a prefill block not aligned to C) yields NaN
  if (t_row0 < 0 || static_cast<int64_t>(t_row0) + a.nq - 1 >= kp.n_cap ||
      (a.nq > 1 && t_row0 % kp.C != 0) || u < 0 || u >= a.n_units) {
    if (x == 0 && a.part_offset == 0) {
      for (int e = tid; e < GQ * D; e += kAttThreads) {
        const int64_t off = ((static_cast<int64_t>(b) * kp.Hq + h * GQ + e / D) * a.nq + qi) * D + e % D;
        if (a.out_bf16) reinterpret_cast<uint16_t*>(a.O)[off] = 0x7fc0u;
        else reinterpret_cast<float*>(a.O)[off] = __builtin_nanf("");
      }
      if (a.lse && tid < GQ)
        a.lse[(static_cast<int64_t>(b) * kp.Hq + h * GQ + tid) * a.nq + qi] = __builtin_nanf("");
    }
    return;
  }

  // ---- routed group list of the unit (entries outside [0, n_cap/G) are masked)
  const int32_t* glg = a.group_idx + (static_cast<int64_t>(bh) * a.n_units + u) * kp.top_g;
  for (int e = tid; e < kp.top_g; e += kAttThreads) sm.gl[e] = glg[e];

  // ---- this lane's sixteenth of the query rows of the GQ heads
  const T* Qb = static_cast<const T*>(a.Q);
  uint32_t qbf[GQ][EPL / 2];  // bf16 pairs (bf16 inputs)
  float qf[kBF ? 1 : GQ][kBF ? 1 : EPL];
#pragma unroll
  for (int hh = 0; hh < GQ; ++hh) {
    const T* qr = Qb + ((static_cast<int64_t>(b) * kp.Hq + h * GQ + hh) * a.nq + qi) * D + cc * EPL;
    const RawVec<RB> r = load_raw<RB>(qr);
    if constexpr (kBF) {
#pragma unroll
      for (int w = 0; w < EPL / 2; ++w) qbf[hh][w] = word(r, w);
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[hh][e] = __uint_as_float(word(r, e));
    }
  }
  __syncthreads();

  const Forced fc = forced_chunks(j, kp.n_sink, kp.n_local);
  const int nF = fc.n * kp.C;
  const int n_slots = nF + kp.top_g * kp.G;
  int R0 = 0, R1 = n_slots;
  if (a.part == 1) R1 = nF;
  if (a.part == 2) R0 = nF;
  const int nblocks = (R1 - R0 + kBlockRows - 1) / kBlockRows;
  const int bb = min(nblocks, x * a.tiles_per_split);
  const int be = min(nblocks, bb + a.tiles_per_split);
  const int n_groups_cap = static_cast<int>(kp.n_cap / kp.G);

  const T* Kb = static_cast<const T*>(a.K);
  const T* Vb = static_cast<const T*>(a.V);
  const T* Ks = static_cast<const T*>(a.K_stage);
  const T* Vs = static_cast<const T*>(a.V_stage);
  const bool staged_routed = Ks != nullptr;

  // element offset of slot s's row, or -1 when the slot is masked
  auto row_of = [&](int s) -> int64_t {
    if (s >= R1) return -1;
    if (s < nF) {
      const int fi = kp.log2C >= 0 ? s >> kp.log2C : s / kp.C;
      const int off = s - fi * kp.C;
      const int c = forced_chunk_at(fc, fi);
      const int64_t tok = static_cast<int64_t>(c) * kp.C + off;
      if (tok > t) return -1;
      int64_t hs = c;
      if (a.kv.ring && c >= kp.n_sink) hs = kp.n_sink + (c - kp.n_sink) % (kp.n_local + 1);
      return (static_cast<int64_t>(bh) * a.kv.bh_rows + hs * kp.C + off) * D;
    }
    const int rs = s - nF;
    const int e = kp.log2G >= 0 ? rs >> kp.log2G : rs / kp.G;
    const int g = sm.gl[e];
    if (g < 0 || g >= n_groups_cap) return -1;
    const int64_t tok = static_cast<int64_t>(g) * kp.G + (rs - e * kp.G);
    if (tok > t) return -1;
    if (staged_routed) return (static_cast<int64_t>(bh) * kp.top_g * kp.G + rs) * D;
    return (static_cast<int64_t>(bh) * a.kv.bh_rows + tok) * D;
  };

  float m_run[GQ], l_run[GQ], o[GQ][EPL];
#pragma unroll
  for (int hh = 0; hh < GQ; ++hh) {
    m_run[hh] = -__builtin_huge_valf();
    l_run[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[hh][e] = 0.f;
  }

  RawVec<RB> kc[4], vc[4];
  bool okc[4];
  auto fetch = [&](int blkid, RawVec<RB>* kr, RawVec<RB>* vr, bool* ok) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = R0 + blkid * kBlockRows + rg + 4 * i;
      const int64_t ro = row_of(s);
      ok[i] = ro >= 0;
      if (ok[i]) {
        const bool st = staged_routed && s >= nF;
        kr[i] = load_raw<RB>((st ? Ks : Kb) + ro + cc * EPL);
        vr[i] = load_raw<RB>((st ? Vs : Vb) + ro + cc * EPL);
      } else {
        kr[i] = zero_raw<RB>();
        vr[i] = zero_raw<RB>();
      }
    }
  };

  int blk = bb + wid;
  if (blk < be) fetch(blk, kc, vc, okc);
  for (; blk < be; blk += kAttWaves) {
    RawVec<RB> kn[4], vn[4];
    bool okn[4];
    const int nxt = blk + kAttWaves;
    if (nxt < be) fetch(nxt, kn, vn, okn);

    // ---- scores (base 2) of the lane's 4 rows for every head
    float s[4][GQ];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) {
        float acc = 0.f;
        if constexpr (kBF) {
#pragma unroll
          for (int w = 0; w < EPL / 2; ++w)
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, qbf[hh][w]),
                                                   __builtin_bit_cast(bf16x2_t, word(kc[i], w)), acc, false);
        } else {
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc = fmaf(qf[hh][e], __uint_as_float(word(kc[i], e)), acc);
        }
        acc = sum16(acc);
        s[i][hh] = okc[i] ? acc * kp.scale_log2 : -__builtin_huge_valf();
      }
    }
    // ---- online softmax over this block's 16 rows
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      float bm = fmaxf(fmaxf(s[0][hh], s[1][hh]), fmaxf(s[2][hh], s[3][hh]));
      bm = max_rows(bm);
      const float m_new = fmaxf(m_run[hh], bm);
      const float alpha = m_new == -__builtin_huge_valf() ? 1.f : exp2f(m_run[hh] - m_new);
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = okc[i] ? exp2f(s[i][hh] - m_new) : 0.f;
        s[i][hh] = p;
        ps += p;
      }
      l_run[hh] = l_run[hh] * alpha + sum_rows(ps);
      m_run[hh] = m_new;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[hh][e] *= alpha;
    }
    // ---- PV
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float vf[EPL];
      if constexpr (kBF) {
#pragma unroll
        for (int w = 0; w < EPL / 2; ++w) {
          const uint32_t x2 = word(vc[i], w);
          vf[2 * w] = bf16lo(x2);
          vf[2 * w + 1] = bf16hi(x2);
        }
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) vf[e] = __uint_as_float(word(vc[i], e));
      }
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh)
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[hh][e] = fmaf(s[i][hh], vf[e], o[hh][e]);
    }
    if (nxt < be) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kc[i] = kn[i];
        vc[i] = vn[i];
        okc[i] = okn[i];
      }
    }
  }

  // ---- wave result: sum the 4 row groups, then merge the waves in LDS
#pragma unroll
  for (int hh = 0; hh < GQ; ++hh)
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[hh][e] = sum_rows(o[hh][e]);
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      sm.wm[wid][hh] = m_run[hh];
      sm.wl[wid][hh] = l_run[hh];
    }
  }
  if (rg == 0) {
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh)
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm.ow[wid][hh * D + cc * EPL + e] = o[hh][e];
  }
  __syncthreads();
  if (tid < GQ) {
    float M = -__builtin_huge_valf();
    for (int w = 0; w < kAttWaves; ++w) M = fmaxf(M, sm.wm[w][tid]);
    float L = 0.f;
    for (int w = 0; w < kAttWaves; ++w) {
      const float mw = sm.wm[w][tid];
      const float wt = mw == -__builtin_huge_valf() ? 0.f : exp2f(mw - M);
      sm.wgt[w][tid] = wt;
      L += sm.wl[w][tid] * wt;
    }
    sm.M[tid] = M;
    sm.L[tid] = L;
  }
  __syncthreads();

  const int64_t row_id = static_cast<int64_t>(bh) * a.nq + qi;  // (b, kv head, query row)
  auto write_out = [&](int hh, int dd, float val) {
    const int64_t off = ((static_cast<int64_t>(b) * kp.Hq + h * GQ + hh) * a.nq + qi) * D + dd;
    if (a.out_bf16) reinterpret_cast<uint16_t*>(a.O)[off] = f32_to_bf16(val);
    else reinterpret_cast<float*>(a.O)[off] = val;
  };
  auto write_lse = [&](int hh, float mlog2, float lsum) {
    if (a.lse) {
      const int64_t off = (static_cast<int64_t>(b) * kp.Hq + h * GQ + hh) * a.nq + qi;
      a.lse[off] = (mlog2 + log2f(lsum)) * 0.69314718055994531f;
    }
  };
  auto wave_sum = [&](int e) {
    const int hh = e / D;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kAttWaves; ++w) v += sm.ow[w][e] * sm.wgt[w][hh];
    return v;
  };

  if (a.parts_total == 1) {
    for (int e = tid; e < GQ * D; e += kAttThreads) write_out(e / D, e % D, wave_sum(e) / sm.L[e / D]);
    if (tid < GQ) write_lse(tid, sm.M[tid], sm.L[tid]);
    return;
  }

  // ---- partial to the workspace: [o (GQ*D) | m (GQ) | l (GQ)], device-coherent stores
  const int stride = GQ * (D + 2);
  float* part = a.partials + (row_id * a.parts_total + a.part_offset + x) * stride;
  for (int e = tid; e < GQ * D; e += kAttThreads) st_agent(part + e, wave_sum(e));
  if (tid < GQ) {
    st_agent(part + GQ * D + tid, sm.M[tid]);
    st_agent(part + GQ * D + GQ + tid, sm.L[tid]);
  }
  if (!arrive_last(&a.counters[row_id], static_cast<uint32_t>(a.parts_total), &sm.is_last)) return;

  // ---- last workgroup: merge the parts (plain loads after the acquire).  The
  // output values of all parts are loaded together with their maxima and sums.
  const float* parts = a.partials + row_id * a.parts_total * stride;
  const int P = a.parts_total;
  constexpr int kOut = GQ * D / kAttThreads > 0 ? GQ * D / kAttThreads : 1;  // outputs per thread
  constexpr int kPR = 16;  // parts held in registers per pass
  float num[kOut];
#pragma unroll
  for (int r = 0; r < kOut; ++r) num[r] = 0.f;
  for (int p0 = 0; p0 < P; p0 += kPR) {
    const int np = min(kPR, P - p0);
    float ov[kPR][kOut];
#pragma unroll
    for (int q = 0; q < kPR; ++q)
#pragma unroll
      for (int r = 0; r < kOut; ++r) {
        const int e = tid + r * kAttThreads;
        ov[q][r] = (q < np && e < GQ * D) ? parts[(p0 + q) * stride + e] : 0.f;
      }
    for (int e = tid; e < np * GQ; e += kAttThreads) {
      const int p = p0 + e / GQ, hh = e % GQ;
      sm.pm[p * GQ + hh] = parts[p * stride + GQ * D + hh];
      sm.pl[p * GQ + hh] = parts[p * stride + GQ * D + GQ + hh];
    }
    __syncthreads();
    if (p0 == 0 && tid < GQ) {
      float M = -__builtin_huge_valf();
      for (int p = 0; p < P && p < kPR; ++p) M = fmaxf(M, sm.pm[p * GQ + tid]);
      sm.M[tid] = M;
    }
    if (p0 > 0 && tid < GQ) {
      float M = sm.M[tid];
      for (int p = p0; p < p0 + np; ++p) M = fmaxf(M, sm.pm[p * GQ + tid]);
      sm.M[tid] = M;
    }
    __syncthreads();
    if (P <= kPR) {
#pragma unroll
      for (int r = 0; r < kOut; ++r) {
        const int e = tid + r * kAttThreads;
        if (e >= GQ * D) continue;
        const int hh = e / D;
        const float M = sm.M[hh];
        for (int q = 0; q < np; ++q) {
          const float mp = sm.pm[q * GQ + hh];
          if (mp != -__builtin_huge_valf()) num[r] += exp2f(mp - M) * ov[q][r];
        }
      }
    }
  }
  if (P > kPR) {
    // second pass with the final maxima (rare: more than 16 parts per row)
    for (int r = 0; r < kOut; ++r) {
      const int e = tid + r * kAttThreads;
      if (e >= GQ * D) continue;
      const int hh = e / D;
      const float M = sm.M[hh];
      float acc = 0.f;
      for (int p = 0; p < P; ++p) {
        const float mp = sm.pm[p * GQ + hh];
        if (mp != -__builtin_huge_valf()) acc += exp2f(mp - M) * parts[p * stride + e];
      }
      num[r] = acc;
    }
  }
  if (tid < GQ) {
    const float M = sm.M[tid];
    float L = 0.f;
    for (int p = 0; p < P; ++p) {
      const float mp = sm.pm[p * GQ + tid];
      if (mp != -__builtin_huge_valf()) L += exp2f(mp - M) * sm.pl[p * GQ + tid];
    }
    sm.L[tid] = L;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kOut; ++r) {
    const int e = tid + r * kAttThreads;
    if (e >= GQ * D) continue;
    const int hh = e / D;
    write_out(hh, e % D, num[r] / sm.L[hh]);
    if (e % D == 0) write_lse(hh, sm.M[hh], sm.L[hh]);
  }
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
