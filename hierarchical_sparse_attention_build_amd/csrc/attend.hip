// Steps 4-5 of HGA on the vector ALUs: visibility union + exact softmax
// attention over the gathered original K/V rows, split over workgroups.
// [HGA technical summary (it), Meccanismo Core, item 2 third bullet (current,
// sink and recent local chunks always visible) and item 4 (standard softmax
// over the bounded exact token set; no summary enters the output)].
//
// Token slots of a query at position t in chunk j: first the forced chunks
// (sink + local + current, C slots each, tokens after t masked), then the
// routed groups (G slots each).  Slots are cut into tiles of 64; a workgroup
// takes a contiguous range of tiles and each of its four waves owns 16 rows of
// every tile, keeping its own running max / sum / output (online softmax, base
// 2).  Per tile a lane loads one quarter of a K row and of a V row (16-byte
// loads, 4 lanes per row): QK^T reduces over the 4 lanes, the V rows and the
// probabilities go through LDS and PV runs with lanes over output dims.  All
// query heads sharing the KV head are served by the same K/V loads.  The
// waves are merged in LDS; with several workgroups per query the partial
// (max, sum, output) goes to the workspace and the last workgroup (device
// counter) merges them.  In decode this kernel is bound by HBM bandwidth.
#include "hga_kernels.hpp"
#include "hga_device.hpp"

namespace hga {

constexpr int kAttThreads = 256;
constexpr int kAttWaves = kAttThreads / kWave;
constexpr int kRowsPerWave = kTileSlots / kAttWaves;  // 16

template <typename T, int D, int GQ>
struct AttSmem {
  static constexpr int kVRowBytes = D * static_cast<int>(sizeof(T)) + 16;  // padded against bank conflicts
  float q[GQ][D];
  float p[kAttWaves][kRowsPerWave][GQ];
  alignas(16) unsigned char v[kAttWaves][kRowsPerWave][kVRowBytes];
  float wm[kAttWaves][GQ];
  float wl[kAttWaves][GQ];
  int gl[1024];
  BlockScanSmem<kAttThreads> scan;
  int n_routed;
  int is_last;
};

struct SlotMap {
  Forced f;
  int C, G, nF_slots, n_slots;
};

template <typename T, int D, int GQ>
__global__ __launch_bounds__(kAttThreads) void attend_splitk_kernel(AttendArgs a) {
  constexpr int QD = D / 4;          // dims per lane in the QK layout
  constexpr int DPL = D / kWave;     // dims per lane in the PV layout
  static_assert(DPL >= 1, "head_dim >= 64");
  const KParams& kp = a.kp;
  const int bh = blockIdx.z;
  const int qi = blockIdx.y;
  const int x = blockIdx.x;
  const int b = bh / kp.Hkv;
  const int h = bh % kp.Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int t_row0 = (a.q_pos ? a.q_pos[b] : 0) + a.pos_bias;
  const int t = t_row0 + qi;
  const int j = t / kp.C;
  const int u = a.nq == 1 ? 0 : j - t_row0 / kp.C;

  __shared__ AttSmem<T, D, GQ> sm;

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

  // ---- query rows of the GQ heads (pre-scaled to base-2 logits), group list
  const T* Qb = static_cast<const T*>(a.Q);
  for (int e = tid; e < GQ * D; e += kAttThreads) {
    const int hh = e / D, dd = e % D;
    const int64_t off = ((static_cast<int64_t>(b) * kp.Hq + h * GQ + hh) * a.nq + qi) * D + dd;
    sm.q[hh][dd] = elem<T>::get(Qb, off) * kp.scale_log2;
  }
  // routed groups of the unit, compacted (-1 and out-of-range ids dropped)
  {
    const int32_t* gl = a.group_idx + (static_cast<int64_t>(bh) * a.n_units + u) * kp.top_g;
    const int n_groups_cap = static_cast<int>(kp.n_cap / kp.G);
    const int per = (kp.top_g + kAttThreads - 1) / kAttThreads;
    const int e0 = min(kp.top_g, tid * per), e1 = min(kp.top_g, e0 + per);
    int cnt = 0;
    for (int e = e0; e < e1; ++e) {
      const int g = gl[e];
      cnt += (g >= 0 && g < n_groups_cap);
    }
    int tot;
    int pos = block_excl_scan<kAttThreads>(cnt, tot, sm.scan);
    for (int e = e0; e < e1; ++e) {
      const int g = gl[e];
      if (g >= 0 && g < n_groups_cap) sm.gl[pos++] = g;
    }
    if (tid == 0) sm.n_routed = tot;
  }
  __syncthreads();

  SlotMap sl;
  sl.f = forced_chunks(j, kp.n_sink, kp.n_local);
  sl.C = kp.C;
  sl.G = kp.G;
  sl.nF_slots = sl.f.n * kp.C;
  sl.n_slots = sl.nF_slots + sm.n_routed * kp.G;
  int R0 = 0, R1 = sl.n_slots;
  if (a.part == 1) R1 = sl.nF_slots;
  if (a.part == 2) R0 = sl.nF_slots;
  const int ntiles = (R1 - R0 + kTileSlots - 1) / kTileSlots;
  const int tb = min(ntiles, x * a.tiles_per_split);
  const int te = min(ntiles, tb + a.tiles_per_split);

  const T* Kb = static_cast<const T*>(a.K);
  const T* Vb = static_cast<const T*>(a.V);
  const T* Ks = static_cast<const T*>(a.K_stage);
  const T* Vs = static_cast<const T*>(a.V_stage);
  const int r_in_wave = lane >> 2;
  const int qd = lane & 3;

  float m_w[GQ], l_w[GQ], o_acc[GQ][DPL];
#pragma unroll
  for (int hh = 0; hh < GQ; ++hh) {
    m_w[hh] = -__builtin_huge_valf();
    l_w[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o_acc[hh][e] = 0.f;
  }

  for (int tile = tb; tile < te; ++tile) {
    // ---- which token this lane's row holds
    const int slot = R0 + tile * kTileSlots + wid * kRowsPerWave + r_in_wave;
    bool valid = slot < R1;
    const T* krow = nullptr;
    const T* vrow = nullptr;
    if (valid) {
      int64_t tok, row;
      if (slot < sl.nF_slots) {
        const int fi = slot / sl.C, off = slot % sl.C;
        const int c = forced_chunk_at(sl.f, fi);
        tok = static_cast<int64_t>(c) * sl.C + off;
        int64_t hs = c;
        if (a.kv.ring && c >= kp.n_sink) hs = kp.n_sink + (c - kp.n_sink) % (kp.n_local + 1);
        row = static_cast<int64_t>(bh) * a.kv.bh_rows + hs * sl.C + off;
        krow = Kb + row * D;
        vrow = Vb + row * D;
      } else {
        const int rs = slot - sl.nF_slots;
        const int g = sm.gl[rs / sl.G];
        tok = static_cast<int64_t>(g) * sl.G + rs % sl.G;
        if (Ks) {
          row = static_cast<int64_t>(bh) * kp.top_g * sl.G + rs;
          krow = Ks + row * D;
          vrow = Vs + row * D;
        } else {
          row = static_cast<int64_t>(bh) * a.kv.bh_rows + tok;
          krow = Kb + row * D;
          vrow = Vb + row * D;
        }
      }
      valid = tok <= t;
    }
    float kf[QD], vf[QD];
    if (valid) {
      load_row<T, QD>(krow + qd * QD, kf);
      load_row<T, QD>(vrow + qd * QD, vf);
    } else {
#pragma unroll
      for (int e = 0; e < QD; ++e) kf[e] = vf[e] = 0.f;
    }
    // ---- scores (base 2) of this row for every head
    float s[GQ];
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      const float4* q4 = reinterpret_cast<const float4*>(&sm.q[hh][qd * QD]);
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < QD / 4; ++e) {
        const float4 qq = q4[e];
        acc = fmaf(qq.x, kf[4 * e + 0], acc);
        acc = fmaf(qq.y, kf[4 * e + 1], acc);
        acc = fmaf(qq.z, kf[4 * e + 2], acc);
        acc = fmaf(qq.w, kf[4 * e + 3], acc);
      }
      acc += __shfl_xor(acc, 1, kWave);
      acc += __shfl_xor(acc, 2, kWave);
      s[hh] = valid ? acc : -__builtin_huge_valf();
    }
    // ---- online softmax update of this wave's 16 rows
    float alpha[GQ];
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      float tm = s[hh];
      tm = wave_xor_max(tm, 4);
      tm = wave_xor_max(tm, 8);
      tm = wave_xor_max(tm, 16);
      tm = wave_xor_max(tm, 32);
      const float m_new = fmaxf(m_w[hh], tm);
      alpha[hh] = m_new == -__builtin_huge_valf() ? 1.f : exp2f(m_w[hh] - m_new);
      const float p = valid ? exp2f(s[hh] - m_new) : 0.f;
      float ps = qd == 0 ? p : 0.f;
      ps += __shfl_xor(ps, 4, kWave);
      ps += __shfl_xor(ps, 8, kWave);
      ps += __shfl_xor(ps, 16, kWave);
      ps += __shfl_xor(ps, 32, kWave);
      l_w[hh] = l_w[hh] * alpha[hh] + ps;
      m_w[hh] = m_new;
      if (qd == 0) sm.p[wid][r_in_wave][hh] = p;
    }
    // ---- V rows to LDS (as stored), then PV with lanes over output dims
    {
      unsigned char* dst = &sm.v[wid][r_in_wave][0] + qd * QD * static_cast<int>(sizeof(T));
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < QD / 8; ++e) {
          uint4 w;
          w.x = (__float_as_uint(vf[8 * e + 0]) >> 16) | (__float_as_uint(vf[8 * e + 1]) & 0xffff0000u);
          w.y = (__float_as_uint(vf[8 * e + 2]) >> 16) | (__float_as_uint(vf[8 * e + 3]) & 0xffff0000u);
          w.z = (__float_as_uint(vf[8 * e + 4]) >> 16) | (__float_as_uint(vf[8 * e + 5]) & 0xffff0000u);
          w.w = (__float_as_uint(vf[8 * e + 6]) >> 16) | (__float_as_uint(vf[8 * e + 7]) & 0xffff0000u);
          reinterpret_cast<uint4*>(dst)[e] = w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < QD / 4; ++e)
          reinterpret_cast<float4*>(dst)[e] = make_float4(vf[4 * e], vf[4 * e + 1], vf[4 * e + 2], vf[4 * e + 3]);
      }
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh)
#pragma unroll
      for (int e = 0; e < DPL; ++e) o_acc[hh][e] *= alpha[hh];
#pragma unroll 4
    for (int r = 0; r < kRowsPerWave; ++r) {
      float vv[DPL];
      const unsigned char* src = &sm.v[wid][r][0];
      if constexpr (sizeof(T) == 2) {
        if constexpr (DPL == 2) {
          const uint32_t w = reinterpret_cast<const uint32_t*>(src)[lane];
          vv[0] = bf16lo(w);
          vv[1] = bf16hi(w);
        } else {
          vv[0] = bf16_to_f32(reinterpret_cast<const uint16_t*>(src)[lane]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < DPL; ++e) vv[e] = reinterpret_cast<const float*>(src)[lane * DPL + e];
      }
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) {
        const float p = sm.p[wid][r][hh];
#pragma unroll
        for (int e = 0; e < DPL; ++e) o_acc[hh][e] = fmaf(p, vv[e], o_acc[hh][e]);
      }
    }
    __syncthreads();
  }

  // ---- merge the four waves
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      sm.wm[wid][hh] = m_w[hh];
      sm.wl[wid][hh] = l_w[hh];
    }
  }
  __syncthreads();
  float M[GQ], L[GQ], wgt[GQ];
#pragma unroll
  for (int hh = 0; hh < GQ; ++hh) {
    M[hh] = -__builtin_huge_valf();
    for (int w = 0; w < kAttWaves; ++w) M[hh] = fmaxf(M[hh], sm.wm[w][hh]);
    L[hh] = 0.f;
    for (int w = 0; w < kAttWaves; ++w) {
      const float mw = sm.wm[w][hh];
      if (mw != -__builtin_huge_valf()) L[hh] += sm.wl[w][hh] * exp2f(mw - M[hh]);
    }
    wgt[hh] = m_w[hh] == -__builtin_huge_valf() ? 0.f : exp2f(m_w[hh] - M[hh]);
  }
  __syncthreads();
  // o of the block, summed over waves through LDS (reuse the V area as floats)
  float* osum = reinterpret_cast<float*>(&sm.v[0][0][0]);  // GQ*D floats fit: 4*16*(D*sizeof(T)+16) >= GQ*D*4 for GQ<=16
  for (int e = tid; e < GQ * D; e += kAttThreads) osum[e] = 0.f;
  __syncthreads();
  for (int w = 0; w < kAttWaves; ++w) {
    if (wid == w) {
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh)
#pragma unroll
        for (int e = 0; e < DPL; ++e) osum[hh * D + lane * DPL + e] += o_acc[hh][e] * wgt[hh];
    }
    __syncthreads();
  }

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

  if (a.parts_total == 1) {
    for (int e = tid; e < GQ * D; e += kAttThreads) {
      const int hh = e / D;
      write_out(hh, e % D, osum[e] / L[hh]);
    }
    if (tid < GQ) write_lse(tid, M[tid], L[tid]);
    return;
  }

  // ---- partial to the workspace: [o (GQ*D) | m (GQ) | l (GQ)]
  const int stride = GQ * (D + 2);
  float* part = a.partials + (row_id * a.parts_total + a.part_offset + x) * stride;
  for (int e = tid; e < GQ * D; e += kAttThreads) st_agent(part + e, osum[e]);
  if (tid < GQ) {
    st_agent(part + GQ * D + tid, M[tid]);
    st_agent(part + GQ * D + GQ + tid, L[tid]);
  }
  if (!arrive_last(&a.counters[row_id], static_cast<uint32_t>(a.parts_total), &sm.is_last)) return;
  const float* parts = a.partials + row_id * a.parts_total * stride;
  for (int e = tid; e < GQ * D; e += kAttThreads) {
    const int hh = e / D;
    float mx = -__builtin_huge_valf();
    for (int p = 0; p < a.parts_total; ++p) mx = fmaxf(mx, ld_agent(parts + p * stride + GQ * D + hh));
    float num = 0.f, den = 0.f;
    for (int p = 0; p < a.parts_total; ++p) {
      const float mp = ld_agent(parts + p * stride + GQ * D + hh);
      if (mp == -__builtin_huge_valf()) continue;
      const float w = exp2f(mp - mx);
      num += w * ld_agent(parts + p * stride + e);
      den += w * ld_agent(parts + p * stride + GQ * D + GQ + hh);
    }
    write_out(hh, e % D, num / den);
    if (e % D == 0) write_lse(hh, mx, den);
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
