// Step 5 of HGA: exact softmax attention of one query row (all query heads
// that share a KV head) over a list of token slots, the building block of the
// decode and generic attention kernels.
// [HGA technical summary (it), Meccanismo Core, item 4: standard softmax over
// the bounded set of exact tokens; no summary enters the output].
//
// Two lane engines share the block walk and the merge below (AttnLaneSel picks
// one): AttnLane does the arithmetic on the vector ALUs (fp32 inputs);
// AttnLaneMfma (bf16 inputs) puts QK^T and PV of each pair of 16-row blocks on
// v_mfma_f32_16x16x32_bf16, the query heads padded to 16 columns.  Decode
// moves a few bytes per FLOP either way, so the matrix cores serve here to cut
// vector-ALU instructions per byte, not for their FLOP rate.
//
// AttnLane: slots are cut into blocks of 16 rows.  A wave walks its blocks with an
// online softmax in base 2 and no LDS or barrier: lane (g, c) holds rows g,
// g+4, g+8, g+12 of the block and the c-th sixteenth of each row, so one load
// instruction fetches four whole rows; QK^T reduces over the 16 lanes of a row
// with DPP, the block max and sum over the 4 row groups with permlane swaps,
// and PV accumulates per lane into its sixteenth of the output.  Up to PF
// blocks are in flight: a block's registers are refilled with the loads of a
// later block as soon as it has been computed.
//
// Afterwards the waves of a workgroup merge in LDS; the workgroup's result is
// either final (written to O) or a partial (max, sum, output) published to the
// workspace with device-coherent stores, and the last of the parts of a row
// merges them.
#pragma once
#include <type_traits>

#include "hga_device.hpp"
#include "hga_kparams.hpp"

namespace hga {

constexpr int kAttnBlock = 16;   // rows per block
constexpr int kAttnMaxParts = 128;

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
__device__ __forceinline__ void store_raw(void* p, const RawVec<BYTES>& r) {
  if constexpr (BYTES == 8) *reinterpret_cast<uint2*>(p) = r.v;
  else if constexpr (BYTES == 16) *reinterpret_cast<uint4*>(p) = r.v;
  else {
    reinterpret_cast<uint4*>(p)[0] = r.v0;
    reinterpret_cast<uint4*>(p)[1] = r.v1;
  }
}

// Row write-back of the lane engines' run(): wb(s, kdst, vdst) returns true
// and sets where the K and V rows of slot s, as loaded, are also stored (the
// warm tier's missing groups, read from host memory, go into their cache
// slots on the way).  The default stores nothing and compiles to nothing.
struct NoWriteBack {
  template <typename P>
  __device__ __forceinline__ bool operator()(int, P*&, P*&) const { return false; }
};

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

// Per-lane state of one wave: its sixteenth of the GQ query rows and the
// running (max, sum, output) of every head.
template <typename T, int D, int GQ>
struct AttnLane {
  static constexpr int EPL = D / 16;                            // elements of a row per lane
  static constexpr int RB = EPL * static_cast<int>(sizeof(T));  // bytes of a row per lane
  static constexpr bool kBF = sizeof(T) == 2;
  uint32_t qbf[GQ][kBF ? EPL / 2 : 1];
  float qf[kBF ? 1 : GQ][kBF ? 1 : EPL];
  float m_run[GQ], l_run[GQ], o[GQ][EPL];
  __device__ __forceinline__ void finish() {}

  // q(hh) points at the row of head hh; cc = lane's sixteenth
  template <typename QFn>
  __device__ __forceinline__ void init(QFn q, int cc) {
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      const RawVec<RB> r = load_raw<RB>(q(hh) + cc * EPL);
      if constexpr (kBF) {
#pragma unroll
        for (int w = 0; w < EPL / 2; ++w) qbf[hh][w] = word(r, w);
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) qf[hh][e] = __uint_as_float(word(r, e));
      }
      m_run[hh] = -__builtin_huge_valf();
      l_run[hh] = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[hh][e] = 0.f;
    }
  }

  // Attend blocks blk = first, first + step, ... < end of the slot list that
  // starts at slot R0, with up to PF blocks in flight.  row(s, kptr, vptr)
  // sets the K and V row pointers of slot s and returns false for a masked
  // slot; it must then still point them at a readable row of finite values
  // (its score is replaced by -inf, so that row's values get weight 0).
  template <int PF = 2, typename RowFn, typename WbFn = NoWriteBack>
  __device__ __forceinline__ void run(int R0, int first, int end, int step, float scale_log2, RowFn row,
                                      WbFn wb = WbFn{}) {
    const int lane = threadIdx.x & (kWave - 1);
    const int rg = lane >> 4;
    const int cc = lane & 15;
    // blocks of this wave (wave-uniform, so that the block loop branches on the scalar unit)
    const int n = __builtin_amdgcn_readfirstlane(first < end ? (end - first + step - 1) / step : 0);
    RawVec<RB> kb[PF][4], vb[PF][4];
    bool okb[PF][4];
    auto fetch = [&](int blkid, RawVec<RB>* kr, RawVec<RB>* vr, bool* ok) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int s = R0 + blkid * kAttnBlock + rg + 4 * i;
        const T* kp;
        const T* vp;
        ok[i] = row(s, kp, vp);
        kr[i] = load_raw<RB>(kp + cc * EPL);
        vr[i] = load_raw<RB>(vp + cc * EPL);
        T* kd;
        T* vd;
        if (wb(s, kd, vd)) {
          store_raw<RB>(kd + cc * EPL, kr[i]);
          store_raw<RB>(vd + cc * EPL, vr[i]);
        }
      }
    };
    // fill the ring, then consume block c from slot c % PF and refill it with block c + PF
#pragma unroll
    for (int p = 0; p < PF; ++p)
      if (p < n) fetch(first + p * step, kb[p], vb[p], okb[p]);
    for (int c0 = 0; c0 < n; c0 += PF) {
#pragma unroll
      for (int p = 0; p < PF; ++p) {
        const int c = c0 + p;
        if (c < n) {
          block(kb[p], vb[p], okb[p], scale_log2);
          if (c + PF < n) fetch(first + (c + PF) * step, kb[p], vb[p], okb[p]);
        }
      }
    }
  }

  // one block of 16 rows: QK^T, online softmax, PV
  __device__ __forceinline__ void block(const RawVec<RB> (&kc)[4], const RawVec<RB> (&vc)[4], const bool (&okc)[4],
                                        float scale_log2) {
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
        s[i][hh] = okc[i] ? acc * scale_log2 : -__builtin_huge_valf();
      }
    }
    // ---- online softmax over this block's 16 rows.  The block max is the
    // same in every lane, so the rescale of the running state (only when the
    // max rises) is a wave-uniform branch.
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      float bm = fmaxf(fmaxf(s[0][hh], s[1][hh]), fmaxf(s[2][hh], s[3][hh]));
      bm = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, max_rows(bm))));
      if (bm > m_run[hh]) {
        const float alpha = __builtin_amdgcn_exp2f(m_run[hh] - bm);  // 0 when m_run = -inf
        l_run[hh] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[hh][e] *= alpha;
        m_run[hh] = bm;
      }
      const float mref = m_run[hh] == -__builtin_huge_valf() ? 0.f : m_run[hh];
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(s[i][hh] - mref);  // 0 for a masked row
        s[i][hh] = p;
        ps += p;
      }
      l_run[hh] += sum_rows(ps);
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
  }

  // (no LDS staging on this path)
  __device__ __forceinline__ void set_tile(unsigned char*) {}

  // This wave's unnormalised output, ow[hh * D + d] for every head hh < GQ:
  // the four row groups are summed first.
  __device__ __forceinline__ void store_o(float* ow) {
    const int lane = threadIdx.x & (kWave - 1);
    const int rg = lane >> 4;
    const int cc = lane & 15;
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh)
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[hh][e] = sum_rows(o[hh][e]);
    if (rg == 0) {
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh)
#pragma unroll
        for (int e = 0; e < EPL; ++e) ow[hh * D + cc * EPL + e] = o[hh][e];
    }
  }
};

// The same per-wave attention for bf16 inputs on the matrix cores, two
// 16-row blocks at a time.
//   S = K Q^T   v_mfma_f32_16x16x32_bf16 per block, the K rows as the A operand
//               and the query heads as the B operand (head l%16, zero-padded
//               to 16): lane (g, h) = (l/16, l%16) gets S[row 4g+i][head h],
//               item i.  K rows are loaded like V rows (each load instruction
//               covers four whole rows, so every cache line is fetched once
//               and in full) and pass through a per-wave LDS tile to reach the
//               operand layout (lane l: 16 bytes of row l%16).
//   O += P V    v_mfma_f32_16x16x32_bf16 with the 32 rows of the block pair as
//               the reduction index, ordered k = 8g + 4b + i for row 4g+i of
//               block b.  In that order lane (g, h) already holds the A
//               operand P[h][k] (its own scores), and lane (g, c) the B
//               operand for output column d = c*(D/16) + e: element e of the
//               rows 4g..4g+3 it loaded from each block (one v_perm_b32 per
//               pair of rows).  P (<= 1) enters as the sum of two bf16 values,
//               hi = bf16(p) and lo = bf16(p - hi), so it keeps 16 significant
//               bits; V is bf16 already, and the products accumulate in fp32.
// O lands as O[head 4g+i][column c*(D/16)+e] in lane (g, c), item i of
// accumulator e.  The softmax statistics are per head as in AttnLane.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// LDS bytes per wave for the matrix-core path's K tile (16 rows of D bf16, padded)
template <int D>
__host__ __device__ constexpr int attn_ktile_bytes() { return 16 * (D + 8) * 2; }

// two floats rounded to bf16 (to nearest even), packed low first
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

template <int D, int GQ>
struct AttnLaneMfma {
  static_assert(GQ <= 16, "at most 16 query heads per KV head");
  static constexpr int EPL = D / 16;  // output columns per lane
  static constexpr int RB = EPL * 2;  // bytes of a V row per lane
  static constexpr int KS = D / 32;   // MFMA steps of QK^T over the head dimension
  static constexpr int KROWB = (D + 8) * 2;  // bytes per LDS tile row (padded against bank conflicts)
  bf16x8_t qb[KS];
  float m_run[GQ], l_run[GQ];
  // GQ > 4: the running max and sum of head (lane & 15) live in the four lanes
  // of that head (m_run / l_run are filled from them by finish())
  float m_lane, l_lane;
  f32x4_t acc[EPL];
  unsigned char* kt;  // this wave's LDS tile of 16 K rows

  // base: an LDS area of attn_ktile_bytes<D>() bytes per wave of the workgroup
  __device__ __forceinline__ void set_tile(unsigned char* base) { kt = base + wave_id() * 16 * KROWB; }

  template <typename QFn>
  __device__ __forceinline__ void init(QFn q, int /*cc*/) {
    const int lane = threadIdx.x & (kWave - 1);
    const int h = lane & 15;
    const int g = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 w = make_uint4(0u, 0u, 0u, 0u);
      if (h < GQ) w = *reinterpret_cast<const uint4*>(q(h < GQ ? h : 0) + ks * 32 + g * 8);
      qb[ks] = __builtin_bit_cast(bf16x8_t, w);
    }
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      m_run[hh] = -__builtin_huge_valf();
      l_run[hh] = 0.f;
    }
    m_lane = -__builtin_huge_valf();
    l_lane = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // per-head statistics into m_run / l_run (head hh from lane hh)
  __device__ __forceinline__ void finish() {
    if constexpr (GQ > 4) {
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) {
        m_run[hh] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, m_lane), hh));
        l_run[hh] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, l_lane), hh));
      }
    }
  }

  struct Buf {
    RawVec<RB> k[4];       // K rows 4g+i, the lane's columns
    RawVec<RB> v[4];       // V rows 4g+i, the lane's columns
    uint32_t ok;           // bit r: row r of the block is visible
  };

  template <typename RowFn, typename WbFn>
  __device__ __forceinline__ void fetch(int R0, int blkid, Buf& b, RowFn row, WbFn& wb) {
    const int lane = threadIdx.x & (kWave - 1);
    const int g = lane >> 4;
    const int cc = lane & 15;
    const int s0 = R0 + blkid * kAttnBlock;
    uint32_t okm = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16* kp;
      const bf16* vp;
      const bool ok = row(s0 + 4 * g + i, kp, vp);
      b.k[i] = load_raw<RB>(kp + cc * EPL);
      b.v[i] = load_raw<RB>(vp + cc * EPL);
      bf16* kd;
      bf16* vd;
      if (wb(s0 + 4 * g + i, kd, vd)) {
        store_raw<RB>(kd + cc * EPL, b.k[i]);
        store_raw<RB>(vd + cc * EPL, b.v[i]);
      }
      // row 4g+i is visible iff lane 16g saw ok
      const uint64_t m = __ballot(ok);
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) okm |= static_cast<uint32_t>((m >> (16 * gg)) & 1u) << (4 * gg + i);
    }
    b.ok = okm;
  }

  // Without write-back the loads of a round go out as every block's K rows
  // (and visibility bits), then every block's V rows: the scores need only
  // the K rows, so they start while the V rows are still in flight
  // (decode_32k 20.71 against 20.90 us per step, streaming heads 12.77
  // against 12.98).
  template <typename RowFn>
  __device__ __forceinline__ void fetch_k(int R0, int blkid, Buf& b, RowFn row) {
    const int lane = threadIdx.x & (kWave - 1);
    const int g = lane >> 4;
    const int cc = lane & 15;
    const int s0 = R0 + blkid * kAttnBlock;
    uint32_t okm = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16* kp;
      const bf16* vp;
      const bool ok = row(s0 + 4 * g + i, kp, vp);
      b.k[i] = load_raw<RB>(kp + cc * EPL);
      const uint64_t m = __ballot(ok);
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) okm |= static_cast<uint32_t>((m >> (16 * gg)) & 1u) << (4 * gg + i);
    }
    b.ok = okm;
  }
  template <typename RowFn>
  __device__ __forceinline__ void fetch_v(int R0, int blkid, Buf& b, RowFn row) {
    const int lane = threadIdx.x & (kWave - 1);
    const int g = lane >> 4;
    const int cc = lane & 15;
    const int s0 = R0 + blkid * kAttnBlock;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16* kp;
      const bf16* vp;
      row(s0 + 4 * g + i, kp, vp);
      b.v[i] = load_raw<RB>(vp + cc * EPL);
    }
  }

  // S[row 4g+i][head h] (raw dot products) of one block: its K rows go
  // through the tile into the A operand layout.
  __device__ __forceinline__ f32x4_t scores(const Buf& b) {
    const int lane = threadIdx.x & (kWave - 1);
    const int g = lane >> 4;
    const int cc = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<RawVec<RB>*>(kt + (4 * g + i) * KROWB + cc * RB) = b.k[i];
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 a = *reinterpret_cast<const uint4*>(kt + cc * KROWB + (ks * 32 + g * 8) * 2);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), qb[ks], s, 0, 0, 0);
    }
    return s;
  }

  // Blocks blk = first, first + step, ... < end, in rounds of PF (even): the
  // loads of a round's blocks are all issued before its first pair is computed.
  template <int PF = 2, typename RowFn, typename WbFn = NoWriteBack>
  __device__ __forceinline__ void run(int R0, int first, int end, int step, float scale_log2, RowFn row,
                                      WbFn wb = WbFn{}) {
    static_assert(PF % 2 == 0, "blocks are computed in pairs");
    // blocks of this wave (wave-uniform, so that the block loop branches on the scalar unit)
    const int n = __builtin_amdgcn_readfirstlane(first < end ? (end - first + step - 1) / step : 0);
    auto compute = [&](int c0, Buf (&buf)[PF]) {
#pragma unroll
      for (int p = 0; p < PF; p += 2) {
        if (c0 + p >= n) break;
        const bool has1 = c0 + p + 1 < n;
        if (!has1) {
          buf[p + 1].ok = 0u;
#pragma unroll
          for (int i = 0; i < 4; ++i) buf[p + 1].v[i] = zero_raw<RB>();
        }
        pair(buf[p], buf[p + 1], has1, scale_log2);
      }
    };
    auto load = [&](int c0, Buf (&buf)[PF]) {
      if constexpr (std::is_same<WbFn, NoWriteBack>::value) {
#pragma unroll
        for (int p = 0; p < PF; ++p)
          if (c0 + p < n) fetch_k(R0, first + (c0 + p) * step, buf[p], row);
#pragma unroll
        for (int p = 0; p < PF; ++p)
          if (c0 + p < n) fetch_v(R0, first + (c0 + p) * step, buf[p], row);
      } else {
#pragma unroll
        for (int p = 0; p < PF; ++p)
          if (c0 + p < n) fetch(R0, first + (c0 + p) * step, buf[p], row, wb);
      }
    };
    for (int c0 = 0; c0 < n; c0 += PF) {
      Buf buf[PF];
      load(c0, buf);
      compute(c0, buf);
    }
  }

  __device__ __forceinline__ void pair(const Buf& b0, const Buf& b1, bool has1, float scale_log2) {
    const int lane = threadIdx.x & (kWave - 1);
    const int g = lane >> 4;
    const int h = lane & 15;
    // ---- S of both blocks, base 2, masked rows -inf
    const f32x4_t s0 = scores(b0);
    f32x4_t s1 = {0.f, 0.f, 0.f, 0.f};
    if (has1) s1 = scores(b1);
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = (b0.ok >> (4 * g + i)) & 1u ? s0[i] * scale_log2 : -__builtin_huge_valf();
      sv[4 + i] = (b1.ok >> (4 * g + i)) & 1u ? s1[i] * scale_log2 : -__builtin_huge_valf();
    }
    // ---- pair max of head h (same in the 4 lanes of the head), then per head
    // in scalar registers: rescale only when the running max rises
    float bm_lane = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) bm_lane = fmaxf(bm_lane, sv[i]);
    bm_lane = max_rows(bm_lane);
    float mh = 0.f;
    if constexpr (GQ <= 4) {
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh) {
        const float bm = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bm_lane), hh));
        if (bm > m_run[hh]) {
          const float alpha = __builtin_amdgcn_exp2f(m_run[hh] - bm);  // 0 when m_run = -inf
          l_run[hh] *= alpha;
          // head hh sits in item hh%4 of the lanes with g = hh/4 (g = 0 here)
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[e][hh & 3] *= alpha;
          m_run[hh] = bm;
        }
        const float mref = m_run[hh] == -__builtin_huge_valf() ? 0.f : m_run[hh];
        mh = h == hh ? mref : mh;
      }
    } else {
      // every head at once: its four lanes hold its pair max; a rise anywhere
      // rescales, the accumulator item i of lane (g, c) (head 4g+i) by the
      // factor of lane 4g+i
      const bool rise = h < GQ && bm_lane > m_lane;
      if (__ballot(rise)) {
        const float alpha = rise ? __builtin_amdgcn_exp2f(m_lane - bm_lane) : 1.f;  // 0 when m_lane = -inf
        l_lane *= alpha;
        m_lane = rise ? bm_lane : m_lane;
        float a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = __shfl(alpha, 4 * g + i);
#pragma unroll
        for (int e = 0; e < EPL; ++e)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[e][i] *= a[i];
      }
      mh = m_lane == -__builtin_huge_valf() ? 0.f : m_lane;
    }
    float p[8], ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = __builtin_amdgcn_exp2f(sv[i] - mh);  // 0 for a masked row
      ps += p[i];
    }
    ps = sum_rows(ps);
    if constexpr (GQ <= 4) {
#pragma unroll
      for (int hh = 0; hh < GQ; ++hh)
        l_run[hh] += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ps), hh));
    } else {
      l_lane += ps;
    }
    // ---- P as hi + lo bf16 pairs (A operand, k = 8g + 4b + i)
    uint4 phi, plo;
    uint32_t* hw = reinterpret_cast<uint32_t*>(&phi);
    uint32_t* lw = reinterpret_cast<uint32_t*>(&plo);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t x = pack_bf16x2(p[2 * w], p[2 * w + 1]);
      hw[w] = x;
      lw[w] = pack_bf16x2(p[2 * w] - __uint_as_float(x << 16), p[2 * w + 1] - __uint_as_float(x & 0xffff0000u));
    }
    const bf16x8_t ahi = __builtin_bit_cast(bf16x8_t, phi);
    const bf16x8_t alo = __builtin_bit_cast(bf16x8_t, plo);
    // ---- PV: B operand of column e = element e of the lane's rows (k order)
    uint4 vb[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;  // high or low halves
      const int wi = e >> 1;
      vb[e].x = __builtin_amdgcn_perm(word(b0.v[1], wi), word(b0.v[0], wi), sel);
      vb[e].y = __builtin_amdgcn_perm(word(b0.v[3], wi), word(b0.v[2], wi), sel);
      vb[e].z = __builtin_amdgcn_perm(word(b1.v[1], wi), word(b1.v[0], wi), sel);
      vb[e].w = __builtin_amdgcn_perm(word(b1.v[3], wi), word(b1.v[2], wi), sel);
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, __builtin_bit_cast(bf16x8_t, vb[e]), acc[e], 0, 0, 0);
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, __builtin_bit_cast(bf16x8_t, vb[e]), acc[e], 0, 0, 0);
  }

  // This wave's unnormalised output, ow[hh * D + d] for every head hh < GQ.
  __device__ __forceinline__ void store_o(float* ow) const {
    const int lane = threadIdx.x & (kWave - 1);
    const int g = lane >> 4;
    const int c = lane & 15;
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh)
      if (g == (hh >> 2)) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) ow[hh * D + c * EPL + e] = acc[e][hh & 3];
      }
  }
};

// The per-wave attention used for element type T: the matrix-core version for bf16.
template <typename T, int D, int GQ>
struct AttnLaneSel {
  using type = AttnLane<T, D, GQ>;
};
template <int D, int GQ>
struct AttnLaneSel<bf16, D, GQ> {
  using type = AttnLaneMfma<D, GQ>;
};
template <typename T, int D, int GQ>
using AttnLaneFor = typename AttnLaneSel<T, D, GQ>::type;

// LDS of the workgroup merge (NWV waves) and of the parts merge.
template <int GQ, int D, int NWV>
struct AttnMergeSmem {
  float wm[NWV][GQ];
  float wl[NWV][GQ];
  float wgt[NWV][GQ];
  float L[GQ];
  float M[GQ];
  float ow[NWV][GQ * D];
  float pm[kAttnMaxParts * GQ];  // parts merge: per-part max
  float pl[kAttnMaxParts * GQ];  // and sum
  int is_last;
};

// Destination of a finished row: O (fp32 or bf16) and the optional lse, for
// query head h0 + hh of row qi.
struct AttnOut {
  void* O;
  float* lse;
  int32_t out_bf16;
  int64_t head0;   // b * Hq + first query head of the group
  int64_t nq;
  int64_t qi;
  template <int D>
  __device__ __forceinline__ void put(int hh, int dd, float v) const {
    const int64_t off = ((head0 + hh) * nq + qi) * D + dd;
    if (out_bf16) reinterpret_cast<uint16_t*>(O)[off] = f32_to_bf16(v);
    else reinterpret_cast<float*>(O)[off] = v;
  }
  __device__ __forceinline__ void put_lse(int hh, float mlog2, float lsum) const {
    if (lse) lse[(head0 + hh) * nq + qi] = (mlog2 + log2f(lsum)) * 0.69314718055994531f;
  }
  // NaN output (a position outside the cache)
  template <int D, int NT>
  __device__ __forceinline__ void put_nan(int GQn) const {
    for (int e = threadIdx.x; e < GQn * D; e += NT) {
      const int64_t off = ((head0 + e / D) * nq + qi) * D + e % D;
      if (out_bf16) reinterpret_cast<uint16_t*>(O)[off] = 0x7fc0u;
      else reinterpret_cast<float*>(O)[off] = __builtin_nanf("");
    }
    if (lse && static_cast<int>(threadIdx.x) < GQn) lse[(head0 + threadIdx.x) * nq + qi] = __builtin_nanf("");
  }
};

// Merge the waves of the workgroup: after it, wg_value(e) is the workgroup's
// unnormalised output element e (head e / D), sm.M / sm.L its max and sum.
// Each wave's raw (max, sum, unnormalised output) into sm.wm / wl / ow, then a
// barrier.
template <typename Lane, int D, int GQ, int NWV>
__device__ __forceinline__ void attn_waves_to_lds(Lane& st, AttnMergeSmem<GQ, D, NWV>& sm) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  st.finish();
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
      sm.wm[wid][hh] = st.m_run[hh];
      sm.wl[wid][hh] = st.l_run[hh];
    }
  }
  st.store_o(sm.ow[wid]);
  __syncthreads();
}

// After attn_waves_to_lds: the per-head max, sum and wave weights.
template <int D, int GQ, int NWV>
__device__ __forceinline__ void attn_merge_waves_rest(AttnMergeSmem<GQ, D, NWV>& sm) {
  if (static_cast<int>(threadIdx.x) < GQ) {
    const int hh = threadIdx.x;
    float M = -__builtin_huge_valf();
    for (int w = 0; w < NWV; ++w) M = fmaxf(M, sm.wm[w][hh]);
    float L = 0.f;
    for (int w = 0; w < NWV; ++w) {
      const float mw = sm.wm[w][hh];
      const float wt = mw == -__builtin_huge_valf() ? 0.f : exp2f(mw - M);
      sm.wgt[w][hh] = wt;
      L += sm.wl[w][hh] * wt;
    }
    sm.M[hh] = M;
    sm.L[hh] = L;
  }
  __syncthreads();
}

template <typename Lane, int D, int GQ, int NWV>
__device__ __forceinline__ void attn_merge_waves(Lane& st, AttnMergeSmem<GQ, D, NWV>& sm) {
  attn_waves_to_lds(st, sm);
  attn_merge_waves_rest(sm);
}

template <int D, int GQ, int NWV>
__device__ __forceinline__ float attn_wg_value(const AttnMergeSmem<GQ, D, NWV>& sm, int e) {
  const int hh = e / D;
  float v = 0.f;
#pragma unroll
  for (int w = 0; w < NWV; ++w) v += sm.ow[w][e] * sm.wgt[w][hh];
  return v;
}

// The workgroup holds the whole row: normalise and write.
template <int D, int GQ, int NWV, int NT>
__device__ __forceinline__ void attn_write_final(const AttnMergeSmem<GQ, D, NWV>& sm, const AttnOut& out) {
  for (int e = threadIdx.x; e < GQ * D; e += NT) out.put<D>(e / D, e % D, attn_wg_value<D, GQ, NWV>(sm, e) / sm.L[e / D]);
  if (static_cast<int>(threadIdx.x) < GQ) out.put_lse(threadIdx.x, sm.M[threadIdx.x], sm.L[threadIdx.x]);
}

// Partial layout per (row, part): [o (GQ*D) | m (GQ) | l (GQ)].
template <int D, int GQ>
__host__ __device__ constexpr int attn_part_stride() { return GQ * (D + 2); }

// Publish this workgroup's partial into part slot `part` of the row, count
// the arrival, and when it is the last of `parts` merge all of them into the
// output.  Every thread calls it.
template <int D, int GQ, int NWV, int NT>
__device__ __forceinline__ void attn_publish_and_merge(AttnMergeSmem<GQ, D, NWV>& sm, float* row_parts, int part,
                                                       int parts, uint32_t* counter, const AttnOut& out) {
  const int tid = threadIdx.x;
  constexpr int stride = attn_part_stride<D, GQ>();
  float* mine = row_parts + static_cast<int64_t>(part) * stride;
  for (int e = tid; e < GQ * D; e += NT) st_agent(mine + e, attn_wg_value<D, GQ, NWV>(sm, e));
  if (tid < GQ) {
    st_agent(mine + GQ * D + tid, sm.M[tid]);
    st_agent(mine + GQ * D + GQ + tid, sm.L[tid]);
  }
  if (!arrive_last(counter, static_cast<uint32_t>(parts), &sm.is_last)) return;

  // last workgroup: merge the parts (plain loads after the acquire); the output
  // values of all parts are loaded together with their maxima and sums
  const float* ps = row_parts;
  const int P = parts;
  constexpr int kOut = GQ * D / NT > 0 ? GQ * D / NT : 1;  // outputs per thread
  constexpr int kPR = 16;                                   // parts held in registers per pass
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
        const int e = tid + r * NT;
        ov[q][r] = (q < np && e < GQ * D) ? ps[(p0 + q) * stride + e] : 0.f;
      }
    for (int e = tid; e < np * GQ; e += NT) {
      const int p = p0 + e / GQ, hh = e % GQ;
      sm.pm[p * GQ + hh] = ps[p * stride + GQ * D + hh];
      sm.pl[p * GQ + hh] = ps[p * stride + GQ * D + GQ + hh];
    }
    __syncthreads();
    if (tid < GQ) {
      float M = p0 == 0 ? -__builtin_huge_valf() : sm.M[tid];
      for (int p = p0; p < p0 + np; ++p) M = fmaxf(M, sm.pm[p * GQ + tid]);
      sm.M[tid] = M;
    }
    __syncthreads();
    if (P <= kPR) {
#pragma unroll
      for (int r = 0; r < kOut; ++r) {
        const int e = tid + r * NT;
        if (e >= GQ * D) continue;
        const int hh = e / D;
        const float M = sm.M[hh];
        // unrolled to the register array's bound, so that ov stays in registers
        // (a loop to np would index it at run time and place it in scratch)
#pragma unroll
        for (int q = 0; q < kPR; ++q) {
          const float mp = q < np ? sm.pm[q * GQ + hh] : -__builtin_huge_valf();
          if (mp != -__builtin_huge_valf()) num[r] += exp2f(mp - M) * ov[q][r];
        }
      }
    }
  }
  if (P > kPR) {
    // second pass with the final maxima (more than kPR parts per row)
    for (int r = 0; r < kOut; ++r) {
      const int e = tid + r * NT;
      if (e >= GQ * D) continue;
      const int hh = e / D;
      const float M = sm.M[hh];
      float acc = 0.f;
      for (int p = 0; p < P; ++p) {
        const float mp = sm.pm[p * GQ + hh];
        if (mp != -__builtin_huge_valf()) acc += exp2f(mp - M) * ps[p * stride + e];
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
    const int e = tid + r * NT;
    if (e >= GQ * D) continue;
    const int hh = e / D;
    out.put<D>(hh, e % D, num[r] / sm.L[hh]);
    if (e % D == 0) out.put_lse(hh, sm.M[hh], sm.L[hh]);
  }
}

}  // namespace hga
