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
// lo = bf16(s - hi); the lo and then the hi products accumulate in one fp32
// chain (relative error of the split about 2^-17).  The split is done once
// per call by a pre-pass over both tables (every unit of a KV head reads the
// same rows); the units copy their tiles of hi and lo rows from memory
// straight into LDS.  Top-k on the chunk scores, then the same contraction
// over the C/G groups of every routed chunk and a top-g.  Where the shape
// allows (at most 1024 candidate chunks and routed groups, k <= 64) the score
// and selection arrays are sized for it, so three 512-thread workgroups
// share a CU.
#include "hga_device.hpp"
#include "hga_kernels.hpp"
#include "hga_select.hpp"

#include <algorithm>

namespace hga {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRTile = 32;  // summaries per tile

// Selection scratch: the compact variant's k <= 64; the general one also holds
// the radix path's scratch for a k too large for the ballot search.
template <int NT, bool SMALL>
union RouteSelSmem;
template <int NT>
union RouteSelSmem<NT, true> {
  SelSmem<NT, 64> sel;
};
template <int NT>
union RouteSelSmem<NT, false> {
  SelSmem<NT> sel;
  TopkSmem<NT> topk;
};

template <int D, int NW, bool SMALL>
struct RoutePrefillSmem {
  static constexpr int ROW = D * 2 + 16;       // bytes per bf16 row (padded by one 16-byte piece)
  static constexpr int PART = kRTile * ROW;    // one table's rows of a tile
  static constexpr int MAXN = SMALL ? 1024 : 4096;  // candidate chunks, and routed chunks x C/G
  static constexpr int MAXK = SMALL ? 64 : 1024;
  alignas(16) unsigned char tile[2][2 * PART];  // per buffer: hi rows, then lo rows
  float wmax[2][NW][kRTile];  // per tile parity: each wave's column maxima
  float scores[MAXN];         // chunk scores of the unit, then group scores
  int sel_chunks[MAXK];
  int sel_groups[MAXK];
  RouteSelSmem<NW * 64, SMALL> u;
};

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

// Split tables: rows [0, R) of an fp32 table into hi and lo bf16 rows, 8
// values per thread.  Layout of the split area: chunk hi, chunk lo, group hi,
// group lo, each [B*Hkv*rows, d].
template <int D>
__global__ __launch_bounds__(256) void summary_split_kernel(const float* __restrict__ src, int64_t rows,
                                                            uint16_t* __restrict__ hi, uint16_t* __restrict__ lo) {
  const int64_t e = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (e >= rows * D) return;
  const float4 a = *reinterpret_cast<const float4*>(src + e);
  const float4 b = *reinterpret_cast<const float4*>(src + e + 4);
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float h0 = bf16_to_f32(f32_to_bf16(v[2 * i])), h1 = bf16_to_f32(f32_to_bf16(v[2 * i + 1]));
    h[i] = pack_bf16x2(h0, h1);
    l[i] = pack_bf16x2(v[2 * i] - h0, v[2 * i + 1] - h1);
  }
  *reinterpret_cast<uint4*>(hi + e) = make_uint4(h[0], h[1], h[2], h[3]);
  *reinterpret_cast<uint4*>(lo + e) = make_uint4(l[0], l[1], l[2], l[3]);
}

size_t route_prefill_split_bytes(const KParams& kp) {
  const size_t rows = static_cast<size_t>(kp.B) * kp.Hkv * kp.n_chunks_cap * (1 + kp.m);
  return rows * kp.d * 2 * sizeof(uint16_t);
}

// Waves per SIMD the compact variant is compiled for: three workgroups of
// eight waves per CU need at most 80 VGPRs per lane.
template <int NW, bool SMALL>
constexpr int route_waves_per_eu() { return SMALL && NW == 8 ? 6 : 1; }

template <int D, int NW, bool SMALL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(route_waves_per_eu<NW, SMALL>(), 8)))
void route_prefill_mfma_kernel(RouteArgs a) {
  constexpr int NT = NW * 64;
  constexpr int KSTEPS = D / 16;
  constexpr int P8 = D / 8;                     // 16-byte pieces per bf16 row
  using Smem = RoutePrefillSmem<D, NW, SMALL>;
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

  // scores of n rows (row(i): index of the summary row in the split tables
  // hi, lo) into out[0..n).  Tiles are loaded two ahead (register sets A and B
  // alternate, the loop is unrolled by two so each set is named statically)
  // and copied into the LDS buffer of their parity.
  // scores of n rows (row(i): index of the summary row in the split tables
  // hi, lo) into out[0..n).  A tile's hi and lo rows go from memory straight
  // into the LDS buffer of its parity (17 copies of 1 KB per tile: each row
  // is 16 pieces of 16 bytes plus a padding piece, which loads a duplicate),
  // one tile ahead; one barrier per tile.
  constexpr int PIECES = 2 * kRTile * (P8 + 1);        // pieces of a tile, padding included
  constexpr int NCOPY = (PIECES + 63) / 64;            // 1 KB copies per tile
  constexpr int CPW = (NCOPY + NW - 1) / NW;           // copies per wave
  static_assert(PIECES % 64 == 0, "whole copies");
  int c_part[CPW], c_row[CPW], c_off[CPW];
#pragma unroll
  for (int k = 0; k < CPW; ++k) {
    const int q = 64 * (wid + NW * k) + lane;
    const int part = q / (kRTile * (P8 + 1)), rq = q % (kRTile * (P8 + 1));
    const int pc = rq % (P8 + 1);
    c_part[k] = part;
    c_row[k] = rq / (P8 + 1);
    c_off[k] = (pc < P8 ? pc : 0) * 8;  // elements; the padding piece repeats piece 0
  }
  auto score_tiles = [&](int n, auto row, const uint16_t* hi, const uint16_t* lo, float* out) {
    const int n_tiles = (n + kRTile - 1) / kRTile;
    auto copy = [&](int tt, int buf) {
#pragma unroll
      for (int k = 0; k < CPW; ++k) {
        if (wid + NW * k < NCOPY) {
          const int idx = min(tt * kRTile + c_row[k], n - 1);  // rows past n: any valid row
          const uint16_t* src = (c_part[k] ? lo : hi) + row(idx) * D + c_off[k];
          __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src),
                                           (__attribute__((address_space(3))) void*)(&sm.tile[buf][1024 * (wid + NW * k)]),
                                           16, 0, 0);
        }
      }
    };
    auto compute = [&](int buf) {
      f32x16_t acc = f32x16_t{};
      const unsigned char* th = sm.tile[buf];
      const unsigned char* tl = sm.tile[buf] + Smem::PART;
#pragma unroll
      for (int d = 0; d < KSTEPS; ++d) {
        const int off = ql * Smem::ROW + (16 * d + 8 * hb) * 2;
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[d], *reinterpret_cast<const bf16x8_t*>(tl + off), acc, 0, 0, 0);
      }
#pragma unroll
      for (int d = 0; d < KSTEPS; ++d) {
        const int off = ql * Smem::ROW + (16 * d + 8 * hb) * 2;
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[d], *reinterpret_cast<const bf16x8_t*>(th + off), acc, 0, 0, 0);
      }
      float mx = acc[0];
#pragma unroll
      for (int v = 1; v < 16; ++v) mx = fmaxf(mx, acc[v]);
      {
        float pa, pb;
        dpp::swap32(mx, pa, pb);
        mx = fmaxf(pa, pb);
      }
      if (hb == 0) sm.wmax[buf][wid][ql] = mx;
    };
    auto reduce = [&](int tt) {
      if (tid < kRTile) {
        const int idx = tt * kRTile + tid;
        float m = sm.wmax[tt & 1][0][tid];
#pragma unroll
        for (int w = 1; w < NW; ++w) m = fmaxf(m, sm.wmax[tt & 1][w][tid]);
        if (idx < n) out[idx] = m * kp.inv_sqrt_d;
      }
    };
    if (n_tiles == 0) return;
    // tile tt computes from buffer tt % 2 while tile tt + 1 lands in the
    // other; that buffer was last read by tile tt - 1, before the previous
    // barrier.  Each wave waits for its own copies, then the barrier publishes
    // the tile to all waves.
    copy(0, 0);
    wait_vmem();
    __syncthreads();
    for (int tt = 0; tt < n_tiles; ++tt) {
      if (tt + 1 < n_tiles) copy(tt + 1, (tt + 1) & 1);
      compute(tt & 1);
      wait_vmem();
      __syncthreads();
      reduce(tt);
    }
    __syncthreads();  // the last scores are in out
  };

  // ---- level 1: chunk scores and top-k
  const int64_t crow0 = static_cast<int64_t>(bh) * kp.n_chunks_cap + kp.n_sink;
  const int64_t n_ctab = static_cast<int64_t>(kp.B) * kp.Hkv * kp.n_chunks_cap * D;
  const uint16_t* c_hi = a.split;
  const uint16_t* c_lo = a.split + n_ctab;
  const uint16_t* g_hi = a.split + 2 * n_ctab;
  const uint16_t* g_lo = a.split + 2 * n_ctab + n_ctab * kp.m;
  score_tiles(nM, [&](int i) { return crow0 + i; }, c_hi, c_lo, sm.scores);
  // exact top-k of sm.scores[0, n) into out (ascending positions): ballot
  // search by whole waves, or the radix path for a k too large for it
  auto select = [&](int n, int k, int* out) -> int {
    if constexpr (SMALL) {
      return block_select<NT, 4, 64>([&](int i) { return sm.scores[i]; }, n, k, out, sm.u.sel);
    } else {
      if (block_select_fits<NT>(n, k))
        return block_select<NT>([&](int i) { return sm.scores[i]; }, n, k, out, sm.u.sel);
      return block_topk<NT>([&](int i) { return sm.scores[i]; }, n, k, out, sm.u.topk);
    }
  };
  const int cnt = select(nM, kp.top_k, sm.sel_chunks);
  int32_t* ci = a.chunk_idx + unit * kp.top_k;
  for (int i = tid; i < kp.top_k; i += NT) ci[i] = i < cnt ? kp.n_sink + sm.sel_chunks[i] : -1;

  // ---- level 2: group scores of the routed chunks and top-g
  const int m = kp.m;
  const int nG = cnt * m;
  const int64_t grow0 = static_cast<int64_t>(bh) * kp.n_chunks_cap * m;
  score_tiles(nG,
              [&](int i) { return grow0 + static_cast<int64_t>(kp.n_sink + sm.sel_chunks[i / m]) * m + i % m; },
              g_hi, g_lo, sm.scores);
  const int gcnt = select(nG, kp.top_g, sm.sel_groups);
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
         static_cast<int64_t>(kp.top_k) * kp.m <= 4096 && kp.top_k <= 1024 && kp.top_g <= 1024;
}

// The compact variant holds every unit of this shape: at most 1024 candidate
// chunks and 1024 routed groups, k <= 64, and both selections within four
// keys per lane (block_select_fits is monotone in n, so the largest unit
// decides).
template <int NW>
static bool route_small_fits(const KParams& kp) {
  constexpr int NT = NW * 64;
  const int max_cand = std::max(0, kp.n_chunks_cap - 1 - kp.n_local - kp.n_sink);
  const int max_groups = kp.top_k * kp.m;
  return max_cand <= 1024 && max_groups <= 1024 && kp.top_k <= 64 && kp.top_g <= 64 &&
         block_select_fits<NT, 4, 64>(max_cand, kp.top_k) && block_select_fits<NT, 4, 64>(max_groups, kp.top_g);
}

template <int D, int NW>
static hipError_t launch_t(const RouteArgs& a, hipStream_t st) {
  const KParams& kp = a.kp;
  const int64_t crows = static_cast<int64_t>(kp.B) * kp.Hkv * kp.n_chunks_cap;
  const int64_t n_ctab = crows * D;
  auto split = [&](const float* src, int64_t rows, uint16_t* hi, uint16_t* lo) {
    const int64_t threads = rows * D / 8;
    summary_split_kernel<D><<<static_cast<unsigned>((threads + 255) / 256), 256, 0, st>>>(src, rows, hi, lo);
  };
  split(a.chunk_sum, crows, a.split, a.split + n_ctab);
  split(a.group_sum, crows * kp.m, a.split + 2 * n_ctab, a.split + 2 * n_ctab + n_ctab * kp.m);
  const unsigned n_wg = static_cast<unsigned>(kp.B) * kp.Hkv * a.n_units;
  if (route_small_fits<NW>(kp))
    route_prefill_mfma_kernel<D, NW, true><<<n_wg, NW * 64, 0, st>>>(a);
  else
    route_prefill_mfma_kernel<D, NW, false><<<n_wg, NW * 64, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_route_prefill_mfma(const RouteArgs& a, hipStream_t st) {
  if (!a.split) return hipErrorInvalidValue;
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
