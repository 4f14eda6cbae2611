// Backward of the prefill attention on the matrix cores (bf16 Q, K, V; C = 64).
// [HGA technical summary (it), Meccanismo Core, item 4: the output is an exact
// softmax over the selected tokens; the routing is held fixed.]
//
// For one query row with z_u = q.k_u / sqrt(d) over its visible set,
// p = softmax(z) and D = sum_u p_u (do.v_u):
//   dq   = sum_u p_u (do.v_u - D) k_u / sqrt(d),
//   dk_u = sum_q p_u (do.v_u - D) q / sqrt(d),   dv_u = sum_q p_u do.
// Every contraction runs on v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
// Q, K and V are bf16 already; dO, P and dS are not, so each enters as two
// bf16 parts (hi = the rounded value, lo = the rounded remainder: 16
// significant bits), and a product of two split operands takes three MFMAs
// (hi.hi + hi.lo + lo.hi).
//
// Kernels, in launch order:
//   * bwd_split_do_kernel: dO -> dO_hi, dO_lo.
//   * bwd_vis_kernel: per (key chunk c, query chunk j), the 16-key blocks of c
//     that j's routed groups cover (4 bits; a bitmap zeroed before).
//   * bwd_count_kernel: the number of query chunks that see each key chunk (the
//     forced windows and the bitmap); the dK, dV rows of a key chunk whose
//     query chunks are split over several workgroups are zeroed.
//   * bwd_dq_mfma_kernel: one workgroup per routing unit (query chunk, b, kv
//     head), the forward's tile schedule (current chunk, other forced chunks,
//     routed groups) through a ring of three LDS tiles of K and V rows; each
//     wave owns 32 query rows of one head.  Pass 1 over the tiles:
//     S^T = K Q^T and dP^T = V dO^T, online max / sum / D per row.  Pass 2:
//     the same products, P = exp2(S - lse), dS = P (dP - D),
//     dq^T += K^T dS^T, the K^T fragments read from the K rows with
//     transposing LDS reads.  The rows' (lse, D) go to the workspace for the
//     key side.
//   * bwd_dkv_mfma_kernel: one workgroup per key chunk and piece of up to
//     kPiece of the query chunks that see it (in ascending order).  A step is
//     one such query chunk and one query head: its 64 rows of Q, dO_hi, dO_lo
//     and (lse, D), copied into one of two LDS slots while the other is used.
//     Wave (kh, qh) owns keys 32 kh.. of the chunk and query rows 32 qh.. of
//     every step: S = Q K^T and dP = dO V^T put P and dS in the layout of an
//     A operand over query rows; the B operands (Q, dO with the query rows
//     along k) are transposing LDS reads of the same rows; dV += P^T dO,
//     dK += dS^T Q.  K and V fragments and the dK, dV accumulators stay in
//     registers for the piece.  The two query halves meet in LDS at the end;
//     a key chunk with a single piece stores its rows, several pieces add
//     into zeroed rows with float atomics.
#include "hga_device.hpp"
#include "hga_kernels.hpp"
#include "hga_mfma.hpp"

#include <type_traits>

namespace hga {

namespace {

constexpr int kTile = 64;       // keys (and query rows) per tile = C
constexpr int kRing = 3;        // LDS tiles of the dq kernel
constexpr int kMaxTiles = 320;  // tiles of a unit
constexpr int kPiece = 32;      // query chunks per dK/dV workgroup
constexpr int kDkvWaves = 4;

// x = hi + lo with hi, lo bf16 (round to nearest each)
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = static_cast<__bf16>(x);
  lo = static_cast<__bf16>(x - static_cast<float>(hi));
}

// s_waitcnt vmcnt(N): all but this wave's N most recent vector memory
// operations have completed (GFX9 encoding, expcnt and lgkmcnt not waited).
template <int N>
__device__ __forceinline__ void wait_vmem_but() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// 16-key blocks of key chunk c that query chunk j sees: every block when c is
// one of j's forced chunks, else the routed bits of the bitmap.
__device__ __forceinline__ int visit_mask(const KParams& kp, const uint32_t* vis_row, int c, int j) {
  if (j < c) return 0;
  if (c < kp.n_sink || j - c <= kp.n_local) return 0xF;
  return vis_row ? static_cast<int>((vis_row[j >> 3] >> (4 * (j & 7))) & 0xFu) : 0;
}

}  // namespace

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_split_do_kernel(const float4* __restrict__ dO, uint2* __restrict__ hi,
                                                           uint2* __restrict__ lo, int64_t n4) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n4; i += static_cast<int64_t>(gridDim.x) * 256) {
    const float4 x = dO[i];
    const float xs[4] = {x.x, x.y, x.z, x.w};
    uint32_t h[2], l[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      __bf16 h0, l0, h1, l1;
      split_bf16(xs[2 * k], h0, l0);
      split_bf16(xs[2 * k + 1], h1, l1);
      h[k] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h0)) |
             (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h1)) << 16);
      l[k] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, l0)) |
             (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, l1)) << 16);
    }
    hi[i] = make_uint2(h[0], h[1]);
    lo[i] = make_uint2(l[0], l[1]);
  }
}

__global__ __launch_bounds__(256) void bwd_fill_zero_kernel(uint4* __restrict__ p, int64_t n16) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n16; i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// One wave per (query chunk j, b, kv head): the routed groups of j's
// (canonical) list set their blocks' bits in key chunk g / m's bitmap row.
__global__ __launch_bounds__(64) void bwd_vis_kernel(BackwardArgs a) {
  const KParams& kp = a.kp;
  const int j = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int32_t* gl = a.group_idx + (bh * a.n_units + j) * kp.top_g;
  const int bpg = kp.G / kBlk;  // blocks per group
  const int n_groups = static_cast<int>(kp.n_cap / kp.G);
  for (int e = threadIdx.x; e < kp.top_g; e += 64) {
    const int g = gl[e];
    if (g < 0 || g >= n_groups) continue;
    const int c = g / kp.m;
    const uint32_t blocks = ((1u << bpg) - 1u) << ((g % kp.m) * bpg);
    atomicOr(a.vis + (bh * a.n_units + c) * a.vis_words + (j >> 3), blocks << (4 * (j & 7)));
  }
}

// One wave per (key chunk c, b, kv head): how many query chunks see c; when
// more than one dK/dV workgroup will take them, zero the chunk's dK, dV rows.
template <int D>
__global__ __launch_bounds__(64) void bwd_count_kernel(BackwardArgs a) {
  const KParams& kp = a.kp;
  const int c = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int lane = threadIdx.x;
  const uint32_t* vrow = kp.top_g > 0 ? a.vis + (bh * a.n_units + c) * a.vis_words : nullptr;
  int total = 0;
  for (int j0 = c; j0 < a.n_units; j0 += 64) {
    const int j = j0 + lane;
    const int mk = j < a.n_units ? visit_mask(kp, vrow, c, j) : 0;
    total += __popcll(__ballot(mk != 0));
  }
  if (lane == 0) a.counts[bh * a.n_units + c] = total;
  if (total > kPiece) {
    float4* dk = reinterpret_cast<float4*>(a.dK + (bh * kp.n_cap + static_cast<int64_t>(c) * kTile) * D);
    float4* dv = reinterpret_cast<float4*>(a.dV + (bh * kp.n_cap + static_cast<int64_t>(c) * kTile) * D);
    for (int i = lane; i < kTile * D / 4; i += 64) {
      dk[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      dv[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
}

// ---------------------------------------------------------------------------
// dq kernel.  LDS: three ring slots, each a K tile and a V tile (bf16 rows
// padded by 16 bytes: conflict-free A-fragment reads) and a K^T tile (4
// transposed blocks).
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void bwd_dq_mfma_kernel(BackwardArgs a) {
  constexpr int NT = NW * 64;
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int CH = D / 8;          // 16-byte pieces per row
  constexpr int RB = D * 2;          // bytes per row
  constexpr int KP = CH + 1;
  constexpr int KRB = KP * 16;
  constexpr int KTB = kTile * KRB;
  const KParams& kp = a.kp;

  int x = blockIdx.x;
  const int h = x % kp.Hkv;
  x /= kp.Hkv;
  const int b = x % kp.B;
  x /= kp.B;
  const int u = a.n_units - 1 - x;  // later (heavier) query chunks first
  const int bh = b * kp.Hkv + h;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int ql = lane & 31;
  const int hb = lane >> 5;
  const int hh = wid / 2;
  const int pos0 = (wid & 1) * 32;
  const int qrow = u * kTile + pos0 + ql;
  const int64_t orow = (static_cast<int64_t>(b) * kp.Hq + static_cast<int64_t>(h) * kp.gq + hh) * a.n + qrow;

  __shared__ __align__(16) unsigned char k0[KTB], k1[KTB], k2[KTB];
  __shared__ __align__(16) unsigned char v0[KTB], v1[KTB], v2[KTB];
  __shared__ uint32_t tk[kMaxTiles][4];
  __shared__ int tvm[kMaxTiles];
  auto kslot = [&](auto S) -> unsigned char* {
    if constexpr (decltype(S)::value == 0) return k0;
    else if constexpr (decltype(S)::value == 1) return k1;
    else return k2;
  };
  auto vslot = [&](auto S) -> unsigned char* {
    if constexpr (decltype(S)::value == 0) return v0;
    else if constexpr (decltype(S)::value == 1) return v1;
    else return v2;
  };

  const int j = u;
  const int32_t* glg = kp.top_g > 0 ? a.group_idx + (static_cast<int64_t>(bh) * a.n_units + u) * kp.top_g : nullptr;
  const Forced fc = forced_chunks(j, kp.n_sink, kp.n_local);
  const int n_forced_other = fc.n - 1;
  const int bpg = kp.G / kBlk;
  const int gpt = kTile / kp.G;
  const int n_routed_tiles = (kp.top_g + gpt - 1) / gpt;
  const int n_tiles = 1 + n_forced_other + n_routed_tiles;
  const int n_groups_cap = static_cast<int>(kp.n_cap / kp.G);
  for (int q = tid; q < n_tiles * 4; q += NT) {
    const int tt = q >> 2, t = q & 3;
    int kb;
    if (tt == 0) {
      kb = j * 4 + t;
    } else if (tt <= n_forced_other) {
      kb = forced_chunk_at(fc, tt - 1) * 4 + t;
    } else {
      const int e = (tt - 1 - n_forced_other) * gpt + t / bpg;
      const int g = e < kp.top_g ? glg[e] : -1;
      kb = g >= 0 && g < n_groups_cap ? g * bpg + t % bpg : -1;
    }
    tk[tt][t] = kb >= 0 ? static_cast<uint32_t>(kb) * (kBlk * RB) : 0u;
    const uint64_t ok = __ballot(kb >= 0);
    if (t == 0) tvm[tt] = static_cast<int>((ok >> (lane & ~3)) & 0xf);
  }

  // the wave's query rows as B operands: Q, dO_hi, dO_lo
  bf16x8_t qv[KSTEPS], ohv[KSTEPS], olv[KSTEPS];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(static_cast<const bf16*>(a.Q) + orow * D);
    const uint4* hp = reinterpret_cast<const uint4*>(a.dOh + orow * D);
    const uint4* lp = reinterpret_cast<const uint4*>(a.dOl + orow * D);
#pragma unroll
    for (int d = 0; d < KSTEPS; ++d) {
      qv[d] = __builtin_bit_cast(bf16x8_t, qp[2 * d + hb]);
      ohv[d] = __builtin_bit_cast(bf16x8_t, hp[2 * d + hb]);
      olv[d] = __builtin_bit_cast(bf16x8_t, lp[2 * d + hb]);
    }
  }
  __syncthreads();

  const unsigned char* Kb = reinterpret_cast<const unsigned char*>(static_cast<const bf16*>(a.K) +
                                                                   static_cast<int64_t>(bh) * kp.n_cap * D);
  const unsigned char* Vb = reinterpret_cast<const unsigned char*>(static_cast<const bf16*>(a.V) +
                                                                   static_cast<int64_t>(bh) * kp.n_cap * D);
  // This lane's part of the copies: copy c fills bytes [1024 c, 1024 c + 1024)
  // of the padded K and V tiles; position p = 64 c + lane is piece p % KP of
  // row p / KP (the padding piece loads a duplicate).
  constexpr int NKC = (KP + NW - 1) / NW;
  uint32_t koff[NKC];
  int kblk[NKC];
#pragma unroll
  for (int i = 0; i < NKC; ++i) {
    const int p = 64 * (wid + i * NW) + lane;
    const int kr = (p / KP) & (kTile - 1), kpc = p % KP;
    koff[i] = static_cast<uint32_t>((kr & (kBlk - 1)) * RB + ((kpc < CH ? kpc : 0) << 4));
    kblk[i] = kr >> 4;
  }
  auto copy_tile = [&](auto S, int tt) __attribute__((always_inline)) {
    if (tt >= n_tiles) return;
    unsigned char* ks = kslot(S);
    unsigned char* vs = vslot(S);
#pragma unroll
    for (int i = 0; i < NKC; ++i) {
      const int c = wid + i * NW;
      if (c < KP) {
        const uint32_t o = tk[tt][kblk[i]] + koff[i];
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(Kb + o),
                                         (__attribute__((address_space(3))) void*)(ks + 1024 * c), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(Vb + o),
                                         (__attribute__((address_space(3))) void*)(vs + 1024 * c), 16, 0, 0);
      }
    }
  };

  // S^T (or dP^T) of sub-block sb: lane (ql, hb) gets query ql against keys
  // 32 sb + 8 (v / 4) + 4 hb + v % 4
  auto qk = [&](const unsigned char* ks, int sb) -> f32x16_t {
    f32x16_t acc = f32x16_t{};
    const unsigned char* rowp = ks + (32 * sb + ql) * KRB + hb * 16;
#pragma unroll
    for (int d = 0; d < KSTEPS; ++d)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t*>(rowp + 32 * d), qv[d], acc, 0, 0, 0);
    return acc;
  };
  auto dpk = [&](const unsigned char* vs, int sb) -> f32x16_t {
    f32x16_t acc = f32x16_t{};
    const unsigned char* rowp = vs + (32 * sb + ql) * KRB + hb * 16;
#pragma unroll
    for (int d = 0; d < KSTEPS; ++d) {
      const bf16x8_t va = *reinterpret_cast<const bf16x8_t*>(rowp + 32 * d);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, ohv[d], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, olv[d], acc, 0, 0, 0);
    }
    return acc;
  };
  // bit v: value v of sub-block sb of tile tt is visible (key
  // 32 sb + 8 (v / 4) + 4 hb + v % 4 of the tile; value v is in block
  // 2 sb + v / 8)
  auto visible_bits = [&](int tt, int sb) -> uint32_t {
    const int vm = (tvm[tt] >> (2 * sb)) & 3;
    uint32_t bits = (vm & 1 ? 0xffu : 0u) | (vm & 2 ? 0xff00u : 0u);
    if (tt == 0) {  // causal inside the current chunk
      const int q = pos0 + ql;
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (32 * sb + 8 * (v >> 2) + 4 * hb + (v & 3) > q) bits &= ~(1u << v);
    }
    return bits;
  };
  const float scale = kp.scale_log2;

  // ---- pass 1: per lane (its 16 keys of every sub-block) max, sum, sum p.dp
  float m_l = -__builtin_huge_valf(), l_l = 0.f, d_l = 0.f;
  // ---- pass 2 state
  float lse2 = 0.f, dv_row = 0.f;
  f32x16_t dq[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) dq[db] = f32x16_t{};

  auto sub = [&](auto PASS, const unsigned char* ks, const unsigned char* vs, int tt, int sb)
      __attribute__((always_inline)) {
    constexpr bool P2 = decltype(PASS)::value == 1;
    const f32x16_t s = qk(ks, sb);
    const f32x16_t dp = dpk(vs, sb);
    const uint32_t vb = visible_bits(tt, sb);
    auto visible = [&](int v) -> bool { return (vb >> v) & 1u; };
    if constexpr (!P2) {
      float mx = -__builtin_huge_valf();
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (visible(v)) mx = fmaxf(mx, s[v] * scale);
      if (mx > m_l) {
        const float al = __builtin_amdgcn_exp2f(m_l - mx);
        l_l *= al;
        d_l *= al;
        m_l = mx;
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float e = visible(v) ? __builtin_amdgcn_exp2f(fmaf(s[v], scale, -m_l)) : 0.f;
        l_l += e;
        d_l = fmaf(e, dp[v], d_l);
      }
    } else {
      bf16x8_t dsh[2], dsl[2];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = visible(v) ? __builtin_amdgcn_exp2f(fmaf(s[v], scale, -lse2)) : 0.f;
        __bf16 hi, lo;
        split_bf16(p * (dp[v] - dv_row), hi, lo);
        dsh[v >> 3][v & 7] = hi;
        dsl[v >> 3][v & 7] = lo;
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
          const bf16x8_t ka = lds_frag_tr(ks, KRB, 32 * sb + 16 * t, 32 * db, lane);
          dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, dsh[t], dq[db], 0, 0, 0);
          dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, dsl[t], dq[db], 0, 0, 0);
        }
    }
  };
  // Tile T in slot S: both sub-blocks, a barrier (every wave is past its reads
  // of tile T - 1's slot, and tile T + 1 has landed), then tile T + 2 starts
  // copying into tile T - 1's slot.
  auto run_pass = [&](auto PASS) __attribute__((always_inline)) {
    auto tile = [&](auto S, int T) __attribute__((always_inline)) {
      constexpr int s0 = decltype(S)::value, s2 = (s0 + 2) % kRing;
      sub(PASS, kslot(S), vslot(S), T, 0);
      sub(PASS, kslot(S), vslot(S), T, 1);
      __syncthreads();
      copy_tile(std::integral_constant<int, s2>{}, T + 2);
    };
    copy_tile(std::integral_constant<int, 0>{}, 0);
    __syncthreads();
    copy_tile(std::integral_constant<int, 1>{}, 1);
    for (int T = 0; T < n_tiles; T += kRing) {
      tile(std::integral_constant<int, 0>{}, T);
      if (T + 1 < n_tiles) tile(std::integral_constant<int, 1>{}, T + 1);
      if (T + 2 < n_tiles) tile(std::integral_constant<int, 2>{}, T + 2);
    }
  };
  static_assert(kRing == 3, "the tile loop names three slots");

  run_pass(std::integral_constant<int, 0>{});
  {
    // the two lane halves hold different keys of the same query row
    float mo, lo, dlo, t0v, t1v;
    dpp::swap32(m_l, t0v, t1v);
    mo = hb ? t0v : t1v;
    dpp::swap32(l_l, t0v, t1v);
    lo = hb ? t0v : t1v;
    dpp::swap32(d_l, t0v, t1v);
    dlo = hb ? t0v : t1v;
    const float m = fmaxf(m_l, mo);
    const float a0 = __builtin_amdgcn_exp2f(m_l - m), a1 = __builtin_amdgcn_exp2f(mo - m);
    const float l = l_l * a0 + lo * a1;
    lse2 = m + __builtin_log2f(l);
    dv_row = (d_l * a0 + dlo * a1) / l;
    if (hb == 0) {
      a.stats[2 * orow] = lse2;
      a.stats[2 * orow + 1] = dv_row;
    }
  }
  run_pass(std::integral_constant<int, 1>{});

  // ---- dQ = dq^T / sqrt(d): lane (query, half) holds dims 32db + 8i + 4 half + {0..3}
#pragma unroll
  for (int db = 0; db < DBLK; ++db) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = 32 * db + 8 * i + 4 * hb;
      const float sc = kp.inv_sqrt_d;
      *reinterpret_cast<float4*>(a.dQ + orow * D + d0) =
          make_float4(dq[db][4 * i] * sc, dq[db][4 * i + 1] * sc, dq[db][4 * i + 2] * sc, dq[db][4 * i + 3] * sc);
    }
  }
}

// ---------------------------------------------------------------------------
// dK/dV kernel.  LDS: a ring of three step slots (32 rows of Q, dO_hi, dO_lo
// padded by 16 bytes, then their (lse, D)), the piece's visit list; about
// 79 KB, so two workgroups share a CU.
constexpr int kDkvRows = 32;  // query rows per step

template <int D>
struct DkvSlot {
  static constexpr int KRB = (D / 8 + 1) * 16;
  unsigned char q[kDkvRows * KRB];
  unsigned char oh[kDkvRows * KRB];
  unsigned char ol[kDkvRows * KRB];
  float st[kDkvRows * 2];
};

template <int D>
__global__ __launch_bounds__(kDkvWaves * 64) void bwd_dkv_mfma_kernel(BackwardArgs a) {
  constexpr int KS = D / 32;                     // k-steps of 32 dimensions
  constexpr int DT = D / 16;                     // 16-dimension output tiles
  constexpr int CH = D / 8;
  constexpr int RB = D * 2;
  constexpr int KP = CH + 1;
  constexpr int KRB = KP * 16;
  constexpr int CPM = (kDkvRows * KP + 63) / 64;  // 1 KB copies per matrix (the last one partly)
  constexpr int NC = 3 * CPM + 1;                 // and one of 256 bytes of statistics
  constexpr int NCW = NC / kDkvWaves;             // copies per wave per step
  static_assert(NC % kDkvWaves == 0, "every wave issues the same number of step copies");
  const KParams& kp = a.kp;

  // ---- key chunk.  Workgroups are dealt to the dies in turn, so die x % 8
  // takes every 8th chunk: the early chunks, which far more query chunks see
  // (a chunk is a routing candidate for every later one), spread over all dies.
  const int n_units = a.n_units;
  const int c = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int piece = blockIdx.z;
  const int b = static_cast<int>(bh / kp.Hkv), h = static_cast<int>(bh % kp.Hkv);
  const int total = a.counts[bh * n_units + c];
  if (piece * kPiece >= total) return;
  const bool shared_rows = total > kPiece;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int blk = tid >> 6;  // wave w owns 16-key block w of the chunk
  const int l16 = lane & 15, g = lane >> 4;

  __shared__ __align__(16) DkvSlot<D> s0, s1, s2;
  __shared__ int vis_j[kPiece], vis_m[kPiece];
  __shared__ int n_vis_sh;
  auto slot = [&](auto S) -> DkvSlot<D>& {
    if constexpr (decltype(S)::value == 0) return s0;
    else if constexpr (decltype(S)::value == 1) return s1;
    else return s2;
  };

  // ---- the piece's query chunks
  if (blk == 0) {
    const uint32_t* vrow = kp.top_g > 0 ? a.vis + (bh * n_units + c) * a.vis_words : nullptr;
    const int first = piece * kPiece;
    int seen = 0;
    for (int j0 = c; j0 < n_units && seen < first + kPiece; j0 += 64) {
      const int j = j0 + lane;
      const int mk = j < n_units ? visit_mask(kp, vrow, c, j) : 0;
      const uint64_t bal = __ballot(mk != 0);
      const int r = seen + static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal >> 32),
                                                                       __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0u)));
      if (mk != 0 && r >= first && r < first + kPiece) {
        vis_j[r - first] = j;
        vis_m[r - first] = mk;
      }
      seen += __popcll(bal);
    }
    if (lane == 0) n_vis_sh = min(max(seen - first, 0), kPiece);
  }

  // ---- the block's keys as B operands (k = dimension): K and V fragments
  const int64_t krow = bh * kp.n_cap + static_cast<int64_t>(c) * kTile + 16 * blk + l16;
  bf16x8_t kf[KS], vf[KS];
  {
    const uint4* kp4 = reinterpret_cast<const uint4*>(static_cast<const bf16*>(a.K) + krow * D);
    const uint4* vp4 = reinterpret_cast<const uint4*>(static_cast<const bf16*>(a.V) + krow * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = __builtin_bit_cast(bf16x8_t, kp4[4 * ks + g]);
      vf[ks] = __builtin_bit_cast(bf16x8_t, vp4[4 * ks + g]);
    }
  }
  f32x4_t dk[DT], dv[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) dk[t] = dv[t] = f32x4_t{};

  // ---- this lane's part of the step copies: copy cc = wave + 4 i is 1 KB
  // cm = cc % CPM of matrix cc / CPM (0 Q, 1 dO_hi, 2 dO_lo): lane position
  // p = 64 cm + lane (< 32 KP) = piece p % KP of row p / KP; copy 3 CPM: the
  // statistics, 16 bytes per lane (< 16)
  uint32_t coff[NCW];
  bool con[NCW];
#pragma unroll
  for (int i = 0; i < NCW; ++i) {
    const int cc = blk + kDkvWaves * i;
    const int p = 64 * (cc % CPM) + lane;
    const int r = p / KP, pc = p % KP;
    const bool row_copy = cc < 3 * CPM;
    coff[i] = row_copy ? static_cast<uint32_t>(r * RB + ((pc < CH ? pc : 0) << 4)) : static_cast<uint32_t>(16 * lane);
    con[i] = row_copy ? p < kDkvRows * KP : lane < kDkvRows * 8 / 16;
  }
  __syncthreads();
  const int steps_per_visit = kp.gq * (kTile / kDkvRows);
  const int n_steps = n_vis_sh * steps_per_visit;

  // step st: visit st / steps_per_visit, head (st / 2) % gq, rows 32 (st % 2)..
  auto copy_step = [&](auto S, int st) __attribute__((always_inline)) {
    if (st >= n_steps) return;
    DkvSlot<D>& sl = slot(S);
    const int vi = st / steps_per_visit;
    const int rem = st - vi * steps_per_visit;
    const int hh = rem >> 1, half = rem & 1;
    const int64_t row0 = (static_cast<int64_t>(b) * kp.Hq + static_cast<int64_t>(h) * kp.gq + hh) * a.n +
                         static_cast<int64_t>(vis_j[vi]) * kTile + kDkvRows * half;
    const unsigned char* srcq = reinterpret_cast<const unsigned char*>(static_cast<const bf16*>(a.Q) + row0 * D);
    const unsigned char* srch = reinterpret_cast<const unsigned char*>(a.dOh + row0 * D);
    const unsigned char* srcl = reinterpret_cast<const unsigned char*>(a.dOl + row0 * D);
    const unsigned char* srcs = reinterpret_cast<const unsigned char*>(a.stats + row0 * 2);
#pragma unroll
    for (int i = 0; i < NCW; ++i) {
      const int cc = blk + kDkvWaves * i;
      const unsigned char* src;
      unsigned char* dst;
      if (cc < CPM) {
        src = srcq;
        dst = sl.q + 1024 * cc;
      } else if (cc < 2 * CPM) {
        src = srch;
        dst = sl.oh + 1024 * (cc - CPM);
      } else if (cc < 3 * CPM) {
        src = srcl;
        dst = sl.ol + 1024 * (cc - 2 * CPM);
      } else {
        src = srcs;
        dst = reinterpret_cast<unsigned char*>(sl.st);
      }
      if (con[i])
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + coff[i]),
                                         (__attribute__((address_space(3))) void*)(dst), 16, 0, 0);
    }
  };

  const float scale = kp.scale_log2;
  const int kl = 16 * blk + l16;  // this lane's key within the chunk
  auto compute_step = [&](auto S, int st) __attribute__((always_inline)) {
    const DkvSlot<D>& sl = slot(S);
    const int vi = st / steps_per_visit;
    const int q0 = kDkvRows * (st & 1);  // first query row of the step within the chunk
    const bool diag = vis_j[vi] == c;
    // the block unseen, or (current chunk) entirely after the step's queries
    if (!((vis_m[vi] >> blk) & 1) || (diag && 16 * blk > q0 + kDkvRows - 1)) return;
    // S = Q K^T, dP = dO V^T on two 16-query tiles: lane (key l16, group g)
    // gets the step's query rows 16 qt + 4 g + i
    f32x4_t sc[2], pa[2], pb[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      sc[qt] = pa[qt] = pb[qt] = f32x4_t{};
      const int rb = (16 * qt + l16) * KRB + 16 * g;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        sc[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8_t*>(sl.q + rb + 64 * ks), kf[ks],
                                                         sc[qt], 0, 0, 0);
        pa[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8_t*>(sl.oh + rb + 64 * ks), vf[ks],
                                                         pa[qt], 0, 0, 0);
        pb[qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8_t*>(sl.ol + rb + 64 * ks), vf[ks],
                                                         pb[qt], 0, 0, 0);
      }
    }
    // P and dS as A operands over the step's 32 query rows (slot 4 qt + i)
    bf16x8_t ph, pl, dsh, dsl;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int r0 = 16 * qt + 4 * g;
      const float4 st01 = *reinterpret_cast<const float4*>(sl.st + 2 * r0);
      const float4 st23 = *reinterpret_cast<const float4*>(sl.st + 2 * r0 + 4);
      const float lse[4] = {st01.x, st01.z, st23.x, st23.z};
      const float dr[4] = {st01.y, st01.w, st23.y, st23.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = !diag || kl <= q0 + r0 + i;
        const float p = ok ? __builtin_amdgcn_exp2f(fmaf(sc[qt][i], scale, -lse[i])) : 0.f;
        __bf16 hi, lo;
        split_bf16(p, hi, lo);
        ph[4 * qt + i] = hi;
        pl[4 * qt + i] = lo;
        split_bf16(p * (pa[qt][i] + pb[qt][i] - dr[i]), hi, lo);
        dsh[4 * qt + i] = hi;
        dsl[4 * qt + i] = lo;
      }
    }
    // per 16-dimension tile: Q, dO_hi, dO_lo with the query rows along k
    // (transposing LDS reads); dV += P^T dO, dK += dS^T Q
#pragma unroll
    for (int t = 0; t < DT; ++t) {
      const bf16x8_t bq = lds_frag_tr16(sl.q, KRB, 0, 16 * t, lane);
      const bf16x8_t bh_ = lds_frag_tr16(sl.oh, KRB, 0, 16 * t, lane);
      const bf16x8_t bl = lds_frag_tr16(sl.ol, KRB, 0, 16 * t, lane);
      dv[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, bh_, dv[t], 0, 0, 0);
      dv[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, bl, dv[t], 0, 0, 0);
      dv[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, bh_, dv[t], 0, 0, 0);
      dk[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dsh, bq, dk[t], 0, 0, 0);
      dk[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dsl, bq, dk[t], 0, 0, 0);
    }
  };

  // ---- steps through a ring of three slots: step s computes while the copies
  // of steps s + 1 and s + 2 are in flight.  The barrier after step s waits
  // (per wave) for every copy but its newest NCW loads, i.e. for step s + 1's,
  // then LDS-only fences order the slot reads and the next copy into the slot
  // just read.
  auto step_barrier = [&](bool newest_in_flight) __attribute__((always_inline)) {
    if (newest_in_flight) wait_vmem_but<NCW>();
    else wait_vmem_but<0>();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };
  auto one = [&](auto S, int st) __attribute__((always_inline)) {
    constexpr int s2 = (decltype(S)::value + 2) % 3;
    copy_step(std::integral_constant<int, s2>{}, st + 2);
    compute_step(S, st);
    step_barrier(st + 2 < n_steps);
  };
  copy_step(std::integral_constant<int, 0>{}, 0);
  copy_step(std::integral_constant<int, 1>{}, 1);
  step_barrier(1 < n_steps);
  for (int st = 0; st < n_steps; st += 3) {
    one(std::integral_constant<int, 0>{}, st);
    if (st + 1 < n_steps) one(std::integral_constant<int, 1>{}, st + 1);
    if (st + 2 < n_steps) one(std::integral_constant<int, 2>{}, st + 2);
  }

  // ---- the block's rows of dK (scaled by 1/sqrt(d)) and dV: lane (l16, g)
  // holds dimension 16 t + l16 of keys 4 g + i
  const int64_t key0 = bh * kp.n_cap + static_cast<int64_t>(c) * kTile + 16 * blk + 4 * g;
#pragma unroll
  for (int t = 0; t < DT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float* pk = a.dK + (key0 + i) * D + 16 * t + l16;
      float* pv = a.dV + (key0 + i) * D + 16 * t + l16;
      const float vk = dk[t][i] * kp.inv_sqrt_d, vv = dv[t][i];
      if (shared_rows) {
        __hip_atomic_fetch_add(pk, vk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(pv, vv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        *pk = vk;
        *pv = vv;
      }
    }
}

// ---------------------------------------------------------------------------
bool backward_mfma_supported(const KParams& kp, bool bf16_in) {
  if (!(bf16_in && kp.C == kTile && (kp.d == 64 || kp.d == 128) && (kp.gq == 1 || kp.gq == 2 || kp.gq == 4) &&
        kp.G % kBlk == 0 && kTile % kp.G == 0))
    return false;
  const int64_t tiles = 1 + static_cast<int64_t>(kp.n_sink) + kp.n_local +
                        (static_cast<int64_t>(kp.top_g) * kp.G + kTile - 1) / kTile;
  return tiles <= kMaxTiles && kp.n_cap * kp.d * 2 <= 0xffffffffll;
}

int backward_vis_words(int n_units) { return (n_units + 7) / 8; }
int backward_max_pieces(int n_units) { return (n_units + kPiece - 1) / kPiece; }

template <int D, int NW>
static hipError_t launch_mfma_t(const BackwardArgs& a, hipStream_t st) {
  const KParams& kp = a.kp;
  const int64_t bhkv = static_cast<int64_t>(kp.B) * kp.Hkv;
  const int64_t n4 = static_cast<int64_t>(kp.B) * kp.Hq * a.n * D / 4;
  bwd_split_do_kernel<<<2048, 256, 0, st>>>(reinterpret_cast<const float4*>(a.dO), reinterpret_cast<uint2*>(a.dOh),
                                            reinterpret_cast<uint2*>(a.dOl), n4);
  if (kp.top_g > 0) {
    const int64_t words = bhkv * a.n_units * a.vis_words;
    bwd_fill_zero_kernel<<<256, 256, 0, st>>>(reinterpret_cast<uint4*>(a.vis), (words + 3) / 4);
    bwd_vis_kernel<<<dim3(a.n_units, static_cast<unsigned>(bhkv)), 64, 0, st>>>(a);
  }
  bwd_count_kernel<D><<<dim3(a.n_units, static_cast<unsigned>(bhkv)), 64, 0, st>>>(a);
  bwd_dq_mfma_kernel<D, NW><<<static_cast<unsigned>(bhkv * a.n_units), NW * 64, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  bwd_dkv_mfma_kernel<D><<<dim3(a.n_units, static_cast<unsigned>(bhkv), backward_max_pieces(a.n_units)),
                           kDkvWaves * 64, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_backward_mfma(const BackwardArgs& a, hipStream_t st) {
  const int nw = 2 * a.kp.gq;
  if (a.kp.d == 128) {
    if (nw == 2) return launch_mfma_t<128, 2>(a, st);
    if (nw == 4) return launch_mfma_t<128, 4>(a, st);
    if (nw == 8) return launch_mfma_t<128, 8>(a, st);
  } else {
    if (nw == 2) return launch_mfma_t<64, 2>(a, st);
    if (nw == 4) return launch_mfma_t<64, 4>(a, st);
    if (nw == 8) return launch_mfma_t<64, 8>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace hga
