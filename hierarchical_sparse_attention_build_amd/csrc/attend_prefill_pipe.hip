// Steps 4-5 of HGA for prefill on the matrix cores, software-pipelined:
// visibility union + exact softmax attention of one routing unit (a query
// chunk of C = 64 positions and all query heads of a KV head) over its
// gathered K/V tiles.
// [HGA technical summary (it), Meccanismo Core, item 2 third bullet and item 4].
//
// V goes through a pre-pass first: each 16-key block of V (bf16 rows) becomes
// one block of D x 16 fp16 values, the 16 keys of a dimension side by side in
// the order the P.V step reads them (keys 0-3, 8-11 | 4-7, 12-15) and the two
// 16-byte halves of a dimension swapped on every other 8 dimensions (no LDS
// bank conflict on the reads).  A routed group of G = 16k keys is k blocks;
// a chunk is 4 blocks.  The conversion is done once per call instead of once
// per unit that routes to the block.
//
// One workgroup per unit; each wave owns 32 query rows (one head, 32
// positions).  Keys come in tiles of 64 (the current chunk (causal), the other
// forced chunks, then the routed groups), copied from HBM straight into a
// ring of three LDS tiles two tiles ahead, one barrier per tile.  K
// rows keep their bf16 layout, padded by 16 bytes (a row starts one bank
// group after the previous one), so the A-fragment reads are free of bank
// conflicts and every k-step's offset is an immediate.
//
// Per wave the work is pipelined over 32-key sub-blocks b:
//   the max of S(b) (launched during b - 1) decides whether the reference
//   max m rises (when it exceeds m by more than 2^8, base 2); a rise rescales
//   O, l and the pending P(b-1);
//   O^T   += V^T P^T(b-1) (fp16 MFMA, V fragments read during b-1) \  matrix
//   S(b+1) = K Q^T     (bf16 MFMA, 32x32x16)                        /  cores
//   P(b)   = exp2(S(b) scale - m) (vector ALUs, concurrently), and the V
//            fragments of b are read for the next step.  P is rounded to fp16 toward zero (relative error < 2^-10; the row
// sum adds the same rounded values), V to fp16 exactly for |v| < 65504.
#include "hga_device.hpp"
#include "hga_kernels.hpp"
#include "hga_mfma.hpp"

#include <type_traits>

namespace hga {

namespace {

constexpr int kTile = 64;      // keys per tile (= C)
constexpr int kRing = 3;       // LDS tiles
constexpr int kMaxTiles = 320;  // tiles of a unit: the forced chunks and the routed groups

}  // namespace

// ---------------------------------------------------------------------------
// V pre-pass: blocks [0, ceil(limit / 16)) of every (b, KV head), limit = the
// last key any query of the call sees + 1.  One workgroup converts 64 keys.
template <int D>
__global__ __launch_bounds__(256) void v16_blocks_kernel(const bf16* __restrict__ V, uint16_t* __restrict__ V16,
                                                         KParams kp, const int32_t* q_pos, int32_t pos_bias,
                                                         int64_t nq) {
  constexpr int RB = D * 2;  // bytes per V row
  __shared__ __align__(16) unsigned char rows[kTile * RB];
  const int bh = blockIdx.y;
  const int b = bh / kp.Hkv;
  const int64_t t0 = (q_pos ? q_pos[b] : 0) + static_cast<int64_t>(pos_bias);
  const int64_t lim0 = t0 + nq > 0 ? t0 + nq : 0;
  const int64_t limit = lim0 < kp.n_cap ? lim0 : kp.n_cap;
  const int64_t key0 = static_cast<int64_t>(blockIdx.x) * kTile;
  if (key0 >= limit) return;
  const int tid = threadIdx.x;
  const unsigned char* src = reinterpret_cast<const unsigned char*>(V + (static_cast<int64_t>(bh) * kp.n_cap + key0) * D);
  for (int q = tid; q < kTile * RB / 16; q += 256)
    *reinterpret_cast<uint4*>(rows + q * 16) = *reinterpret_cast<const uint4*>(src + q * 16);
  __syncthreads();
  // output pieces: 4 blocks x D dimensions x 2 halves of 16 bytes
  unsigned char* dst = reinterpret_cast<unsigned char*>(V16 + (static_cast<int64_t>(bh) * kp.n_cap + key0) * D);
  for (int q = tid; q < 4 * D * 2; q += 256) {
    const int t = q / (2 * D);
    const int w = q % (2 * D);
    const int d = w >> 1, hp = w & 1;
    const int h = hp ^ ((d >> 3) & 1);
    uint32_t pk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k0 = vblock_key(8 * h + 2 * i), k1 = vblock_key(8 * h + 2 * i + 1);
      const float f0 = __uint_as_float(static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(rows + (t * kBlk + k0) * RB + d * 2)) << 16);
      const float f1 = __uint_as_float(static_cast<uint32_t>(*reinterpret_cast<const uint16_t*>(rows + (t * kBlk + k1) * RB + d * 2)) << 16);
      const f16x2_t h2 = {static_cast<_Float16>(f0), static_cast<_Float16>(f1)};
      pk[i] = __builtin_bit_cast(uint32_t, h2);
    }
    *reinterpret_cast<uint4*>(dst + t * (D * 32) + d * 32 + hp * 16) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  }
}

// Three LDS tiles (ring slots), each a K tile and a V tile, copied straight from
// HBM into LDS.  The slots are separate variables and every access names its
// slot at compile time: the compiler then knows that reading one slot does not
// depend on the copy still in flight into another.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attend_prefill_pipe_kernel(AttendArgs a) {
  constexpr int NT = NW * 64;
  constexpr int KSTEPS = D / 16;  // QK^T k-steps
  constexpr int DBLK = D / 32;    // output blocks of 32 dims
  constexpr int CH = D / 8;       // 16-byte pieces per K row
  constexpr int RB = D * 2;       // bytes per K row
  constexpr int VB = D * 32;      // bytes per V block
  constexpr int TB = kTile * D * 2;     // bytes of a V tile
  constexpr int KP = CH + 1;            // 16-byte positions per padded K row
  constexpr int KRB = KP * 16;          // bytes per padded K row
  constexpr int KTB = kTile * KRB;      // bytes of a K tile (KP copies of 1 KB)
  constexpr int NI = TB / 1024 / NW;    // 1 KB copies per wave of the V tile
  static_assert(NI * NW * 1024 == TB, "V tile copies split evenly over the waves");
  const KParams& kp = a.kp;

  // ---- unit: KV head fastest (consecutive workgroups share a head's K/V in L2),
  // later (heavier) query chunks first
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
  const int hh = wid / 2;           // query head within the KV group
  const int pos0 = (wid & 1) * 32;  // first of the wave's 32 positions
  const int t_row0 = (a.q_pos ? a.q_pos[b] : 0) + a.pos_bias;
  const int qrow = u * kTile + pos0 + ql;
  const int64_t orow = (static_cast<int64_t>(b) * kp.Hq + static_cast<int64_t>(h) * kp.gq + hh) * a.nq + qrow;

  __shared__ __align__(16) unsigned char k0[KTB], k1[KTB], k2[KTB];
  __shared__ __align__(16) unsigned char v0[TB], v1[TB], v2[TB];
  // tile table: byte offsets of block t (16 keys) of tile tt in K and in the
  // fp16 V blocks (0 for an empty block), and the tile's valid blocks (bit t)
  __shared__ uint32_t tk[kMaxTiles][4], tv[kMaxTiles][4];
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

  if (t_row0 < 0 || static_cast<int64_t>(t_row0) + a.nq - 1 >= kp.n_cap || t_row0 % kTile != 0) {
    for (int e = lane; e < D; e += 64) {
      for (int r = 0; r < 32; ++r) {
        const int64_t off = ((static_cast<int64_t>(b) * kp.Hq + h * kp.gq + hh) * a.nq + u * kTile + pos0 + r) * D + e;
        if (a.out_bf16) reinterpret_cast<uint16_t*>(a.O)[off] = 0x7fc0u;
        else reinterpret_cast<float*>(a.O)[off] = __builtin_nanf("");
      }
    }
    return;
  }
  const int j = t_row0 / kTile + u;
  const int32_t* glg = a.group_idx + (static_cast<int64_t>(bh) * a.n_units + u) * kp.top_g;

  // ---- tile schedule: the current chunk, the other forced chunks, the routed groups
  const Forced fc = forced_chunks(j, kp.n_sink, kp.n_local);  // ascending, ends with j
  const int n_forced_other = fc.n - 1;
  const int bpg = kp.G / kBlk;       // blocks per routed group
  const int gpt = kTile / kp.G;      // routed groups per tile
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
    tv[tt][t] = kb >= 0 ? static_cast<uint32_t>(kb) * VB : 0u;
    // the valid bits of the tile, gathered by its block 0 thread
    const uint64_t ok = __ballot(kb >= 0);
    if (t == 0) tvm[tt] = static_cast<int>((ok >> (lane & ~3)) & 0xf);
  }

  // ---- the wave's query rows as the B operand of S^T = K Q^T
  bf16x8_t qv[KSTEPS];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(static_cast<const bf16*>(a.Q) + orow * D);
#pragma unroll
    for (int d = 0; d < KSTEPS; ++d) qv[d] = __builtin_bit_cast(bf16x8_t, qp[2 * d + hb]);
  }
  __syncthreads();

  const unsigned char* Kb = reinterpret_cast<const unsigned char*>(static_cast<const bf16*>(a.K) +
                                                                   static_cast<int64_t>(bh) * kp.n_cap * D);
  const unsigned char* Vb = reinterpret_cast<const unsigned char*>(static_cast<const uint16_t*>(a.V16) +
                                                                   static_cast<int64_t>(bh) * kp.n_cap * D);
  // Copy tile tt into slot S (no-op past the last tile).  Copy c fills bytes
  // [1024 c, 1024 c + 1024) of the slot's K or V tile, lane l writing 16 bytes
  // at 16 l.  K: position p = 64 c + l is piece p % KP of row p / KP (the last
  // position of a row is padding and loads a duplicate); V: the tile is its 4
  // blocks back to back.
  // This lane's part of the copies, fixed for the whole unit: K copy i of
  // this wave is copy c = wid + i NW (while c < KP), its lane loads piece
  // kpc of row kr (kr / 16 = its block); V copy i is c = wid NI + i, its lane
  // loads byte voff of block vt.
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
  uint32_t voff[NI];
  int vblk[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int p = 64 * (wid * NI + i) + lane;
    vblk[i] = p / (2 * D);
    voff[i] = static_cast<uint32_t>((p % (2 * D)) * 16);
  }
  auto copy_tile = [&](auto S, int tt) __attribute__((always_inline)) {
    if (tt >= n_tiles) return;
    unsigned char* ks = kslot(S);
    unsigned char* vs = vslot(S);
#pragma unroll
    for (int i = 0; i < NKC; ++i) {
      const int c = wid + i * NW;
      if (c < KP) {
        const unsigned char* src = Kb + tk[tt][kblk[i]] + koff[i];
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src),
                                         (__attribute__((address_space(3))) void*)(ks + 1024 * c), 16, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int c = wid * NI + i;
      const unsigned char* src = Vb + tv[tt][vblk[i]] + voff[i];
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src),
                                       (__attribute__((address_space(3))) void*)(vs + 1024 * c), 16, 0, 0);
    }
  };

  // S^T of sub-block sb (keys 32 sb .. 32 sb + 31 of the K tile ks): lane
  // (ql, hb) gets query ql against keys 32 sb + 8 (v / 4) + 4 hb + v % 4
  auto qk = [&](const unsigned char* ks, int sb) -> f32x16_t {
    f32x16_t acc = f32x16_t{};
    const unsigned char* rowp = ks + (32 * sb + ql) * KRB + hb * 16;
#pragma unroll
    for (int d = 0; d < KSTEPS; ++d) {
      const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(rowp + 32 * d);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qv[d], acc, 0, 0, 0);
    }
    return acc;
  };
  f32x16_t o[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) o[db] = f32x16_t{};
  // V fragments of the sub-block whose P.V comes next, read one sub-block
  // ahead (zeros before the first: its P is zero too)
  f16x8_t vf[2][DBLK];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int db = 0; db < DBLK; ++db) vf[t][db] = f16x8_t{};
  auto read_v = [&](const unsigned char* vs, int sb) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < DBLK; ++db)
        vf[t][db] = *reinterpret_cast<const f16x8_t*>(vs + (2 * sb + t) * VB + vblock_off(32 * db + ql, hb));
  };
  // O^T += V^T P^T with the fragments read ahead; pk[t] = P^T of k-step t
  auto pv = [&](const f16x8_t (&pk)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < DBLK; ++db) o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[t][db], pk[t], o[db], 0, 0, 0);
  };
  // masked scores (-inf) of sub-block sb of tile tt
  auto mask = [&](f32x16_t& s, int tt, int sb) {
    const int vm = __builtin_amdgcn_readfirstlane(tvm[tt]);
    if (tt > 0 && vm == 0xf) return;  // uniform: no masked key
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int kt = 32 * sb + 8 * (v >> 2) + 4 * hb + (v & 3);
      bool ok = (vm >> (kt >> 4)) & 1;
      if (tt == 0) ok = ok && kt <= pos0 + ql;  // causal inside the current chunk
      s[v] = ok ? s[v] : -__builtin_huge_valf();
    }
  };
  const float scale = kp.scale_log2;
  auto tile_max = [&](const f32x16_t& s) -> float {
    float mx = fmaxf(s[0], s[1]);
#pragma unroll
    for (int v = 2; v < 16; v += 2) mx = fmaxf(mx, fmaxf(s[v], s[v + 1]));
    float pa, pb;
    dpp::swap32(mx, pa, pb);
    return fmaxf(pa, pb) * scale;
  };

  // ---- prologue: tile 0 in slot 0, tile 1 in flight into slot 1, m from sub-block 0
  copy_tile(std::integral_constant<int, 0>{}, 0);
  __syncthreads();
  copy_tile(std::integral_constant<int, 1>{}, 1);
  f32x16_t s_cur = qk(k0, 0);
  mask(s_cur, 0, 0);
  float m_run = tile_max(s_cur);  // finite: key 0 of the current chunk is visible to every query
  float l_run = 0.f;
  f16x8_t pk_prev[2] = {f16x8_t{}, f16x8_t{}};
  const int nsb = 2 * n_tiles;
  const f16x2_t ones = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};

  // One 32-key sub-block bsb.  Its scores S(bsb) were launched one sub-block
  // earlier, so their mask and max come first (a rise of the reference max
  // rescales O, l and the pending P(bsb - 1)); then P.V of the previous
  // sub-block and S of the next one (K tile kn) go to the matrix cores while
  // P(bsb) and its row sum are computed and the V fragments of this
  // sub-block (V tile vs) are read for the next P.V.  The last sub-block's
  // "next" scores read whatever the slot holds and are dropped.
  auto sub = [&](int bsb, const unsigned char* kn, const unsigned char* vs) __attribute__((always_inline)) {
    if (bsb > 0) {  // sub-block 0's max is the initial reference
      mask(s_cur, bsb >> 1, bsb & 1);
      const float tmax = tile_max(s_cur);
      const bool raise = !(tmax <= m_run + 8.f);
      if (__ballot(raise)) {
        const float m_new = raise ? fmaxf(m_run, tmax) : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DBLK; ++db) o[db] *= alpha;
        const _Float16 ah = static_cast<_Float16>(alpha);
        pk_prev[0] *= ah;
        pk_prev[1] *= ah;
        m_run = m_new;
      }
    }
    pv(pk_prev);
    const f32x16_t s_nxt = qk(kn, (bsb + 1) & 1);
    f16x8_t pk_cur[2];
    float rs = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e0 = __builtin_amdgcn_exp2f(fmaf(s_cur[8 * t + 2 * i], scale, -m_run));
        const float e1 = __builtin_amdgcn_exp2f(fmaf(s_cur[8 * t + 2 * i + 1], scale, -m_run));
        const f16x2_t h2 = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_pkrtz(e0, e1));
        rs = __builtin_amdgcn_fdot2(h2, ones, rs, false);
        pk_cur[t][2 * i] = h2[0];
        pk_cur[t][2 * i + 1] = h2[1];
      }
    }
    read_v(vs, bsb & 1);
    {
      float pa, pb;
      dpp::swap32(rs, pa, pb);
      l_run += pa + pb;
    }
    pk_prev[0] = pk_cur[0];
    pk_prev[1] = pk_cur[1];
    s_cur = s_nxt;
  };
  // Tile T in slot S: sub-block 2T (next scores from this K tile), then,
  // once every wave is past its reads of slot S + 2 (the last were tile
  // T - 1's V fragments, in sub-block 2T - 1) and tile T + 1 has landed, tile
  // T + 2 starts copying into slot S + 2; then sub-block 2T + 1 (next scores
  // from slot S + 1).  Both read their V fragments from slot S.
  auto tile = [&](auto S, int T) __attribute__((always_inline)) {
    constexpr int s0 = decltype(S)::value, s1 = (s0 + 1) % kRing, s2 = (s0 + 2) % kRing;
    const std::integral_constant<int, s1> S1{};
    const std::integral_constant<int, s2> S2{};
    sub(2 * T, kslot(S), vslot(S));
    __syncthreads();
    copy_tile(S2, T + 2);
    sub(2 * T + 1, kslot(S1), vslot(S));
  };
  static_assert(kRing == 3, "the tile loop names three slots");
  for (int T = 0; T < n_tiles; T += kRing) {
    tile(std::integral_constant<int, 0>{}, T);
    if (T + 1 < n_tiles) tile(std::integral_constant<int, 1>{}, T + 1);
    if (T + 2 < n_tiles) tile(std::integral_constant<int, 2>{}, T + 2);
  }
  pv(pk_prev);  // the last sub-block

  // ---- O = O^T / l: lane (query, half) holds dims 32db + 8i + 4*half + {0..3}
  const float inv = 1.f / l_run;
#pragma unroll
  for (int db = 0; db < DBLK; ++db) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = 32 * db + 8 * i + 4 * hb;
      const float4 v4 = make_float4(o[db][4 * i] * inv, o[db][4 * i + 1] * inv, o[db][4 * i + 2] * inv,
                                    o[db][4 * i + 3] * inv);
      if (a.out_bf16) {
        uint16_t* op = reinterpret_cast<uint16_t*>(a.O) + orow * D + d0;
        const uint2 pk2 = make_uint2(static_cast<uint32_t>(f32_to_bf16(v4.x)) | (static_cast<uint32_t>(f32_to_bf16(v4.y)) << 16),
                                     static_cast<uint32_t>(f32_to_bf16(v4.z)) | (static_cast<uint32_t>(f32_to_bf16(v4.w)) << 16));
        *reinterpret_cast<uint2*>(op) = pk2;
      } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.O) + orow * D + d0) = v4;
      }
    }
  }
  if (a.lse && hb == 0) a.lse[orow] = (m_run + log2f(l_run)) * 0.69314718055994531f;
}

bool prefill_pipe_supported(const KParams& kp, bool bf16_in, int64_t nq) {
  if (!(bf16_in && nq > 1 && kp.C == kTile && (kp.d == 64 || kp.d == 128) &&
        (kp.gq == 1 || kp.gq == 2 || kp.gq == 4) && kp.G % kBlk == 0 && kTile % kp.G == 0))
    return false;
  const int64_t tiles = 1 + static_cast<int64_t>(kp.n_sink) + kp.n_local +
                        (static_cast<int64_t>(kp.top_g) * kp.G + kTile - 1) / kTile;
  // the tile table holds 32-bit byte offsets into one (b, KV head)'s rows
  return tiles <= kMaxTiles && kp.n_cap * kp.d * 2 <= 0xffffffffll;
}

size_t prefill_pipe_v16_bytes(const KParams& kp) {
  return static_cast<size_t>(kp.B) * kp.Hkv * kp.n_cap * kp.d * sizeof(uint16_t);
}

template <int D, int NW>
static hipError_t launch_t(const AttendArgs& a, hipStream_t st) {
  const KParams& kp = a.kp;
  const dim3 pg(static_cast<unsigned>(kp.n_cap / kTile), static_cast<unsigned>(kp.B * kp.Hkv));
  v16_blocks_kernel<D><<<pg, 256, 0, st>>>(static_cast<const bf16*>(a.V), static_cast<uint16_t*>(a.V16), kp,
                                           a.q_pos, a.pos_bias, a.nq);
  const unsigned n_wg = static_cast<unsigned>(kp.B) * kp.Hkv * a.n_units;
  attend_prefill_pipe_kernel<D, NW><<<n_wg, NW * 64, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_attend_prefill_pipe(const AttendArgs& a, hipStream_t st) {
  if (!a.V16) return hipErrorInvalidValue;
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
