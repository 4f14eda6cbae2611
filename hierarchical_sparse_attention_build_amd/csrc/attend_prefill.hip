// Steps 4-5 of HGA for prefill on the matrix cores: visibility union + exact
// softmax attention of one routing unit (a query chunk of C = 64 positions and
// all query heads of a KV head) over its gathered K/V tiles.
// [HGA technical summary (it), Meccanismo Core, item 2 third bullet and item 4].
//
// One workgroup per unit; each wave owns 32 query rows (one head, 32
// positions).  The unit's keys come in tiles of 64 rows: first the current
// chunk (causal), then the other always-visible chunks (sink, local), then the
// routed groups (64/G groups per tile).  Tiles are gathered row by row from
// HBM into LDS (double-buffered; the next tile's loads are in flight while the
// current one is computed): K row-major (bf16), V transposed and converted to
// fp16.
//
// Per tile and wave, with 32x32x16 MFMAs:
//   S^T = K Q^T        (bf16 operands, fp32 accumulate): a lane holds the
//                      scores of one query against 32 of the 64 keys;
//   online softmax     per lane in base 2, partner half-wave via permlane32;
//   O^T += V^T P^T     (fp16 operands): P^T is taken straight from the score
//                      registers (the key order inside each 16-key step is
//                      permuted consistently on the V^T side), so no P
//                      round trip through LDS is needed.
// P is rounded to fp16 (2^-11 relative), V to fp16 exactly for |v| < 65504.
// The running max is raised only when a tile's max exceeds it by more than
// 2^8 (base 2): O / l does not depend on the reference max, p stays <= 256,
// and most tiles skip the rescale of the accumulators.
#include "hga_device.hpp"
#include "hga_kernels.hpp"

namespace hga {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kPTile = 64;  // keys per tile

template <int D>
struct PrefillSmem {
  static constexpr int KROW = D * 2 + 16;     // bytes per K row (padded against bank conflicts)
  static constexpr int VROW = kPTile * 2 + 8;  // bytes per V^T row (padded)
  alignas(16) unsigned char k[2][kPTile * KROW];
  alignas(16) unsigned char vt[2][D * VROW];
  unsigned long long valid[2];  // bit r: tile row r holds a visible token
  int gl[1024];
};

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attend_prefill_mfma_kernel(AttendArgs a) {
  constexpr int NT = NW * 64;
  constexpr int KSTEPS = D / 16;             // QK^T k-steps
  constexpr int DBLK = D / 32;               // output blocks of 32 dims
  constexpr int CH = D / 8;                  // 16-byte chunks per row
  using Smem = PrefillSmem<D>;
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
  const int hh = wid / 2;             // query head within the KV group
  const int pos0 = (wid & 1) * 32;    // first of the wave's 32 positions
  const int t_row0 = (a.q_pos ? a.q_pos[b] : 0) + a.pos_bias;
  const int qrow = u * kPTile + pos0 + ql;
  const int64_t orow = (static_cast<int64_t>(b) * kp.Hq + static_cast<int64_t>(h) * kp.gq + hh) * a.nq + qrow;

  __shared__ Smem sm;

  if (t_row0 < 0 || static_cast<int64_t>(t_row0) + a.nq - 1 >= kp.n_cap || t_row0 % kPTile != 0) {
    for (int e = lane; e < D; e += 64) {
      for (int r = 0; r < 32; ++r) {
        const int64_t off = ((static_cast<int64_t>(b) * kp.Hq + h * kp.gq + hh) * a.nq + u * kPTile + pos0 + r) * D + e;
        if (a.out_bf16) reinterpret_cast<uint16_t*>(a.O)[off] = 0x7fc0u;
        else reinterpret_cast<float*>(a.O)[off] = __builtin_nanf("");
      }
    }
    return;
  }
  const int j = t_row0 / kPTile + u;

  const int32_t* glg = a.group_idx + (static_cast<int64_t>(bh) * a.n_units + u) * kp.top_g;
  for (int e = tid; e < kp.top_g; e += NT) sm.gl[e] = glg[e];

  // ---- the wave's query rows as the B operand of S^T = K Q^T
  bf16x8_t qv[KSTEPS];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(static_cast<const bf16*>(a.Q) + orow * D);
#pragma unroll
    for (int d = 0; d < KSTEPS; ++d) qv[d] = __builtin_bit_cast(bf16x8_t, qp[2 * d + hb]);
  }
  __syncthreads();

  // ---- tile schedule
  const Forced fc = forced_chunks(j, kp.n_sink, kp.n_local);  // ascending, ends with j
  const int n_forced_other = fc.n - 1;
  const int gpt = kPTile / kp.G;  // routed groups per tile
  const int n_routed_tiles = (kp.top_g + gpt - 1) / gpt;
  const int n_tiles = 1 + n_forced_other + n_routed_tiles;
  const int n_groups_cap = static_cast<int>(kp.n_cap / kp.G);
  const bf16* Kb = static_cast<const bf16*>(a.K);
  const bf16* Vb = static_cast<const bf16*>(a.V);

  // token of row r of tile tt, or -1
  auto tile_token = [&](int tt, int r) -> int64_t {
    if (tt == 0) return static_cast<int64_t>(j) * kPTile + r;
    if (tt <= n_forced_other) return static_cast<int64_t>(forced_chunk_at(fc, tt - 1)) * kPTile + r;
    const int rt = tt - 1 - n_forced_other;
    const int rg = kp.log2G >= 0 ? r >> kp.log2G : r / kp.G;
    const int e = rt * gpt + rg;
    if (e >= kp.top_g) return -1;
    const int g = sm.gl[e];
    if (g < 0 || g >= n_groups_cap) return -1;
    return static_cast<int64_t>(g) * kp.G + (r - rg * kp.G);
  };

  // Each thread moves CPT 16-byte pieces of K and of V per tile: pieces of two
  // adjacent rows (same columns), so that V^T gets packed pairs of fp16 keys.
  constexpr int PAIRS = kPTile / 2 * CH;
  constexpr int NPAIR = (PAIRS + NT - 1) / NT;
  uint4 kreg[2 * NPAIR], vreg[2 * NPAIR];
  auto fetch = [&](int tt) {
#pragma unroll
    for (int i = 0; i < NPAIR; ++i) {
      const int q = tid + i * NT;
      if (PAIRS % NT != 0 && q >= PAIRS) break;
      const int r = 2 * (q / CH), c = q % CH;
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const int64_t tok = tile_token(tt, r + w);
        if (tok >= 0) {
          const int64_t off = (static_cast<int64_t>(bh) * kp.n_cap + tok) * D + c * 8;
          kreg[2 * i + w] = *reinterpret_cast<const uint4*>(Kb + off);
          vreg[2 * i + w] = *reinterpret_cast<const uint4*>(Vb + off);
        } else {
          kreg[2 * i + w] = make_uint4(0u, 0u, 0u, 0u);
          vreg[2 * i + w] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
    }
  };
  auto stage = [&](int buf, int tt) {
#pragma unroll
    for (int i = 0; i < NPAIR; ++i) {
      const int q = tid + i * NT;
      if (PAIRS % NT != 0 && q >= PAIRS) break;
      const int r = 2 * (q / CH), c = q % CH;
      *reinterpret_cast<uint4*>(&sm.k[buf][r * Smem::KROW + c * 16]) = kreg[2 * i];
      *reinterpret_cast<uint4*>(&sm.k[buf][(r + 1) * Smem::KROW + c * 16]) = kreg[2 * i + 1];
      const uint32_t w0[4] = {vreg[2 * i].x, vreg[2 * i].y, vreg[2 * i].z, vreg[2 * i].w};
      const uint32_t w1[4] = {vreg[2 * i + 1].x, vreg[2 * i + 1].y, vreg[2 * i + 1].z, vreg[2 * i + 1].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f0 = (e & 1) ? bf16hi(w0[e >> 1]) : bf16lo(w0[e >> 1]);
        const float f1 = (e & 1) ? bf16hi(w1[e >> 1]) : bf16lo(w1[e >> 1]);
        const f16x2_t h2 = {static_cast<_Float16>(f0), static_cast<_Float16>(f1)};
        *reinterpret_cast<f16x2_t*>(&sm.vt[buf][(c * 8 + e) * Smem::VROW + r * 2]) = h2;
      }
    }
    if (tid < kPTile) {
      const bool ok = tile_token(tt, tid) >= 0;
      const uint64_t m = __ballot(ok);
      if (tid == 0) sm.valid[buf] = m;
    }
  };

  f32x16_t o[DBLK];
#pragma unroll
  for (int db = 0; db < DBLK; ++db) o[db] = f32x16_t{};
  float m_run = -__builtin_huge_valf(), l_run = 0.f;
  const float scale = kp.scale_log2;

  fetch(0);
  stage(0, 0);
  __syncthreads();
  for (int tt = 0; tt < n_tiles; ++tt) {
    const int buf = tt & 1;
    if (tt + 1 < n_tiles) fetch(tt + 1);

    // ---- S^T = K Q^T for keys [0,32) and [32,64) of the tile
    f32x16_t s[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
    for (int d = 0; d < KSTEPS; ++d) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(
            &sm.k[buf][(32 * blk + ql) * Smem::KROW + (16 * d + 8 * hb) * 2]);
        s[blk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qv[d], s[blk], 0, 0, 0);
      }
    }
    // ---- online softmax (this lane: one query, 32 keys; partner lane: the rest)
    const uint64_t vmask = sm.valid[buf];
    const bool full = tt > 0 && vmask == ~0ull;  // uniform: no masked key in the tile
    float tmax = -__builtin_huge_valf();
    if (full) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, s[blk][v]);
    } else {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kt = 32 * blk + 8 * (v >> 2) + 4 * hb + (v & 3);
          bool ok = (vmask >> kt) & 1ull;
          if (tt == 0) ok = ok && kt <= pos0 + ql;  // causal inside the current chunk
          const float sv = ok ? s[blk][v] : -__builtin_huge_valf();
          s[blk][v] = sv;
          tmax = fmaxf(tmax, sv);
        }
      }
    }
    {
      float pa, pb;
      dpp::swap32(tmax, pa, pb);
      tmax = fmaxf(pa, pb) * scale;
    }
    // raise the reference max only when this tile's max exceeds it by > 8
    const bool raise = !(tmax <= m_run + 8.f);
    if (__ballot(raise)) {
      const float m_new = raise ? fmaxf(m_run, tmax) : m_run;
      const float alpha = m_run == -__builtin_huge_valf() ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DBLK; ++db) o[db] *= alpha;
      m_run = m_new;
    }
    float rs = 0.f;
    f16x8_t pk[4];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const _Float16 ph = static_cast<_Float16>(__builtin_amdgcn_exp2f(fmaf(s[blk][v], scale, -m_run)));
        rs += static_cast<float>(ph);  // normalise by the weights actually used
        pk[2 * blk + (v >> 3)][v & 7] = ph;
      }
    }
    {
      float pa, pb;
      dpp::swap32(rs, pa, pb);
      rs = pa + pb;
    }
    l_run += rs;
    // ---- O^T += V^T P^T
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int db = 0; db < DBLK; ++db) {
        const unsigned char* vrow = &sm.vt[buf][(32 * db + ql) * Smem::VROW];
        const f16x4_t lo = *reinterpret_cast<const f16x4_t*>(vrow + (16 * t + 4 * hb) * 2);
        const f16x4_t hi = *reinterpret_cast<const f16x4_t*>(vrow + (16 * t + 4 * hb + 8) * 2);
        const f16x8_t va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pk[t], o[db], 0, 0, 0);
      }
    }
    if (tt + 1 < n_tiles) stage(buf ^ 1, tt + 1);
    __syncthreads();
  }

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

bool prefill_mfma_supported(const KParams& kp, bool bf16_in, int64_t nq) {
  return bf16_in && nq > 1 && kp.C == kPTile && (kp.d == 64 || kp.d == 128) &&
         (kp.gq == 1 || kp.gq == 2 || kp.gq == 4) && kPTile % kp.G == 0 && kp.top_g <= 1024;
}

template <int D, int NW>
static hipError_t launch_t(const AttendArgs& a, hipStream_t st) {
  const unsigned n_wg = static_cast<unsigned>(a.kp.B) * a.kp.Hkv * a.n_units;
  attend_prefill_mfma_kernel<D, NW><<<n_wg, NW * 64, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_attend_prefill_mfma(const AttendArgs& a, hipStream_t st) {
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
