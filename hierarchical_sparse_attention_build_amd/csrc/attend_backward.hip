// Backward of the prefill attention: gradients of O with respect to Q, K and V
// over each query's selected token set, with the routing held fixed (the
// selection is a piecewise-constant function of the inputs, so no gradient
// flows through it).  [HGA technical summary (it), Meccanismo Core, item 4:
// the output is an exact softmax over the selected tokens.]
//
// For one query row with scores z_u = q.k_u / sqrt(d) over its visible set,
// p = softmax(z) and o = sum_u p_u v_u:
//   D = sum_u p_u (do.v_u) (= do.o),   dz_u = p_u (do.v_u - D),
//   dq = sum_u dz_u k_u / sqrt(d),   dk_u += dz_u q / sqrt(d),   dv_u += p_u do.
//
// This file is the path for fp32 inputs and for shapes the matrix-core
// backward (attend_backward_mfma.hip, bf16 inputs) does not take.  Two gather
// kernels, all arithmetic in fp32 on the vector ALUs:
//   * bwd_dq_kernel, one workgroup per (query chunk, b, kv head, query head):
//     thread (row, quarter) holds a quarter of one query row.  A first pass
//     over the visible tiles gets the row's softmax statistics (max, sum) and
//     D; a second pass accumulates dq.  It also stores (log-sum-exp, D) of
//     every row for the second kernel.
//   * bwd_dkv_kernel, one workgroup per (block of 16 key rows, slice of query
//     chunks, b, kv head): lane (key row, quarter) of every wave holds a
//     quarter of one key and one value row; the workgroup walks the query
//     chunks of its slice that see rows of the block (always-visible windows,
//     or routed groups in the query chunk's list), each wave taking a quarter
//     of their query rows, and accumulates dk and dv.  The waves' partials
//     meet in LDS and the slices' sums in dK and dV through device-scope float
//     atomics.
// Dot products over a row reduce across the four quarter-threads of a quad
// with two DPP steps.
#include "hga_device.hpp"
#include "hga_kernels.hpp"

namespace hga {

constexpr int kBwdRows = 64;                 // rows per workgroup (one chunk, C = 64)
constexpr int kBwdThreads = kBwdRows * 4;    // a quad of threads per row

typedef __bf16 bwd_bf16x2 __attribute__((ext_vector_type(2)));

// a.b over N/2 packed bf16 pairs on v_dot2_f32_bf16 (products exact in fp32,
// fp32 sums), four partial sums
template <int NW>
__device__ __forceinline__ float dot_bf16(const uint32_t (&a)[NW], const uint32_t (&b)[NW]) {
  float x[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NW; ++i)
    x[i & 3] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bwd_bf16x2, a[i]), __builtin_bit_cast(bwd_bf16x2, b[i]),
                                               x[i & 3], false);
  return (x[0] + x[1]) + (x[2] + x[3]);
}

template <int NW>
__device__ __forceinline__ void load_words(const void* p, uint32_t (&w)[NW]) {
  const uint4* s = static_cast<const uint4*>(p);
#pragma unroll
  for (int v = 0; v < NW / 4; ++v) {
    const uint4 x = s[v];
    w[4 * v] = x.x;
    w[4 * v + 1] = x.y;
    w[4 * v + 2] = x.z;
    w[4 * v + 3] = x.w;
  }
}

// Two dot products of N-element rows with four partial sums each (short
// dependency chains).
template <int N>
__device__ __forceinline__ void dot2(const float (&a)[N], const float (&b)[N], const float (&c)[N],
                                     const float (&e)[N], float& ab, float& ce) {
  float x[4] = {0.f, 0.f, 0.f, 0.f}, y[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < N; ++i) {
    x[i & 3] = fmaf(a[i], b[i], x[i & 3]);
    y[i & 3] = fmaf(c[i], e[i], y[i & 3]);
  }
  ab = (x[0] + x[1]) + (x[2] + x[3]);
  ce = (y[0] + y[1]) + (y[2] + y[3]);
}

__device__ __forceinline__ float quad_sum(float v) {
  v += dpp::movf<dpp::kQuad1032>(v);
  v += dpp::movf<dpp::kQuad2301>(v);
  return v;
}

template <typename T, int D>
struct BwdTileSmem {
  alignas(16) T k[kBwdRows * D];
  alignas(16) T v[kBwdRows * D];
  int tok[kBwdRows];   // token of each tile row, -1 if masked
  int gl[1024];
};

// Token of row r of tile tt of query chunk j (-1 if masked).  Tile 0 is chunk j
// itself, then the other always-visible chunks, then the routed groups in list
// order, 64 / G groups per tile (the forward prefill's schedule).
__device__ __forceinline__ int64_t bwd_tile_token(const KParams& kp, const Forced& fc, int j, const int* gl,
                                                  int tt, int r) {
  const int n_forced_other = fc.n - 1;
  if (tt == 0) return static_cast<int64_t>(j) * kp.C + r;
  if (tt <= n_forced_other) return static_cast<int64_t>(forced_chunk_at(fc, tt - 1)) * kp.C + r;
  const int gpt = kp.C / kp.G;
  const int rt = tt - 1 - n_forced_other;
  const int rg = r >> kp.log2G;
  const int e = rt * gpt + rg;
  if (e >= kp.top_g) return -1;
  const int g = gl[e];
  if (g < 0 || g >= static_cast<int>(kp.n_cap >> kp.log2G)) return -1;
  return (static_cast<int64_t>(g) << kp.log2G) + (r - (rg << kp.log2G));
}

template <typename T, int D>
__device__ __forceinline__ void bwd_stage_tile(const BackwardArgs& a, int64_t bh, const Forced& fc, int j, int tt,
                                               BwdTileSmem<T, D>& sm) {
  const KParams& kp = a.kp;
  constexpr int PER = D * static_cast<int>(sizeof(T)) / 16;  // 16-byte pieces per row
  const T* Kb = static_cast<const T*>(a.K) + bh * kp.n_cap * D;
  const T* Vb = static_cast<const T*>(a.V) + bh * kp.n_cap * D;
  for (int e = threadIdx.x; e < kBwdRows * PER; e += kBwdThreads) {
    const int r = e / PER, c = e % PER;
    const int64_t tok = bwd_tile_token(kp, fc, j, sm.gl, tt, r);
    uint4 kv = make_uint4(0u, 0u, 0u, 0u), vv = kv;
    if (tok >= 0) {
      kv = reinterpret_cast<const uint4*>(Kb + tok * D)[c];
      vv = reinterpret_cast<const uint4*>(Vb + tok * D)[c];
    }
    reinterpret_cast<uint4*>(sm.k + r * D)[c] = kv;
    reinterpret_cast<uint4*>(sm.v + r * D)[c] = vv;
    if (c == 0) sm.tok[r] = static_cast<int>(tok);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kBwdThreads, 3) void bwd_dq_kernel(BackwardArgs a) {
  constexpr int QD = D / 4;
  const KParams& kp = a.kp;
  const int j = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const int hh = blockIdx.z;
  const int b = static_cast<int>(bh / kp.Hkv), h = static_cast<int>(bh % kp.Hkv);
  const int r = threadIdx.x >> 2, qq = threadIdx.x & 3;
  const int pos = j * kp.C + r;
  const int64_t qrow = (static_cast<int64_t>(b) * kp.Hq + h * kp.gq + hh) * a.n + pos;
  __shared__ BwdTileSmem<T, D> sm;

  const int32_t* glg = a.group_idx + (bh * a.n_units + j) * kp.top_g;
  for (int e = threadIdx.x; e < kp.top_g; e += kBwdThreads) sm.gl[e] = glg[e];
  float q[QD], dout[QD], dq[QD];
  uint32_t qw[QD / 2];  // packed bf16 pairs of q (bf16 inputs)
  if constexpr (sizeof(T) == 2) load_words(static_cast<const T*>(a.Q) + qrow * D + qq * QD, qw);
  else load_row<T, QD>(static_cast<const T*>(a.Q) + qrow * D + qq * QD, q);
  load_row<float, QD>(a.dO + qrow * D + qq * QD, dout);
#pragma unroll
  for (int i = 0; i < QD; ++i) dq[i] = 0.f;
  __syncthreads();

  const Forced fc = forced_chunks(j, kp.n_sink, kp.n_local);
  const int n_tiles = fc.n + (kp.top_g + kp.C / kp.G - 1) / (kp.C / kp.G);
  const float sc2 = kp.scale_log2;
  // pass 1: max m and sum l of 2^(z log2 e), and D' = sum 2^(...) (do.v)
  float m = -__builtin_huge_valf(), l = 0.f, dsum = 0.f;
  for (int pass = 0; pass < 2; ++pass) {
    const float lse2 = m + __builtin_log2f(l);
    const float Dv = dsum / l;
    for (int tt = 0; tt < n_tiles; ++tt) {
      bwd_stage_tile<T, D>(a, bh, fc, j, tt, sm);
      __syncthreads();
      for (int kr = 0; kr < kBwdRows; ++kr) {
        const int tok = sm.tok[kr];
        if (tok < 0 || tok > pos) continue;  // masked, or after the query (causal)
        float kv[QD], vv[QD];
        float s, dp;
        if constexpr (sizeof(T) == 2) {
          // bf16: q.k on the packed pairs; k unpacked only for dq
          uint32_t kw[QD / 2];
          load_words(sm.k + kr * D + qq * QD, kw);
          s = dot_bf16(qw, kw);
          if (pass == 1) {
#pragma unroll
            for (int i = 0; i < QD / 2; ++i) {
              kv[2 * i] = bf16lo(kw[i]);
              kv[2 * i + 1] = bf16hi(kw[i]);
            }
          }
          load_row<T, QD>(sm.v + kr * D + qq * QD, vv);
          float y[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int i = 0; i < QD; ++i) y[i & 3] = fmaf(dout[i], vv[i], y[i & 3]);
          dp = (y[0] + y[1]) + (y[2] + y[3]);
        } else {
          load_row<T, QD>(sm.k + kr * D + qq * QD, kv);
          load_row<T, QD>(sm.v + kr * D + qq * QD, vv);
          dot2(q, kv, dout, vv, s, dp);
        }
        s = quad_sum(s) * sc2;
        dp = quad_sum(dp);
        if (pass == 0) {
          if (s > m) {
            const float al = __builtin_amdgcn_exp2f(m - s);  // 0 while m = -inf
            l *= al;
            dsum *= al;
            m = s;
          }
          const float e = __builtin_amdgcn_exp2f(s - m);
          l += e;
          dsum = fmaf(e, dp, dsum);
        } else {
          const float p = __builtin_amdgcn_exp2f(s - lse2);
          const float ds = p * (dp - Dv);
#pragma unroll
          for (int i = 0; i < QD; ++i) dq[i] = fmaf(ds, kv[i], dq[i]);
        }
      }
      __syncthreads();
    }
    if (pass == 1 && qq == 0) {
      a.stats[2 * qrow] = lse2;
      a.stats[2 * qrow + 1] = Dv;
    }
  }
#pragma unroll
  for (int i = 0; i < QD; ++i) a.dQ[qrow * D + qq * QD + i] = dq[i] * kp.inv_sqrt_d;
}

constexpr int kBwdKeyRows = 16;  // key rows per dK/dV workgroup
constexpr int kBwdWaves = kBwdThreads / kWave;

template <typename T, int D>
struct BwdSrcSmem {
  // a source chunk's query rows of one head; reused at the end for the
  // waves' partial dK, dV (kBwdWaves - 1 of them)
  alignas(16) T q[kBwdRows * D];
  alignas(16) float dout[kBwdRows * D];
  float lse2[kBwdRows];
  float dv[kBwdRows];
  int vis;     // bit r: key row r of the block visible to the source chunk
  int causal;  // the source chunk is the key block's own chunk
};

template <typename T, int D>
__global__ __launch_bounds__(kBwdThreads, 3) void bwd_dkv_kernel(BackwardArgs a) {
  constexpr int QD = D / 4;
  static_assert((kBwdWaves - 1) * kBwdKeyRows * D * 2 * sizeof(float) <=
                    kBwdRows * D * (sizeof(T) + sizeof(float)), "partials fit the staging area");
  const KParams& kp = a.kp;
  const int kb = blockIdx.x;                    // key block: rows [16 kb, 16 kb + 16)
  const int c = kb * kBwdKeyRows / kp.C;        // its chunk
  const int s0 = blockIdx.y * a.unit_slice;
  const int64_t bh = blockIdx.z;
  const int b = static_cast<int>(bh / kp.Hkv), h = static_cast<int>(bh % kp.Hkv);
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = wave_id();
  const int kr = lane >> 2, qq = lane & 3;
  const int j_lo = max(s0, c), j_hi = min(s0 + a.unit_slice, a.n_units);
  if (j_lo >= j_hi) return;  // no query chunk of this slice sees the block
  __shared__ BwdSrcSmem<T, D> sm;

  const int64_t ktok0 = static_cast<int64_t>(kb) * kBwdKeyRows;
  const int64_t ktok = ktok0 + kr;
  float kv[QD], vv[QD], dk[QD], dvv[QD];
  uint32_t kw[QD / 2];  // packed bf16 pairs of k (bf16 inputs)
  if constexpr (sizeof(T) == 2) load_words(static_cast<const T*>(a.K) + (bh * kp.n_cap + ktok) * D + qq * QD, kw);
  else load_row<T, QD>(static_cast<const T*>(a.K) + (bh * kp.n_cap + ktok) * D + qq * QD, kv);
  load_row<T, QD>(static_cast<const T*>(a.V) + (bh * kp.n_cap + ktok) * D + qq * QD, vv);
#pragma unroll
  for (int i = 0; i < QD; ++i) dk[i] = dvv[i] = 0.f;
  const float sc2 = kp.scale_log2;
  bool any = false;

  for (int j = j_lo; j < j_hi; ++j) {
    // ---- which rows of the block do chunk j's queries see?
    if (wid == 0) {
      int vis = 0;
      const bool forced = c < kp.n_sink || (c >= j - kp.n_local && c <= j);
      if (forced) {
        vis = (1 << kBwdKeyRows) - 1;
      } else {
        const int32_t* gl = a.group_idx + (bh * a.n_units + j) * kp.top_g;
        for (int e0 = 0; e0 < kp.top_g; e0 += kWave) {
          const int g = e0 + lane < kp.top_g ? gl[e0 + lane] : -1;
          int bits = 0;
          if (g >= 0) {
            const int64_t lo = max(static_cast<int64_t>(g) << kp.log2G, ktok0);
            const int64_t hi = min((static_cast<int64_t>(g) + 1) << kp.log2G, ktok0 + kBwdKeyRows);
            if (lo < hi) bits = ((1 << (hi - lo)) - 1) << (lo - ktok0);
          }
          for (int o = 32; o >= 1; o >>= 1) bits |= __shfl_xor(bits, o);
          vis |= bits;
        }
      }
      if (lane == 0) {
        sm.vis = vis;
        sm.causal = c == j;
      }
    }
    __syncthreads();
    const int vis = sm.vis;
    const bool causal = sm.causal != 0;
    __syncthreads();  // every thread has read vis before wave 0 writes the next one
    if (vis == 0) continue;
    any = true;
    const bool key_visible = (vis >> kr) & 1;
    for (int hh = 0; hh < kp.gq; ++hh) {
      // ---- stage chunk j's rows of query head hh: q, do, log-sum-exp, D
      const int64_t row0 = (static_cast<int64_t>(b) * kp.Hq + h * kp.gq + hh) * a.n + static_cast<int64_t>(j) * kp.C;
      constexpr int QP = D * static_cast<int>(sizeof(T)) / 16;
      for (int e = threadIdx.x; e < kBwdRows * QP; e += kBwdThreads)
        reinterpret_cast<uint4*>(sm.q)[e] = reinterpret_cast<const uint4*>(static_cast<const T*>(a.Q) + row0 * D)[e];
      for (int e = threadIdx.x; e < kBwdRows * D / 4; e += kBwdThreads)
        reinterpret_cast<float4*>(sm.dout)[e] = reinterpret_cast<const float4*>(a.dO + row0 * D)[e];
      if (threadIdx.x < kBwdRows) {
        sm.lse2[threadIdx.x] = a.stats[2 * (row0 + threadIdx.x)];
        sm.dv[threadIdx.x] = a.stats[2 * (row0 + threadIdx.x) + 1];
      }
      __syncthreads();
      if (key_visible) {
        // wave w takes query rows [16 w, 16 w + 16); causal: queries at or after the key
        const int r_lo = wid * (kBwdRows / kBwdWaves);
        const int r_hi = r_lo + kBwdRows / kBwdWaves;
        const int first = causal ? max(r_lo, static_cast<int>(ktok - static_cast<int64_t>(j) * kp.C)) : r_lo;
        for (int r = first; r < r_hi; ++r) {
          float q[QD], dout[QD];
          float s, dp;
          if constexpr (sizeof(T) == 2) {
            uint32_t qw[QD / 2];
            load_words(sm.q + r * D + qq * QD, qw);
            s = dot_bf16(qw, kw);
#pragma unroll
            for (int i = 0; i < QD / 2; ++i) {
              q[2 * i] = bf16lo(qw[i]);
              q[2 * i + 1] = bf16hi(qw[i]);
            }
            load_row<float, QD>(sm.dout + r * D + qq * QD, dout);
            float y[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < QD; ++i) y[i & 3] = fmaf(dout[i], vv[i], y[i & 3]);
            dp = (y[0] + y[1]) + (y[2] + y[3]);
          } else {
            load_row<T, QD>(sm.q + r * D + qq * QD, q);
            load_row<float, QD>(sm.dout + r * D + qq * QD, dout);
            dot2(q, kv, dout, vv, s, dp);
          }
          s = quad_sum(s) * sc2;
          dp = quad_sum(dp);
          const float p = __builtin_amdgcn_exp2f(s - sm.lse2[r]);
          const float ds = p * (dp - sm.dv[r]);
#pragma unroll
          for (int i = 0; i < QD; ++i) {
            dk[i] = fmaf(ds, q[i], dk[i]);
            dvv[i] = fmaf(p, dout[i], dvv[i]);
          }
        }
      }
      __syncthreads();
    }
  }
  if (!any) return;
  // ---- sum the waves' partials in LDS, then add the block's rows to dK, dV
  float* red = reinterpret_cast<float*>(sm.q);  // [wave - 1][row][d][2]
  if (wid > 0) {
    float* mine = red + (wid - 1) * kBwdKeyRows * D * 2 + (kr * D + qq * QD) * 2;
#pragma unroll
    for (int i = 0; i < QD; ++i) {
      mine[2 * i] = dk[i];
      mine[2 * i + 1] = dvv[i];
    }
  }
  __syncthreads();
  if (wid == 0) {
    for (int w = 1; w < kBwdWaves; ++w) {
      const float* other = red + (w - 1) * kBwdKeyRows * D * 2 + (kr * D + qq * QD) * 2;
#pragma unroll
      for (int i = 0; i < QD; ++i) {
        dk[i] += other[2 * i];
        dvv[i] += other[2 * i + 1];
      }
    }
    float* dKr = a.dK + (bh * kp.n_cap + ktok) * D + qq * QD;
    float* dVr = a.dV + (bh * kp.n_cap + ktok) * D + qq * QD;
#pragma unroll
    for (int i = 0; i < QD; ++i) {
      __hip_atomic_fetch_add(dKr + i, dk[i] * kp.inv_sqrt_d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(dVr + i, dvv[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

__global__ void bwd_zero_kernel(float* p, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0.f;
}

bool backward_supported(const KParams& kp) {
  return kp.C == kBwdRows && (kp.d == 64 || kp.d == 128) && kp.log2G >= 0 && kp.top_g <= 1024;
}

template <typename T, int D>
static hipError_t launch_t(const BackwardArgs& a, hipStream_t st) {
  const KParams& kp = a.kp;
  const int64_t kv_elems = static_cast<int64_t>(kp.B) * kp.Hkv * kp.n_cap * D;
  bwd_zero_kernel<<<1024, 256, 0, st>>>(a.dK, kv_elems);
  bwd_zero_kernel<<<1024, 256, 0, st>>>(a.dV, kv_elems);
  bwd_dq_kernel<T, D><<<dim3(a.n_units, kp.B * kp.Hkv, kp.gq), kBwdThreads, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int slices = (a.n_units + a.unit_slice - 1) / a.unit_slice;
  const int blocks = static_cast<int>(kp.n_cap / kBwdKeyRows);
  bwd_dkv_kernel<T, D><<<dim3(blocks, slices, kp.B * kp.Hkv), kBwdThreads, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_backward(const BackwardArgs& a, bool bf16_in, hipStream_t st) {
  if (bf16_in) return a.kp.d == 64 ? launch_t<bf16, 64>(a, st) : launch_t<bf16, 128>(a, st);
  return a.kp.d == 64 ? launch_t<float, 64>(a, st) : launch_t<float, 128>(a, st);
}

}  // namespace hga
