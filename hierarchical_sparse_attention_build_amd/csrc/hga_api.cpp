// C ABI of the HGA library: argument validation, workspace carving and launch
// sequencing.  Nothing here allocates device memory or synchronises; every
// launch goes to the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "hga.h"
#include "hga_kernels.hpp"

using namespace hga;

namespace {

thread_local std::string g_err;

hga_status fail(hga_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

hga_status ok() {
  g_err.clear();
  return HGA_OK;
}

hga_status hip_fail(hipError_t e, const char* what) {
  return fail(HGA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// ------------------------------------------------------------------ params
hga_status build_kparams(const hga_params* p, int64_t n_cap, KParams& kp) {
  if (!p) return fail(HGA_ERR_ARG, "params is null");
  if (p->batch < 1 || p->n_kv_heads < 1 || p->n_q_heads < 1)
    return fail(HGA_ERR_SHAPE, "batch, n_q_heads and n_kv_heads must be >= 1");
  if (p->n_q_heads % p->n_kv_heads != 0)
    return fail(HGA_ERR_SHAPE, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)", p->n_q_heads,
                p->n_kv_heads);
  const int gq = p->n_q_heads / p->n_kv_heads;
  if (gq != 1 && gq != 2 && gq != 4 && gq != 8 && gq != 16)
    return fail(HGA_ERR_UNSUPPORTED, "n_q_heads/n_kv_heads = %d: supported 1, 2, 4, 8, 16", gq);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(HGA_ERR_UNSUPPORTED, "head_dim %d: supported 64, 128", p->head_dim);
  if (p->chunk_size < 1 || p->chunk_size > 256)
    return fail(HGA_ERR_SHAPE, "chunk_size %d out of [1, 256]", p->chunk_size);
  if (p->group_size < 1 || p->chunk_size % p->group_size != 0)
    return fail(HGA_ERR_SHAPE, "group_size %d must divide chunk_size %d", p->group_size, p->chunk_size);
  if (p->chunk_size / p->group_size > 64)
    return fail(HGA_ERR_UNSUPPORTED, "chunk_size/group_size = %d > 64", p->chunk_size / p->group_size);
  if (p->n_sink < 0 || p->n_local < 0) return fail(HGA_ERR_ARG, "n_sink and n_local must be >= 0");
  if (p->top_k < 0 || p->top_k > 1024) return fail(HGA_ERR_ARG, "top_k %d out of [0, 1024]", p->top_k);
  if (p->top_g < 0 || p->top_g > 1024) return fail(HGA_ERR_ARG, "top_g %d out of [0, 1024]", p->top_g);
  if (!(p->rope_base > 1.0) || !std::isfinite(p->rope_base))
    return fail(HGA_ERR_ARG, "rope_base must be a finite number > 1");
  if (!(p->hf_threshold >= 0.0) || !std::isfinite(p->hf_threshold))
    return fail(HGA_ERR_ARG, "hf_threshold must be finite and >= 0");
  if ((p->qkv_dtype != HGA_BF16 && p->qkv_dtype != HGA_F32) ||
      (p->out_dtype != HGA_BF16 && p->out_dtype != HGA_F32))
    return fail(HGA_ERR_ARG, "unknown dtype");
  if (n_cap < 1 || n_cap > (int64_t(1) << 30))
    return fail(HGA_ERR_SHAPE, "n_cap %lld out of [1, 2^30]", static_cast<long long>(n_cap));
  if (n_cap % p->chunk_size != 0)
    return fail(HGA_ERR_SHAPE, "n_cap %lld must be a multiple of chunk_size %d",
                static_cast<long long>(n_cap), p->chunk_size);
  kp = KParams{};
  kp.B = p->batch;
  kp.Hq = p->n_q_heads;
  kp.Hkv = p->n_kv_heads;
  kp.d = p->head_dim;
  kp.C = p->chunk_size;
  kp.G = p->group_size;
  kp.m = p->chunk_size / p->group_size;
  kp.gq = gq;
  kp.n_sink = p->n_sink;
  kp.n_local = p->n_local;
  kp.top_k = p->top_k;
  kp.top_g = p->top_g;
  kp.n_cap = n_cap;
  kp.n_chunks_cap = static_cast<int32_t>(n_cap / p->chunk_size);
  auto ilog2_exact = [](int v) {
    int l = 0;
    while ((1 << l) < v) ++l;
    return (1 << l) == v ? l : -1;
  };
  kp.log2C = ilog2_exact(p->chunk_size);
  kp.log2G = ilog2_exact(p->group_size);
  kp.inv_sqrt_d = static_cast<float>(1.0 / std::sqrt(static_cast<double>(p->head_dim)));
  kp.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(p->head_dim)));
  kp.hf_mask = 0;
  for (int i = 0; i < p->head_dim / 2; ++i) {
    const double th = std::pow(p->rope_base, -2.0 * i / p->head_dim);
    kp.theta_d[i] = th;
    kp.theta_f[i] = static_cast<float>(th);
    if (th * p->chunk_size > p->hf_threshold) kp.hf_mask |= (uint64_t(1) << i);
  }
  return HGA_OK;
}

size_t elem_bytes(const hga_params* p) { return p->qkv_dtype == HGA_BF16 ? 2 : 4; }

template <typename P>
P* at_ws(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

// ------------------------------------------------------------------ workspace plans
struct RoutePlan {
  int n_units, slices, cps;
  size_t scores_off, cand_off, gscores_off, counters_off, split_off, bytes;
  bool split;  // the MFMA prefill routing runs (split summary tables present)
};

RoutePlan plan_route(const KParams& kp, int64_t nq, bool bf16_in, size_t base) {
  RoutePlan r{};
  r.n_units = nq == 1 ? 1 : static_cast<int>(nq / kp.C);
  r.cps = route_chunks_per_slice(kp, nq);
  const int64_t max_cand = std::max<int64_t>(0, kp.n_chunks_cap - 1 - kp.n_local - kp.n_sink);
  r.slices = static_cast<int>(std::max<int64_t>(1, cdiv(max_cand, r.cps)));
  const size_t units = static_cast<size_t>(kp.B) * kp.Hkv * r.n_units;
  size_t off = base;
  r.counters_off = off;
  off = align256(off + units * sizeof(uint32_t));
  r.scores_off = off;
  off = align256(off + units * kp.n_chunks_cap * sizeof(float));
  r.cand_off = off;
  off = align256(off + units * kp.n_chunks_cap * sizeof(int32_t));
  r.gscores_off = off;
  off = align256(off + units * static_cast<size_t>(kp.top_k) * kp.m * sizeof(float));
  r.split = route_prefill_mfma_supported(kp, bf16_in, nq);
  r.split_off = off;
  if (r.split) off = align256(off + route_prefill_split_bytes(kp));
  r.bytes = off - base;
  return r;
}

struct AttendPlan {
  int splits1, splits2, tps, parts_total;  // splits2 > 0 only for the two-part (offload) schedule
  size_t counters_off, partials_off, v16_off, bytes;
  bool v16;  // the pipelined prefill kernel runs (V16 region present)
};

AttendPlan plan_attend(const KParams& kp, int64_t nq, bool two_part, bool bf16_in, size_t base) {
  AttendPlan a{};
  const int64_t rows = static_cast<int64_t>(kp.B) * kp.Hkv * nq;
  const int max_blocks = static_cast<int>(cdiv(attend_max_slots(kp), kAttBlockRows));
  // enough workgroups to give every CU work, each with several 16-row blocks;
  // with more than 4 query heads per KV head the parts are larger and the
  // last workgroup's merge of them costs more, so fewer (8 heads, 128K, given
  // lists: 23 us at 256 workgroups, 25 us at 512, 30 us at 128)
  const int64_t target = kp.gq > 4 ? 2048 / kp.gq : 512;
  const int splits = static_cast<int>(
      std::min<int64_t>(std::min(max_blocks, kAttMaxParts / 2), std::max<int64_t>(1, cdiv(target, rows))));
  a.tps = static_cast<int>(cdiv(max_blocks, splits));
  if (two_part) {
    const int fb = static_cast<int>(cdiv(static_cast<int64_t>(kp.n_sink + kp.n_local + 1) * kp.C, kAttBlockRows));
    const int rb = static_cast<int>(std::max<int64_t>(1, cdiv(static_cast<int64_t>(kp.top_g) * kp.G, kAttBlockRows)));
    a.splits1 = static_cast<int>(cdiv(fb, a.tps));
    a.splits2 = static_cast<int>(cdiv(rb, a.tps));
    a.parts_total = a.splits1 + a.splits2;
  } else {
    a.splits1 = static_cast<int>(cdiv(max_blocks, a.tps));
    a.splits2 = 0;
    a.parts_total = a.splits1;
  }
  size_t off = base;
  a.counters_off = off;
  off = align256(off + static_cast<size_t>(rows) * sizeof(uint32_t));
  a.partials_off = off;
  if (a.parts_total > 1)
    off = align256(off + static_cast<size_t>(rows) * a.parts_total * kp.gq * (kp.d + 2) * sizeof(float));
  a.v16 = !two_part && prefill_pipe_supported(kp, bf16_in, nq);
  a.v16_off = off;
  if (a.v16) off = align256(off + prefill_pipe_v16_bytes(kp));
  a.bytes = off - base;
  return a;
}

// Decode step in one launch: per (b, kv head), R workgroups route and attend
// shares of the routed rows, F attend the forced window; the last merges.
#ifndef HGA_DECODE_ROUTING_WGS
#define HGA_DECODE_ROUTING_WGS 2
#endif

struct FusedPlan {
  bool use;
  int forced_blocks, units_per_xcd;
  size_t sync_off, partials_off, bytes;
};

FusedPlan plan_fused(const KParams& kp, size_t base) {
  FusedPlan r{};
  r.use = decode_fused_supported(kp);
  if (!r.use) return r;
  r.forced_blocks = static_cast<int>(cdiv(static_cast<int64_t>(kp.n_sink + kp.n_local + 1) * kp.C, kAttBlockRows));
  const int64_t units = static_cast<int64_t>(kp.B) * kp.Hkv;
  r.units_per_xcd = static_cast<int>(cdiv(units, kXcds));
  size_t off = base;
  r.sync_off = off;
  off = align256(off + static_cast<size_t>(units) * 4 * sizeof(uint32_t));
  r.partials_off = off;
  off = align256(off + static_cast<size_t>(units) * kDecMaxParts * kp.gq * (kp.d + 2) * sizeof(float));
  r.bytes = off - base;
  return r;
}

// Compute units of the current device (0 if it cannot be queried), cached.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0 && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
    cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Workgroups per unit of a decode launch.  Routing: two routing workgroups
// (each repeats the routing and takes half of the routed rows) and one forced
// one while every workgroup of the launch has a compute unit of its own; else
// one routing workgroup, which finishes last by far, and two forced ones
// (decode_32k, B = 8: 21.2 us with 2 + 1, 21.5 with 2 + 2, 21.6 with 3 + 1;
// with one routing workgroup 22.6 us with two forced, 23.1 with one).  Given
// lists (no routing): the forced rows outnumber each routing workgroup's
// share, so two forced workgroups, with two routing ones while they fit
// (12.3 us against 14.0 with one forced).  No routed rows at all (top_k or
// top_g = 0, streaming heads): one routing workgroup and two forced.  One
// routing workgroup with routing, but a grid of three per unit would share
// CUs: one forced workgroup when that makes it fit (decode_64k, 128 units:
// 44.7 us against 45.1).  With routing and CUs to spare after that, one
// warm-up workgroup per unit reads its candidate summaries into L2 alongside
// the routing scans (decode_32k, B = 8, 256 workgroups: 20.83 us against
// 21.52 without; 20.92 when it reads only the last three quarters, 21.19 the
// second half).
void fused_shape(const KParams& kp, const FusedPlan& fp, bool given, DecodeArgs& da) {
  const int64_t units = static_cast<int64_t>(kp.B) * kp.Hkv;
  const int want = std::max(1, std::min(HGA_DECODE_ROUTING_WGS, kDecMaxRouting));
  const bool routed = kp.top_k > 0 && kp.top_g > 0;
  const int forced_if_split = given ? 2 : 1;
  const bool split = routed && want > 1 && units * (want + forced_if_split) <= device_cus();
  da.routing_wgs = split ? want : 1;
  const int cus = device_cus();
  const bool fit_one_forced = routed && !given && units * 3 > cus && units * 2 <= cus;
  const int forced = split ? forced_if_split : (fit_one_forced ? 1 : 2);
  da.forced_wgs = std::max(1, std::min(std::min(forced, fp.forced_blocks), kDecMaxForced));
  da.forced_bpw = static_cast<int>(cdiv(fp.forced_blocks, da.forced_wgs));
  da.units_per_xcd = fp.units_per_xcd;
  da.warm_wgs = routed && !given && units * (da.routing_wgs + da.forced_wgs + 1) <= cus ? 1 : 0;
}

struct IdxPlan {
  size_t ci_off, gi_off, bytes;
};

IdxPlan plan_idx(const KParams& kp, int n_units, size_t base) {
  IdxPlan r{};
  const size_t units = static_cast<size_t>(kp.B) * kp.Hkv * n_units;
  size_t off = base;
  r.ci_off = off;
  off = align256(off + units * std::max(1, kp.top_k) * sizeof(int32_t));
  r.gi_off = off;
  off = align256(off + units * std::max(1, kp.top_g) * sizeof(int32_t));
  r.bytes = off - base;
  return r;
}

// Warm-tier list of a decode step: the slot of each routed entry.
struct WarmPlan {
  size_t slot_off, bytes;
};

WarmPlan plan_warm(const KParams& kp, size_t base) {
  WarmPlan r{};
  const size_t units = static_cast<size_t>(kp.B) * kp.Hkv;
  const size_t tg = static_cast<size_t>(std::max(1, kp.top_g));
  size_t off = base;
  r.slot_off = off;
  off = align256(off + units * tg * sizeof(int32_t));
  r.bytes = off - base;
  return r;
}

struct FullPlan {
  RoutePlan route;
  AttendPlan attend;
  FusedPlan fused;
  WarmPlan warm;
  IdxPlan idx;
  size_t canon_off;  // canonical copy of a caller-given group list (attend, backward)
  // matrix-core backward: dO split in two bf16 parts, the visibility bitmap
  // and per-key-chunk counts
  bool bwd_mfma;
  size_t doh_off, dol_off, vis_off, counts_off;
  size_t bytes;
};

// Units of a call: one per (b, kv head) in decode, one per query chunk in prefill.
int call_units(const KParams& kp, int64_t nq) { return nq == 1 ? 1 : static_cast<int>(nq / kp.C); }

FullPlan plan(const KParams& kp, int op, int64_t nq, bool bf16_in) {
  FullPlan f{};
  size_t off = 0;
  const bool needs_route = op == HGA_OP_ROUTE || op == HGA_OP_PREFILL || op == HGA_OP_DECODE ||
                           op == HGA_OP_DECODE_OFFLOAD;
  const bool needs_attend = op == HGA_OP_ATTEND || op == HGA_OP_PREFILL || op == HGA_OP_DECODE ||
                            op == HGA_OP_DECODE_OFFLOAD;
  const bool needs_idx = op == HGA_OP_PREFILL || op == HGA_OP_DECODE || op == HGA_OP_DECODE_OFFLOAD;
  // The caller zero-fills the whole workspace once, before its first use; every
  // counter in it is back at zero when a call's kernels end.
  if (needs_route) {
    f.route = plan_route(kp, nq, bf16_in, off);
    off += f.route.bytes;
  }
  if (needs_attend) {
    f.attend = plan_attend(kp, nq, op == HGA_OP_DECODE_OFFLOAD, bf16_in, off);
    off += f.attend.bytes;
  }
  if (op == HGA_OP_DECODE || (op == HGA_OP_ATTEND && nq == 1)) {
    f.fused = plan_fused(kp, off);
    off += f.fused.bytes;
  }
  if (op == HGA_OP_DECODE_OFFLOAD) {
    f.warm = plan_warm(kp, off);
    off += f.warm.bytes;
  }
  if (needs_idx) {
    f.idx = plan_idx(kp, f.route.n_units, off);
    off += f.idx.bytes;
  }
  if (op == HGA_OP_PREFILL_BACKWARD) {
    // per query row: the base-2 log-sum-exp and D of the softmax
    off = align256(off + static_cast<size_t>(kp.B) * kp.Hq * nq * 2 * sizeof(float));
  }
  if (op == HGA_OP_ATTEND || op == HGA_OP_PREFILL_BACKWARD) {
    f.canon_off = off;
    off = align256(off + static_cast<size_t>(kp.B) * kp.Hkv * call_units(kp, nq) *
                             std::max(1, kp.top_g) * sizeof(int32_t));
  }
  if (op == HGA_OP_PREFILL_BACKWARD && backward_mfma_supported(kp, bf16_in)) {
    f.bwd_mfma = true;
    const size_t q_elems = static_cast<size_t>(kp.B) * kp.Hq * nq * kp.d;
    const size_t units = static_cast<size_t>(kp.B) * kp.Hkv * call_units(kp, nq);
    f.doh_off = off;
    off = align256(off + q_elems * sizeof(uint16_t));
    f.dol_off = off;
    off = align256(off + q_elems * sizeof(uint16_t));
    f.vis_off = off;
    off = align256(off + units * backward_vis_words(call_units(kp, nq)) * sizeof(uint32_t));
    f.counts_off = off;
    off = align256(off + units * sizeof(int32_t));
  }
  f.bytes = off;
  return f;
}

// Caller-given group lists in canonical form (repeats and entries that add no
// visible token replaced by -1), written into the workspace; returns them.
hga_status canon_lists(const KParams& kp, const FullPlan& f, void* ws, const int32_t* gi, int64_t nq,
                       const int32_t* q_pos, int32_t bias, hipStream_t st, const int32_t** out) {
  *out = gi;
  if (kp.top_g <= 0) return HGA_OK;
  CanonArgs c{};
  c.kp = kp;
  c.in = gi;
  c.out = at_ws<int32_t>(ws, f.canon_off);
  c.q_pos = q_pos;
  c.pos_bias = bias;
  c.nq = nq;
  c.n_units = call_units(kp, nq);
  const hipError_t e = launch_canon_groups(c, st);
  if (e != hipSuccess) return fail(HGA_ERR_HIP, "canonical group lists: %s", hipGetErrorString(e));
  *out = c.out;
  return HGA_OK;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

hga_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return HGA_OK;
  if (!ws) return fail(HGA_ERR_WORKSPACE, "workspace is null (need %zu bytes)", need);
  if (!aligned16(ws)) return fail(HGA_ERR_ALIGN, "workspace not 16-byte aligned");
  if (ws_bytes < need) return fail(HGA_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", ws_bytes, need);
  return HGA_OK;
}

#define HGA_CHECK_PTR(ptr)                                                         \
  do {                                                                             \
    if (!(ptr)) return fail(HGA_ERR_ARG, "%s is null", #ptr);                      \
    if (!aligned16(ptr)) return fail(HGA_ERR_ALIGN, "%s not 16-byte aligned", #ptr); \
  } while (0)

#define HGA_TRY_HIP(expr, what)              \
  do {                                       \
    hipError_t e_ = (expr);                  \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

RouteArgs route_args(const KParams& kp, const FullPlan& f, void* ws, const void* Q, int64_t nq,
                     const int32_t* q_pos, int32_t bias, const float* cs, const float* gs,
                     int32_t* ci, int32_t* gi, float* scores_out) {
  RouteArgs a{};
  a.kp = kp;
  a.Q = Q;
  a.nq = nq;
  a.q_pos = q_pos;
  a.pos_bias = bias;
  a.chunk_sum = cs;
  a.group_sum = gs;
  a.n_units = f.route.n_units;
  a.slices = f.route.slices;
  a.chunks_per_slice = f.route.cps;
  a.scores = at<float>(ws, f.route.scores_off);
  a.cand_ids = at<int32_t>(ws, f.route.cand_off);
  a.gscores = at<float>(ws, f.route.gscores_off);
  a.counters = at<uint32_t>(ws, f.route.counters_off);
  a.chunk_idx = ci;
  a.group_idx = gi;
  a.scores_out = scores_out;
  a.split = f.route.split ? at<uint16_t>(ws, f.route.split_off) : nullptr;
  a.build_summary = 0;
  return a;
}

AttendArgs attend_args(const KParams& kp, const FullPlan& f, void* ws, const void* Q, int64_t nq,
                       const int32_t* q_pos, int32_t bias, const void* K, const void* V,
                       const int32_t* gi, int n_units, void* O, float* lse, bool out_bf16) {
  AttendArgs a{};
  a.kp = kp;
  a.Q = Q;
  a.nq = nq;
  a.q_pos = q_pos;
  a.pos_bias = bias;
  a.K = K;
  a.V = V;
  a.kv.base = K;
  a.kv.bh_rows = kp.n_cap;
  a.kv.ring = 0;
  a.group_idx = gi;
  a.n_units = n_units;
  a.O = O;
  a.lse = lse;
  a.out_bf16 = out_bf16 ? 1 : 0;
  a.splits = f.attend.splits1;
  a.tiles_per_split = f.attend.tps;
  a.part = 0;
  a.part_offset = 0;
  a.parts_total = f.attend.parts_total;
  a.partials = at<float>(ws, f.attend.partials_off);
  a.counters = at<uint32_t>(ws, f.attend.counters_off);
  a.V16 = f.attend.v16 ? at<void>(ws, f.attend.v16_off) : nullptr;
  return a;
}

// One decode step in one launch (the fused kernel), with the unit counters
// `sync` (zero before the launch, zero again after it) and the partial results.
hipError_t launch_fused_decode(const hga_params* p, const KParams& kp, const FusedPlan& fp, const void* Q,
                               const void* K, const void* V, const int32_t* seq_len, float* chunk_sum,
                               float* group_sum, void* O, int32_t* ci, int32_t* gi, uint32_t* sync, float* partials,
                               hipStream_t st) {
  DecodeArgs da{};
  da.kp = kp;
  da.Q = Q;
  da.seq_len = seq_len;
  da.K = K;
  da.V = V;
  da.chunk_sum = chunk_sum;
  da.group_sum = group_sum;
  da.chunk_sum_w = chunk_sum;
  da.group_sum_w = group_sum;
  da.build_summary = 1;
  da.chunk_idx = ci;
  da.group_idx = gi;
  da.O = O;
  da.out_bf16 = p->out_dtype == HGA_BF16 ? 1 : 0;
  fused_shape(kp, fp, false, da);
  da.partials = partials;
  da.sync = sync;
  da.pos_offset = -1;
  return launch_decode_step(da, p->qkv_dtype == HGA_BF16, st);
}

hga_status check_nq(const KParams& kp, int64_t nq) {
  if (nq < 1) return fail(HGA_ERR_SHAPE, "nq must be >= 1");
  if (nq > 1 && nq % kp.C != 0) return fail(HGA_ERR_SHAPE, "prefill nq %lld must be a multiple of C", (long long)nq);
  if (nq > kp.n_cap) return fail(HGA_ERR_SHAPE, "nq exceeds n_cap");
  if (nq > 1 && nq / kp.C > 65535) return fail(HGA_ERR_UNSUPPORTED, "too many query chunks");
  return HGA_OK;
}

// The split-K attention kernel (shapes the MFMA prefill kernels do not take)
// carries the query row in grid.y.
hga_status check_splitk_rows(int64_t nq) {
  if (nq > 65535)
    return fail(HGA_ERR_UNSUPPORTED, "nq %lld > 65535 rows per call for this shape (split-K attention)",
                static_cast<long long>(nq));
  return HGA_OK;
}

}  // namespace

// ------------------------------------------------------------------ no-allocation decode
// Scratch of hga_decode_static: one copy per device, kept until the process
// ends.  Layout: the arrival counters of up to kStaticMaxUnits units at a
// fixed offset (0), so that calls of different shapes always find them at
// zero; then the partial results and, when the caller passes no index lists,
// the lists.
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
constexpr int kStaticMaxUnits = 1024;
constexpr size_t kStaticSyncBytes = size_t(kStaticMaxUnits) * 4 * sizeof(uint32_t);
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

__global__ void zero_words_kernel(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

namespace {

constexpr int kStaticMaxDevices = 64;
std::mutex g_static_mu;
void* g_static_ptr[kStaticMaxDevices] = {};

// The device address of this device's `scratch` (looked up once per device,
// with the device current); on the first call its counters are cleared on
// `st` by a fill kernel, ahead of the work the call enqueues.
hga_status static_scratch(hipStream_t st, unsigned char** out) {
  int dev = 0;
  HGA_TRY_HIP(hipGetDevice(&dev), "get device");
  if (dev < 0 || dev >= kStaticMaxDevices) return fail(HGA_ERR_UNSUPPORTED, "device index %d >= %d", dev, kStaticMaxDevices);
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (!g_static_ptr[dev]) {
    void* ptr = nullptr;
    HGA_TRY_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "scratch address");
    if (!ptr) return fail(HGA_ERR_HIP, "scratch address is null");
    constexpr int words = static_cast<int>(kStaticSyncBytes / sizeof(uint32_t));
    zero_words_kernel<<<(words + 255) / 256, 256, 0, st>>>(static_cast<uint32_t*>(ptr), words);
    HGA_TRY_HIP(hipGetLastError(), "scratch clear");
    g_static_ptr[dev] = ptr;
  }
  *out = static_cast<unsigned char*>(g_static_ptr[dev]);
  return HGA_OK;
}

}  // namespace

// =================================================================== C ABI
extern "C" {

const char* hga_last_error(void) { return g_err.c_str(); }

const char* hga_version(void) { return "hga-mi355x 0.1 (gfx950)"; }

size_t hga_workspace_size(const hga_params* p, int32_t op, int64_t nq, int64_t n_cap) {
  KParams kp;
  if (build_kparams(p, n_cap, kp) != HGA_OK) return 0;
  if (op < HGA_OP_ROUTE || op > HGA_OP_PREFILL_BACKWARD) {
    fail(HGA_ERR_ARG, "unknown op %d", op);
    return 0;
  }
  if (op == HGA_OP_DECODE || op == HGA_OP_DECODE_OFFLOAD) nq = 1;
  if (check_nq(kp, nq) != HGA_OK) return 0;
  ok();
  return plan(kp, op, nq, p->qkv_dtype == HGA_BF16).bytes;
}

hga_status hga_build_summaries(const hga_params* p, const void* K, int64_t n_cap, int32_t chunk_begin,
                               int32_t chunk_end, int32_t k_is_rotated, void* K_rot_out,
                               float* chunk_sum, float* group_sum, void* stream) {
  KParams kp;
  hga_status s = build_kparams(p, n_cap, kp);
  if (s != HGA_OK) return s;
  HGA_CHECK_PTR(K);
  HGA_CHECK_PTR(chunk_sum);
  HGA_CHECK_PTR(group_sum);
  if (K_rot_out && !aligned16(K_rot_out)) return fail(HGA_ERR_ALIGN, "K_rot_out not 16-byte aligned");
  if (chunk_begin < 0 || chunk_end < chunk_begin || chunk_end > kp.n_chunks_cap)
    return fail(HGA_ERR_SHAPE, "chunk range [%d, %d) outside [0, %d]", chunk_begin, chunk_end, kp.n_chunks_cap);
  if (k_is_rotated && K_rot_out) return fail(HGA_ERR_ARG, "K_rot_out needs k_is_rotated = 0");
  if (static_cast<int64_t>(kp.B) * kp.Hkv > 65535) return fail(HGA_ERR_UNSUPPORTED, "B*Hkv > 65535");
  SummariesArgs a{};
  a.kp = kp;
  a.K = K;
  a.Krot = K_rot_out;
  a.chunk_sum = chunk_sum;
  a.group_sum = group_sum;
  a.chunk_begin = chunk_begin;
  a.chunk_end = chunk_end;
  a.rotated = k_is_rotated ? 1 : 0;
  HGA_TRY_HIP(launch_summaries(a, p->qkv_dtype == HGA_BF16, static_cast<hipStream_t>(stream)), "summaries");
  return ok();
}

hga_status hga_route(const hga_params* p, const void* Q, int64_t nq, const int32_t* q_pos,
                     const float* chunk_sum, const float* group_sum, int64_t n_cap, int32_t* chunk_idx,
                     int32_t* group_idx, float* scores_out, void* ws, size_t ws_bytes, void* stream) {
  KParams kp;
  hga_status s = build_kparams(p, n_cap, kp);
  if (s != HGA_OK) return s;
  if ((s = check_nq(kp, nq)) != HGA_OK) return s;
  HGA_CHECK_PTR(Q);
  HGA_CHECK_PTR(chunk_sum);
  HGA_CHECK_PTR(group_sum);
  HGA_CHECK_PTR(chunk_idx);
  HGA_CHECK_PTR(group_idx);
  if (!q_pos) return fail(HGA_ERR_ARG, "q_pos is null");
  if (scores_out && nq != 1) return fail(HGA_ERR_ARG, "scores_out is for decode (nq == 1) only");
  FullPlan f = plan(kp, HGA_OP_ROUTE, nq, p->qkv_dtype == HGA_BF16);
  if ((s = check_ws(ws, ws_bytes, f.bytes)) != HGA_OK) return s;
  RouteArgs a = route_args(kp, f, ws, Q, nq, q_pos, 0, chunk_sum, group_sum, chunk_idx, group_idx, scores_out);
  const bool bf = p->qkv_dtype == HGA_BF16;
  if (route_prefill_mfma_supported(kp, bf, nq))
    HGA_TRY_HIP(launch_route_prefill_mfma(a, static_cast<hipStream_t>(stream)), "route (mfma)");
  else
    HGA_TRY_HIP(launch_route_scan(a, bf, bf, static_cast<hipStream_t>(stream)), "route");
  return ok();
}

hga_status hga_attend(const hga_params* p, const void* Q, int64_t nq, const int32_t* q_pos, const void* K,
                      const void* V, int64_t n_cap, const int32_t* group_idx, void* O, float* lse_out,
                      void* ws, size_t ws_bytes, void* stream) {
  KParams kp;
  hga_status s = build_kparams(p, n_cap, kp);
  if (s != HGA_OK) return s;
  if ((s = check_nq(kp, nq)) != HGA_OK) return s;
  HGA_CHECK_PTR(Q);
  HGA_CHECK_PTR(K);
  HGA_CHECK_PTR(V);
  HGA_CHECK_PTR(O);
  if (kp.top_g > 0 && !group_idx) return fail(HGA_ERR_ARG, "group_idx is null");
  if (!q_pos) return fail(HGA_ERR_ARG, "q_pos is null");
  if (lse_out && !aligned16(lse_out)) return fail(HGA_ERR_ALIGN, "lse_out not 16-byte aligned");
  FullPlan f = plan(kp, HGA_OP_ATTEND, nq, p->qkv_dtype == HGA_BF16);
  if ((s = check_ws(ws, ws_bytes, f.bytes)) != HGA_OK) return s;
  const int n_units = call_units(kp, nq);
  const bool bf = p->qkv_dtype == HGA_BF16;
  if (nq == 1 && f.fused.use && !lse_out && kp.top_g > 0) {
    // one query per sequence: the decode step's kernel with the lists given
    // (route once, attend many: e.g. one layer's routing reused by the next);
    // it puts each list in canonical form itself
    const FusedPlan& fp = f.fused;
    DecodeArgs da{};
    da.kp = kp;
    da.Q = Q;
    da.seq_len = q_pos;
    da.pos_offset = 0;
    da.K = K;
    da.V = V;
    da.build_summary = 0;
    da.routes_in = group_idx;
    da.O = O;
    da.out_bf16 = p->out_dtype == HGA_BF16 ? 1 : 0;
    fused_shape(kp, fp, true, da);
    da.partials = at<float>(ws, fp.partials_off);
    da.sync = at<uint32_t>(ws, fp.sync_off);
    HGA_TRY_HIP(launch_decode_step(da, bf, static_cast<hipStream_t>(stream)), "attend (decode step)");
    return ok();
  }
  const bool splitk = !f.attend.v16 && !prefill_mfma_supported(kp, bf, nq);
  if (splitk && (s = check_splitk_rows(nq)) != HGA_OK) return s;
  const int32_t* gi = group_idx;
  if ((s = canon_lists(kp, f, ws, group_idx, nq, q_pos, 0, static_cast<hipStream_t>(stream), &gi)) != HGA_OK)
    return s;
  AttendArgs a = attend_args(kp, f, ws, Q, nq, q_pos, 0, K, V, gi, n_units, O, lse_out,
                             p->out_dtype == HGA_BF16);
  if (a.V16) {
    HGA_TRY_HIP(launch_attend_prefill_pipe(a, static_cast<hipStream_t>(stream)), "attend (mfma, pipelined)");
  } else if (prefill_mfma_supported(kp, bf, nq)) {
    HGA_TRY_HIP(launch_attend_prefill_mfma(a, static_cast<hipStream_t>(stream)), "attend (mfma)");
  } else {
    HGA_TRY_HIP(launch_attend_splitk(a, bf, static_cast<hipStream_t>(stream)), "attend");
  }
  return ok();
}

hga_status hga_prefill(const hga_params* p, const void* Q, const void* K, const void* V, int64_t n,
                       float* chunk_sum, float* group_sum, void* O, int32_t* chunk_idx, int32_t* group_idx,
                       void* ws, size_t ws_bytes, void* stream) {
  KParams kp;
  hga_status s = build_kparams(p, n, kp);
  if (s != HGA_OK) return s;
  if ((s = check_nq(kp, n)) != HGA_OK) return s;
  if (n < kp.C) return fail(HGA_ERR_SHAPE, "prefill needs n >= C");
  HGA_CHECK_PTR(Q);
  HGA_CHECK_PTR(K);
  HGA_CHECK_PTR(V);
  HGA_CHECK_PTR(O);
  HGA_CHECK_PTR(chunk_sum);
  HGA_CHECK_PTR(group_sum);
  if (chunk_idx && !aligned16(chunk_idx)) return fail(HGA_ERR_ALIGN, "chunk_idx not 16-byte aligned");
  if (group_idx && !aligned16(group_idx)) return fail(HGA_ERR_ALIGN, "group_idx not 16-byte aligned");
  FullPlan f = plan(kp, HGA_OP_PREFILL, n, p->qkv_dtype == HGA_BF16);
  if ((s = check_ws(ws, ws_bytes, f.bytes)) != HGA_OK) return s;
  if (!f.attend.v16 && !prefill_mfma_supported(kp, p->qkv_dtype == HGA_BF16, n) && (s = check_splitk_rows(n)) != HGA_OK)
    return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf = p->qkv_dtype == HGA_BF16;
  int32_t* ci = chunk_idx ? chunk_idx : at<int32_t>(ws, f.idx.ci_off);
  int32_t* gi = group_idx ? group_idx : at<int32_t>(ws, f.idx.gi_off);

  SummariesArgs sa{};
  sa.kp = kp;
  sa.K = K;
  sa.chunk_sum = chunk_sum;
  sa.group_sum = group_sum;
  sa.chunk_begin = 0;
  sa.chunk_end = kp.n_chunks_cap;
  sa.rotated = 1;
  HGA_TRY_HIP(launch_summaries(sa, bf, st), "summaries");
  RouteArgs ra = route_args(kp, f, ws, Q, n, nullptr, 0, chunk_sum, group_sum, ci, gi, nullptr);
  if (route_prefill_mfma_supported(kp, bf, n))
    HGA_TRY_HIP(launch_route_prefill_mfma(ra, st), "route (mfma)");
  else
    HGA_TRY_HIP(launch_route_scan(ra, bf, bf, st), "route");
  AttendArgs aa = attend_args(kp, f, ws, Q, n, nullptr, 0, K, V, gi, f.route.n_units, O, nullptr,
                              p->out_dtype == HGA_BF16);
  if (aa.V16) {
    HGA_TRY_HIP(launch_attend_prefill_pipe(aa, st), "attend (mfma, pipelined)");
  } else if (prefill_mfma_supported(kp, bf, n)) {
    HGA_TRY_HIP(launch_attend_prefill_mfma(aa, st), "attend (mfma)");
  } else {
    HGA_TRY_HIP(launch_attend_splitk(aa, bf, st), "attend");
  }
  return ok();
}

hga_status hga_prefill_backward(const hga_params* p, const void* Q, const void* K, const void* V, int64_t n,
                                const int32_t* group_idx, const float* dO, float* dQ, float* dK, float* dV,
                                void* ws, size_t ws_bytes, void* stream) {
  KParams kp;
  hga_status s = build_kparams(p, n, kp);
  if (s != HGA_OK) return s;
  if ((s = check_nq(kp, n)) != HGA_OK) return s;
  if (n < kp.C) return fail(HGA_ERR_SHAPE, "backward needs n >= C");
  if (!backward_supported(kp)) return fail(HGA_ERR_UNSUPPORTED, "backward needs C = 64 and d in {64, 128}");
  HGA_CHECK_PTR(Q);
  HGA_CHECK_PTR(K);
  HGA_CHECK_PTR(V);
  HGA_CHECK_PTR(dO);
  HGA_CHECK_PTR(dQ);
  HGA_CHECK_PTR(dK);
  HGA_CHECK_PTR(dV);
  if (kp.top_g > 0 && !group_idx) return fail(HGA_ERR_ARG, "group_idx is null");
  FullPlan f = plan(kp, HGA_OP_PREFILL_BACKWARD, n, p->qkv_dtype == HGA_BF16);
  if ((s = check_ws(ws, ws_bytes, f.bytes)) != HGA_OK) return s;
  const int32_t* gi = group_idx;
  if ((s = canon_lists(kp, f, ws, group_idx, n, nullptr, 0, static_cast<hipStream_t>(stream), &gi)) != HGA_OK)
    return s;
  BackwardArgs a{};
  a.kp = kp;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.group_idx = gi;
  a.dO = dO;
  a.dQ = dQ;
  a.dK = dK;
  a.dV = dV;
  a.stats = static_cast<float*>(ws);
  a.n = n;
  a.n_units = static_cast<int32_t>(n / kp.C);
  a.unit_slice = 64;
  if (f.bwd_mfma) {
    a.dOh = at<uint16_t>(ws, f.doh_off);
    a.dOl = at<uint16_t>(ws, f.dol_off);
    a.vis = at<uint32_t>(ws, f.vis_off);
    a.vis_words = backward_vis_words(a.n_units);
    a.counts = at<int32_t>(ws, f.counts_off);
    HGA_TRY_HIP(launch_backward_mfma(a, static_cast<hipStream_t>(stream)), "backward (mfma)");
    return ok();
  }
  HGA_TRY_HIP(launch_backward(a, p->qkv_dtype == HGA_BF16, static_cast<hipStream_t>(stream)), "backward");
  return ok();
}

hga_status hga_decode(const hga_params* p, const void* Q, const void* K, const void* V, int64_t n_cap,
                      const int32_t* seq_len, float* chunk_sum, float* group_sum, void* O, int32_t* chunk_idx,
                      int32_t* group_idx, void* ws, size_t ws_bytes, void* stream) {
  KParams kp;
  hga_status s = build_kparams(p, n_cap, kp);
  if (s != HGA_OK) return s;
  HGA_CHECK_PTR(Q);
  HGA_CHECK_PTR(K);
  HGA_CHECK_PTR(V);
  HGA_CHECK_PTR(O);
  HGA_CHECK_PTR(chunk_sum);
  HGA_CHECK_PTR(group_sum);
  if (!seq_len) return fail(HGA_ERR_ARG, "seq_len is null");
  if (chunk_idx && !aligned16(chunk_idx)) return fail(HGA_ERR_ALIGN, "chunk_idx not 16-byte aligned");
  if (group_idx && !aligned16(group_idx)) return fail(HGA_ERR_ALIGN, "group_idx not 16-byte aligned");
  FullPlan f = plan(kp, HGA_OP_DECODE, 1, p->qkv_dtype == HGA_BF16);
  if ((s = check_ws(ws, ws_bytes, f.bytes)) != HGA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool bf = p->qkv_dtype == HGA_BF16;
  int32_t* ci = chunk_idx ? chunk_idx : at<int32_t>(ws, f.idx.ci_off);
  int32_t* gi = group_idx ? group_idx : at<int32_t>(ws, f.idx.gi_off);
  if (f.fused.use) {
    HGA_TRY_HIP(launch_fused_decode(p, kp, f.fused, Q, K, V, seq_len, chunk_sum, group_sum, O, ci, gi,
                                    at<uint32_t>(ws, f.fused.sync_off), at<float>(ws, f.fused.partials_off), st),
                "decode step");
    return ok();
  }
  RouteArgs ra = route_args(kp, f, ws, Q, 1, seq_len, -1, chunk_sum, group_sum, ci, gi, nullptr);
  ra.build_summary = 1;
  ra.ksrc.base = K;
  ra.ksrc.bh_rows = kp.n_cap;
  ra.ksrc.ring = 0;
  ra.chunk_sum_w = chunk_sum;
  ra.group_sum_w = group_sum;
  HGA_TRY_HIP(launch_route_scan(ra, bf, bf, st), "route");
  AttendArgs aa = attend_args(kp, f, ws, Q, 1, seq_len, -1, K, V, gi, 1, O, nullptr, p->out_dtype == HGA_BF16);
  HGA_TRY_HIP(launch_attend_splitk(aa, bf, st), "attend");
  return ok();
}

hga_status hga_decode_static(const hga_params* p, const void* Q, const void* K, const void* V, int64_t n_cap,
                             const int32_t* seq_len, float* chunk_sum, float* group_sum, void* O,
                             int32_t* chunk_idx, int32_t* group_idx, void* stream) {
  KParams kp;
  hga_status s = build_kparams(p, n_cap, kp);
  if (s != HGA_OK) return s;
  HGA_CHECK_PTR(Q);
  HGA_CHECK_PTR(K);
  HGA_CHECK_PTR(V);
  HGA_CHECK_PTR(O);
  HGA_CHECK_PTR(chunk_sum);
  HGA_CHECK_PTR(group_sum);
  if (!seq_len) return fail(HGA_ERR_ARG, "seq_len is null");
  if (chunk_idx && !aligned16(chunk_idx)) return fail(HGA_ERR_ALIGN, "chunk_idx not 16-byte aligned");
  if (group_idx && !aligned16(group_idx)) return fail(HGA_ERR_ALIGN, "group_idx not 16-byte aligned");
  const FusedPlan fp = plan_fused(kp, 0);
  if (!fp.use)
    return fail(HGA_ERR_UNSUPPORTED, "hga_decode_static: shape outside the one-launch decode kernel "
                                     "(Hq/Hkv in {1, 2, 4}, d in {64, 128}, C and G powers of two, at most "
                                     "4096 candidate chunks, top_k * C/G <= 4096, top_g <= 256)");
  const int64_t units = static_cast<int64_t>(kp.B) * kp.Hkv;
  if (units > kStaticMaxUnits)
    return fail(HGA_ERR_SHAPE, "hga_decode_static: B*Hkv = %lld > %d", static_cast<long long>(units), kStaticMaxUnits);
  // layout: [sync counters | partial results | chunk list | group list]
  const size_t partials_off = kStaticSyncBytes;
  size_t off = align256(partials_off + static_cast<size_t>(units) * kDecMaxParts * kp.gq * (kp.d + 2) * sizeof(float));
  const size_t ci_off = off;
  if (!chunk_idx) off = align256(off + static_cast<size_t>(units) * std::max(1, kp.top_k) * sizeof(int32_t));
  const size_t gi_off = off;
  if (!group_idx) off = align256(off + static_cast<size_t>(units) * std::max(1, kp.top_g) * sizeof(int32_t));
  if (off > kStaticScratchBytes)
    return fail(HGA_ERR_SHAPE, "hga_decode_static: needs %zu bytes of scratch, limit %zu", off, kStaticScratchBytes);
  hipStream_t st = static_cast<hipStream_t>(stream);
  unsigned char* base = nullptr;
  if ((s = static_scratch(st, &base)) != HGA_OK) return s;
  int32_t* ci = chunk_idx ? chunk_idx : reinterpret_cast<int32_t*>(base + ci_off);
  int32_t* gi = group_idx ? group_idx : reinterpret_cast<int32_t*>(base + gi_off);
  HGA_TRY_HIP(launch_fused_decode(p, kp, fp, Q, K, V, seq_len, chunk_sum, group_sum, O, ci, gi,
                                  reinterpret_cast<uint32_t*>(base), reinterpret_cast<float*>(base + partials_off),
                                  st),
              "decode step (static scratch)");
  return ok();
}

namespace {

// Cold-tier decode step with either a staging buffer (every routed group copied
// each step) or the warm tier (only the missing groups copied).
hga_status decode_offload_impl(const hga_params* p, const void* Q, const void* K_host, const void* V_host,
                               const void* K_hot, const void* V_hot, int64_t n_cap, const int32_t* seq_len,
                               float* chunk_sum, float* group_sum, void* O, int32_t* chunk_idx,
                               int32_t* group_idx, void* staging, size_t staging_bytes, const hga_warm* warm,
                               void* ws, size_t ws_bytes, void* stream, void* copy_stream) {
  KParams kp;
  hga_status s = build_kparams(p, n_cap, kp);
  if (s != HGA_OK) return s;
  HGA_CHECK_PTR(Q);
  HGA_CHECK_PTR(K_host);
  HGA_CHECK_PTR(V_host);
  HGA_CHECK_PTR(K_hot);
  HGA_CHECK_PTR(V_hot);
  HGA_CHECK_PTR(O);
  HGA_CHECK_PTR(chunk_sum);
  HGA_CHECK_PTR(group_sum);
  if (!seq_len) return fail(HGA_ERR_ARG, "seq_len is null");
  if (chunk_idx && !aligned16(chunk_idx)) return fail(HGA_ERR_ALIGN, "chunk_idx not 16-byte aligned");
  if (group_idx && !aligned16(group_idx)) return fail(HGA_ERR_ALIGN, "group_idx not 16-byte aligned");
  void* Kst;
  void* Vst;
  if (warm) {
    HGA_CHECK_PTR(warm->K);
    HGA_CHECK_PTR(warm->V);
    HGA_CHECK_PTR(warm->tags);
    HGA_CHECK_PTR(warm->stamps);
    HGA_CHECK_PTR(warm->clock);
    if (warm->slots < std::max(1, kp.top_g) || warm->slots > kWarmMaxSlots)
      return fail(HGA_ERR_ARG, "warm slots %d out of [max(1, top_g), %d]", warm->slots, kWarmMaxSlots);
    if (kp.top_g > kWarmMaxList)
      return fail(HGA_ERR_ARG, "top_g %d above %d with the warm tier", kp.top_g, kWarmMaxList);
    if (!aligned16(warm->K) || !aligned16(warm->V)) return fail(HGA_ERR_ALIGN, "warm K/V not 16-byte aligned");
    Kst = warm->K;
    Vst = warm->V;
  } else {
    HGA_CHECK_PTR(staging);
    const size_t half =
        static_cast<size_t>(kp.B) * kp.Hkv * std::max(1, kp.top_g) * kp.G * kp.d * elem_bytes(p);
    if (staging_bytes < 2 * half)
      return fail(HGA_ERR_WORKSPACE, "staging has %zu bytes, need %zu", staging_bytes, 2 * half);
    Kst = staging;
    Vst = static_cast<char*>(staging) + half;
  }
  FullPlan f = plan(kp, HGA_OP_DECODE_OFFLOAD, 1, p->qkv_dtype == HGA_BF16);
  if ((s = check_ws(ws, ws_bytes, f.bytes)) != HGA_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipStream_t cst = static_cast<hipStream_t>(copy_stream);
  const bool bf = p->qkv_dtype == HGA_BF16;
  int32_t* ci = chunk_idx ? chunk_idx : at<int32_t>(ws, f.idx.ci_off);
  int32_t* gi = group_idx ? group_idx : at<int32_t>(ws, f.idx.gi_off);

  const int64_t hot_rows = static_cast<int64_t>(kp.n_sink + kp.n_local + 1) * kp.C;
  RouteArgs ra = route_args(kp, f, ws, Q, 1, seq_len, -1, chunk_sum, group_sum, ci, gi, nullptr);
  ra.build_summary = 1;
  ra.ksrc.base = K_hot;
  ra.ksrc.bh_rows = hot_rows;
  ra.ksrc.ring = 1;
  ra.chunk_sum_w = chunk_sum;
  ra.group_sum_w = group_sum;
  int32_t* slot_of = warm ? at<int32_t>(ws, f.warm.slot_off) : nullptr;
  if (warm) {
    // the routing launch's last workgroup of each unit runs the unit's LRU lookup
    ra.warm.tags = warm->tags;
    ra.warm.stamps = warm->stamps;
    ra.warm.clock = warm->clock;
    ra.warm.hits = warm->hits;
    ra.warm.misses = warm->misses;
    ra.warm.slot_of = slot_of;
    ra.warm.slots = warm->slots;
  }
  HGA_TRY_HIP(launch_route_scan(ra, bf, bf, st), "route");
  AttendArgs aa = attend_args(kp, f, ws, Q, 1, seq_len, -1, K_hot, V_hot, gi, 1, O, nullptr,
                              p->out_dtype == HGA_BF16);
  aa.kv.base = K_hot;
  aa.kv.bh_rows = hot_rows;
  aa.kv.ring = 1;
  aa.K_stage = Kst;
  aa.V_stage = Vst;
  if (warm) {
    // The warm tier's copies are the few groups missing from the cache: the
    // attention reads their rows from host memory and writes them into the
    // slots the lookup chose, so the copy overlaps the attention of the
    // cached groups and needs no second stream.  Both parts of the attention
    // go in one grid with the block ranges and merge order of the two
    // launches below.
    aa.stage_slot = slot_of;
    aa.stage_slots = warm->slots;
    aa.K_host = K_host;
    aa.V_host = V_host;
    aa.part = 3;
    aa.part1_splits = f.attend.splits1;
    aa.splits = f.attend.splits1 + f.attend.splits2;
    aa.part_offset = 0;
    HGA_TRY_HIP(launch_attend_splitk(aa, bf, st), "attend");
    return ok();
  }

  // events ordering the copy stream between routing and the routed attention:
  // one pair per thread and device, made on first use and kept
  constexpr int kMaxDevices = 64;
  thread_local hipEvent_t ev_pair[kMaxDevices][2] = {};
  int dev = 0;
  HGA_TRY_HIP(hipGetDevice(&dev), "get device");
  if (dev < 0 || dev >= kMaxDevices) return fail(HGA_ERR_UNSUPPORTED, "device index %d >= %d", dev, kMaxDevices);
  for (int i = 0; i < 2; ++i)
    if (!ev_pair[dev][i]) HGA_TRY_HIP(hipEventCreateWithFlags(&ev_pair[dev][i], hipEventDisableTiming), "event create");
  hipEvent_t ev_routed = ev_pair[dev][0], ev_copied = ev_pair[dev][1];
  HGA_TRY_HIP(hipEventRecord(ev_routed, st), "event record");
  HGA_TRY_HIP(hipStreamWaitEvent(cst, ev_routed, 0), "stream wait");
  {
    GatherArgs ga{};
    ga.kp = kp;
    ga.K_host = K_host;
    ga.V_host = V_host;
    ga.group_idx = gi;
    ga.K_stage = Kst;
    ga.V_stage = Vst;
    ga.elem_bytes = static_cast<int32_t>(elem_bytes(p));
    HGA_TRY_HIP(launch_gather_groups(ga, cst), "gather");
  }
  HGA_TRY_HIP(hipEventRecord(ev_copied, cst), "event record");

  // forced (hot) slots overlap the copy; routed slots read the staging buffer
  aa.part = 1;
  aa.splits = f.attend.splits1;
  aa.part_offset = 0;
  HGA_TRY_HIP(launch_attend_splitk(aa, bf, st), "attend (hot)");
  HGA_TRY_HIP(hipStreamWaitEvent(st, ev_copied, 0), "stream wait");
  aa.part = 2;
  aa.splits = f.attend.splits2;
  aa.part_offset = f.attend.splits1;
  HGA_TRY_HIP(launch_attend_splitk(aa, bf, st), "attend (routed)");
  return ok();
}

}  // namespace

hga_status hga_decode_offload(const hga_params* p, const void* Q, const void* K_host, const void* V_host,
                              const void* K_hot, const void* V_hot, int64_t n_cap, const int32_t* seq_len,
                              float* chunk_sum, float* group_sum, void* O, int32_t* chunk_idx,
                              int32_t* group_idx, void* staging, size_t staging_bytes, void* ws,
                              size_t ws_bytes, void* stream, void* copy_stream) {
  return decode_offload_impl(p, Q, K_host, V_host, K_hot, V_hot, n_cap, seq_len, chunk_sum, group_sum, O,
                             chunk_idx, group_idx, staging, staging_bytes, nullptr, ws, ws_bytes, stream,
                             copy_stream);
}

hga_status hga_decode_offload_warm(const hga_params* p, const void* Q, const void* K_host, const void* V_host,
                                   const void* K_hot, const void* V_hot, int64_t n_cap, const int32_t* seq_len,
                                   float* chunk_sum, float* group_sum, void* O, int32_t* chunk_idx,
                                   int32_t* group_idx, const hga_warm* warm, void* ws, size_t ws_bytes,
                                   void* stream, void* copy_stream) {
  if (!warm) return fail(HGA_ERR_ARG, "warm is null");
  return decode_offload_impl(p, Q, K_host, V_host, K_hot, V_hot, n_cap, seq_len, chunk_sum, group_sum, O,
                             chunk_idx, group_idx, nullptr, 0, warm, ws, ws_bytes, stream, copy_stream);
}

}  // extern "C"
