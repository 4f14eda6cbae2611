// Launch interfaces of the HGA kernels (host side of each .hip file).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hga_kparams.hpp"
#include "hga_warm_state.hpp"

namespace hga {

struct SummariesArgs {
  KParams kp;
  const void* K;      // [B, Hkv, n_cap, d]
  void* Krot;         // nullable (raw mode): RoPE'd rows written here
  float* chunk_sum;   // [B, Hkv, n_chunks_cap, d]
  float* group_sum;   // [B, Hkv, n_chunks_cap * m, d]
  int32_t chunk_begin, chunk_end, rotated;
};

// Where the rows of a chunk live for the fused summary update of a decode step.
struct RowSource {
  const void* base;       // rows of (b, kv head) bh start at base + bh * bh_rows * d
  int64_t bh_rows;
  int32_t ring;           // 0: chunk c at row c*C; 1: hot-window ring (sink slots, then n_local+1 ring slots)
};

struct RouteArgs {
  KParams kp;
  const void* Q;          // [B, Hq, nq, d]
  int64_t nq;
  const int32_t* q_pos;   // [B]: position of query row 0 is q_pos[b] + pos_bias
  int32_t pos_bias;
  const float* chunk_sum;
  const float* group_sum;
  int32_t n_units;        // units per (b, kv head)
  int32_t slices;         // scan workgroups per unit
  int32_t chunks_per_slice;
  float* scores;          // ws [B*Hkv*n_units, n_chunks_cap]: published slice winners
  int32_t* cand_ids;      // ws [B*Hkv*n_units, n_chunks_cap]
  float* gscores;         // ws [B*Hkv*n_units, top_k*m]
  uint32_t* counters;     // ws [B*Hkv*n_units], zero between calls
  int32_t* chunk_idx;     // [B*Hkv*n_units, top_k]
  int32_t* group_idx;     // [B*Hkv*n_units, top_g]
  float* scores_out;      // nullable [B*Hkv, n_chunks_cap] (decode)
  uint16_t* split;        // ws, MFMA prefill routing only: the summary tables as bf16 hi and lo parts
  // fused summary update (decode only): when the query completes its chunk
  int32_t build_summary;
  RowSource ksrc;
  float* chunk_sum_w;
  float* group_sum_w;
  // warm tier (decode, nullable tags): the unit's LRU lookup after its lists
  WarmState warm;
};

struct AttendArgs {
  KParams kp;
  const void* Q;          // [B, Hq, nq, d]
  int64_t nq;
  const int32_t* q_pos;
  int32_t pos_bias;
  const void* K;          // forced rows (and routed rows unless staged)
  const void* V;
  RowSource kv;           // layout of K/V rows for forced chunks (ring = hot window)
  const void* K_stage;    // nullable: routed groups packed [B*Hkv, top_g*G, d]
  const void* V_stage;
  const int32_t* group_idx;  // [B*Hkv*n_units, top_g]
  int32_t n_units;
  void* O;                // [B, Hq, nq, d]
  float* lse;             // nullable [B, Hq, nq]
  int32_t out_bf16;
  int32_t splits;         // workgroups per (bh, query row) in this launch
  int32_t tiles_per_split; // 16-row blocks per workgroup
  int32_t part;           // 0 all slots, 1 forced slots only, 2 routed slots only,
                          // 3 both parts in one grid (part1_splits workgroups on the forced slots)
  int32_t part1_splits;
  int32_t part_offset;    // partial slot of this launch's split 0
  int32_t parts_total;    // partial slots per (bh, row) over all launches
  float* partials;        // ws
  uint32_t* counters;     // ws [B*Hkv*nq]
  const int32_t* stage_slot;  // nullable [B*Hkv, top_g]: routed entry -> slot of K_stage/V_stage
                              // (>= 0 cached; -2 - slot: missing, read from K_host/V_host and
                              // written into that slot; -1 ignored)
  int32_t stage_slots;        // slots per (b, kv head) of K_stage/V_stage when stage_slot is set
  const void* K_host;         // nullable: pinned host [B, Hkv, n_cap, d] (warm tier misses)
  const void* V_host;
  void* V16;                  // ws, pipelined prefill only: V as fp16 blocks of 16 keys [B*Hkv, n_cap, d]
};

// A decode step (nq = 1) in one launch: routing and the routed rows' attention,
// forced-window attention and the summary update, and the merge of the parts.
struct DecodeArgs {
  KParams kp;
  const void* Q;             // [B, Hq, 1, d]
  const int32_t* seq_len;    // [B]: the query sits at position seq_len[b] + pos_offset
  const void* K;             // [B, Hkv, n_cap, d]
  const void* V;
  const float* chunk_sum;    // [B, Hkv, n_chunks_cap, d]
  const float* group_sum;    // [B, Hkv, n_chunks_cap * m, d]
  float* chunk_sum_w;        // the same tables, written for the chunk the query completes
  float* group_sum_w;
  int32_t build_summary;
  int32_t* chunk_idx;        // [B*Hkv, top_k]
  int32_t* group_idx;        // [B*Hkv, top_g]
  void* O;                   // [B, Hq, 1, d] (written here only for a position outside the cache)
  int32_t out_bf16;
  int32_t forced_wgs;        // forced-window workgroups per (b, kv head)
  int32_t forced_bpw;        // 16-row blocks of forced rows per forced workgroup
  int32_t routing_wgs;       // routing workgroups per (b, kv head); each routes and attends a share of the routed rows
  int32_t units_per_xcd;     // ceil(B*Hkv / kXcds)
  float* partials;           // ws [B*Hkv, forced_wgs + routing_wgs, gq * (d + 2)]: partial results
  uint32_t* sync;            // ws [B*Hkv, 4]: arrival counter of each unit (zero between calls)
  const int32_t* routes_in;  // nullable [B*Hkv, top_g]: given group lists (no routing; chunk_idx,
                             // group_idx, chunk_sum and group_sum unused)
  int32_t pos_offset;        // the query position is seq_len[b] + pos_offset
  int32_t warm_wgs;          // 0 or 1 per (b, kv head): reads the unit's candidate summaries
                             // into its XCD's L2 alongside the routing scans
};

struct GatherArgs {
  KParams kp;
  const void* K_host;     // pinned host [B, Hkv, n_cap, d]
  const void* V_host;
  const int32_t* group_idx;  // [B*Hkv, top_g]
  void* K_stage;          // [B*Hkv, top_g*G, d]
  void* V_stage;
  int32_t elem_bytes;
};

// Backward of the prefill attention over the selected sets (routing fixed).
struct BackwardArgs {
  KParams kp;
  const void* Q;             // [B, Hq, n, d]
  const void* K;             // [B, Hkv, n, d]
  const void* V;
  const int32_t* group_idx;  // [B*Hkv, n_units, top_g]
  const float* dO;           // [B, Hq, n, d]
  float* dQ;                 // [B, Hq, n, d]
  float* dK;                 // [B, Hkv, n, d]
  float* dV;
  float* stats;              // ws [B, Hq, n, 2]: base-2 log-sum-exp and D of every query row
  int64_t n;
  int32_t n_units;           // n / C
  int32_t unit_slice;        // query chunks per dK/dV workgroup (vector-ALU path)
  // matrix-core path (bf16): workspace regions
  uint16_t* dOh;             // [B, Hq, n, d] bf16: dO rounded
  uint16_t* dOl;             // [B, Hq, n, d] bf16: dO - dOh rounded
  uint32_t* vis;             // [B*Hkv, n_units, vis_words]: routed 16-key blocks per (key chunk, query chunk)
  int32_t vis_words;         // backward_vis_words(n_units)
  int32_t* counts;           // [B*Hkv, n_units]: query chunks that see each key chunk
};
bool backward_supported(const KParams& kp);
hipError_t launch_backward(const BackwardArgs& a, bool bf16_in, hipStream_t st);
// Matrix-core backward (bf16, C = 64, Hq/Hkv <= 4, G | 64, 16 | G).
bool backward_mfma_supported(const KParams& kp, bool bf16_in);
int backward_vis_words(int n_units);
hipError_t launch_backward_mfma(const BackwardArgs& a, hipStream_t st);

// Canonical form of a caller-given group list: entries that add no token to
// the visible set (repeats, groups of forced chunks, after the query chunk or
// outside the cache) become -1.
struct CanonArgs {
  KParams kp;
  const int32_t* in;      // [B*Hkv*n_units, top_g]
  int32_t* out;           // [B*Hkv*n_units, top_g]
  const int32_t* q_pos;   // [B] (nullable: 0); position of query row 0 is q_pos[b] + pos_bias
  int32_t pos_bias;
  int64_t nq;             // 1: decode (one unit per (b, kv head)); else query chunks of C rows
  int32_t n_units;
};
constexpr int kCanonMaxList = 1024;
hipError_t launch_canon_groups(const CanonArgs& a, hipStream_t st);

hipError_t launch_summaries(const SummariesArgs& a, bool bf16_in, hipStream_t st);
hipError_t launch_route_scan(const RouteArgs& a, bool bf16_q, bool bf16_k, hipStream_t st);
hipError_t launch_attend_splitk(const AttendArgs& a, bool bf16_in, hipStream_t st);
hipError_t launch_gather_groups(const GatherArgs& a, hipStream_t st);
// Decode routing launch (Hq/Hkv <= 4, d in {64, 128}, candidate and index limits).
constexpr int kXcds = 8;             // accelerator dies; workgroups are dealt to them in turn
constexpr int kDecMaxScores = 4096;  // chunk (and group) scores held in LDS per unit
constexpr int kDecMaxForced = 2;    // forced-window workgroups per (b, kv head)
constexpr int kDecMaxRouting = 2;   // routing workgroups per (b, kv head)
constexpr int kDecMaxParts = kDecMaxForced + kDecMaxRouting;
bool decode_fused_supported(const KParams& kp);
hipError_t launch_decode_step(const DecodeArgs& a, bool bf16_in, hipStream_t st);
// Prefill attention on the matrix cores (bf16, C = 64, Hq/Hkv <= 4, G | 64).
bool prefill_mfma_supported(const KParams& kp, bool bf16_in, int64_t nq);
hipError_t launch_attend_prefill_mfma(const AttendArgs& a, hipStream_t st);
// pipelined MFMA prefill attention (groups of whole 16-key blocks); needs the
// V16 region of prefill_pipe_v16_bytes in the workspace
bool prefill_pipe_supported(const KParams& kp, bool bf16_in, int64_t nq);
size_t prefill_pipe_v16_bytes(const KParams& kp);
hipError_t launch_attend_prefill_pipe(const AttendArgs& a, hipStream_t st);
// Prefill routing on the matrix cores (bf16, C = 64, Hq/Hkv <= 4).
bool route_prefill_mfma_supported(const KParams& kp, bool bf16_in, int64_t nq);
hipError_t launch_route_prefill_mfma(const RouteArgs& a, hipStream_t st);
// bytes of the split summary tables that the MFMA prefill routing needs in its workspace
size_t route_prefill_split_bytes(const KParams& kp);

// Workgroup counts and tiling chosen by the host for a given shape.
constexpr int kAttBlockRows = 16;  // K/V rows per attention block
constexpr int kAttMaxParts = 128;  // partial results per query row (workspace merge)
int route_chunks_per_slice(const KParams& kp, int64_t nq);
int attend_max_slots(const KParams& kp);

}  // namespace hga
