/*
 * hga.h — C ABI of the HGA routed-attention library for MI355X (gfx950).
 *
 * Hierarchical Global Attention (HGA) replaces dense causal attention with
 * (1) RoPE-aware chunk and group key summaries, (2) chunk routing against the
 * chunk-summary table, (3) group routing inside the routed chunks, (4) a union
 * with the always-visible current, sink and recent-local chunks, and (5) exact
 * token-level softmax attention over the gathered original K/V.
 * Sources: HGA technical summary, Italian page gist.science/it/paper/2606.30709,
 * section "Meccanismo Core" items 1-4 and section "Architettura della Memoria";
 * the same paper's French page (gist.science/fr/paper/2606.30709), section
 * "Mécanisme Central".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensors are caller-owned, contiguous, row-major, and 16-byte aligned.
 *   Device pointers unless marked "host".  The library keeps no pointer after
 *   a call returns, beyond the work it has enqueued.
 * - Q, O:   [B, Hq, nq, d]        K, V:  [B, Hkv, n_cap, d]
 *   chunk_sum: [B, Hkv, n_cap/C, d] float32; group_sum: [B, Hkv, n_cap/G, d] float32
 *   chunk_idx: [B, Hkv, n_units, top_k] int32; group_idx: [B, Hkv, n_units, top_g] int32
 *   (ascending ids, -1 padded).  Query head hq uses KV head hq / (Hq/Hkv).
 * - Q and K are post-RoPE (as a RoPE'd K/V cache holds them) unless a call says
 *   otherwise.  RoPE pairs are half-split: pair i = (x[i], x[i+d/2]),
 *   theta_i = rope_base^(-2i/d).  Pair i is high-frequency iff
 *   theta_i * C > hf_threshold (radians).
 * - Prefill units: one per (b, kv head, query chunk); nq is a multiple of C and
 *   q_pos[b] (the position of query row 0) is a multiple of C.  Decode: nq == 1,
 *   one unit per (b, kv head), the query at position q_pos[b].
 * - Every call is asynchronous on `stream` (a hipStream_t; NULL = default
 *   stream), allocates nothing, and never synchronises.  Scratch memory comes
 *   from the caller's workspace `ws` of at least hga_workspace_size() bytes.
 *   The workspace must be zero-filled once before its first use; every call
 *   leaves its counter region zeroed again when its kernels complete.  Calls
 *   that share one workspace must be ordered (same stream or events).
 * - Arguments are validated before anything is launched; a failed check
 *   returns a negative hga_status and enqueues nothing.  hga_last_error()
 *   returns a thread-local message for the last failure on the calling thread.
 *   Device faults surface at the caller's next synchronisation.
 */
#ifndef HGA_H
#define HGA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HGA_OK = 0,
  HGA_ERR_ARG = -1,          /* null pointer, negative size, bad enum */
  HGA_ERR_SHAPE = -2,        /* inconsistent or unsupported sizes */
  HGA_ERR_ALIGN = -3,        /* pointer not 16-byte aligned */
  HGA_ERR_WORKSPACE = -4,    /* workspace missing or too small */
  HGA_ERR_UNSUPPORTED = -5,  /* valid but not implemented combination */
  HGA_ERR_HIP = -6           /* a HIP runtime call failed (see hga_last_error) */
} hga_status;

typedef enum { HGA_BF16 = 0, HGA_F32 = 1 } hga_dtype;

typedef enum {
  HGA_OP_ROUTE = 0,
  HGA_OP_ATTEND = 1,
  HGA_OP_PREFILL = 2,
  HGA_OP_DECODE = 3,
  HGA_OP_DECODE_OFFLOAD = 4,
  HGA_OP_PREFILL_BACKWARD = 5
} hga_op;

/* Method parameters.  [HGA-it, Meccanismo Core]: item 1 fixes the chunk size C
 * and its groups; item 2 the routed chunks/groups and the always-visible sink,
 * local and current chunks; item 3 the RoPE-aware summaries. */
typedef struct {
  int32_t batch;         /* B >= 1 */
  int32_t n_q_heads;     /* Hq: Hq/Hkv in {1, 2, 4, 8, 16} */
  int32_t n_kv_heads;    /* Hkv >= 1 */
  int32_t head_dim;      /* d: 64 or 128 */
  int32_t chunk_size;    /* C: 1..256 */
  int32_t group_size;    /* G: divides C, C/G <= 64 */
  int32_t n_sink;        /* always-visible leading chunks, >= 0 */
  int32_t n_local;       /* always-visible chunks right before the current one, >= 0 */
  int32_t top_k;         /* routed chunks per unit, 0..1024 */
  int32_t top_g;         /* routed groups per unit, 0..min(1024, top_k*C/G) */
  double rope_base;      /* > 1 */
  double hf_threshold;   /* radians, >= 0 (1.0 by default) */
  int32_t qkv_dtype;     /* hga_dtype of Q, K, V */
  int32_t out_dtype;     /* hga_dtype of O */
} hga_params;

/* Bytes of workspace an operation needs (0 on invalid params; see
 * hga_last_error).  `nq` is the number of query rows per sequence (1 for
 * decode), `n_cap` the token capacity of the K/V cache.  With bf16 inputs and
 * nq > 1 (prefill), the attention's share includes an fp16 copy of V
 * (B*Hkv*n_cap*d*2 bytes) and the routing's share the summary tables split
 * into bf16 high and low parts; both are rebuilt by every call. */
size_t hga_workspace_size(const hga_params* p, int32_t op, int64_t nq, int64_t n_cap);

/* Step 1: RoPE-aware chunk and group summaries [HGA-it, Meccanismo Core,
 * item 3] for chunks [chunk_begin, chunk_end) of every (b, kv head).  All
 * tokens of those chunks must be present in K (chunk_end*C <= n_cap).
 * For every span S (a chunk or one of its groups) with representative position
 * p_S (the span's centre) and pair i:
 *   high-frequency i: mean over t in S of the key rotated to its own position t;
 *   low-frequency i:  mean over S of the raw key, rotated to p_S.
 * k_is_rotated = 1: K holds post-RoPE keys (computed in the equivalent
 * relative-angle form, no large angles).  k_is_rotated = 0: K holds raw
 * projected keys; if K_rot_out is non-null it receives the RoPE'd keys of the
 * same chunks (same layout and dtype as K).  Writes chunk_sum / group_sum. */
hga_status hga_build_summaries(const hga_params* p, const void* K, int64_t n_cap,
                               int32_t chunk_begin, int32_t chunk_end, int32_t k_is_rotated,
                               void* K_rot_out, float* chunk_sum, float* group_sum,
                               void* stream);

/* Steps 2-3: two-level routing [HGA-it, Meccanismo Core, item 2, first two
 * bullets].  For each unit with query chunk j and query vectors U (all query
 * heads of the KV head; all rows of the chunk in prefill):
 *   candidates  M = chunks [n_sink, j - n_local)
 *   score(c)    = max over q in U of q . chunk_sum[c] / sqrt(d)
 *   chunk_idx   = best min(top_k, |M|) by (score desc, id asc), ascending
 *   groups      = the C/G groups of every routed chunk
 *   group_idx   = best min(top_g, |groups|) by group score, ascending (global ids)
 * q_pos: [B] int32 device, position of query row 0.  chunk_sum/group_sum must
 * be built for every candidate chunk.  scores_out (nullable, decode only):
 * [B, Hkv, n_cap/C] float32 chunk scores (candidates only are written). */
hga_status hga_route(const hga_params* p, const void* Q, int64_t nq, const int32_t* q_pos,
                     const float* chunk_sum, const float* group_sum, int64_t n_cap,
                     int32_t* chunk_idx, int32_t* group_idx, float* scores_out,
                     void* ws, size_t ws_bytes, void* stream);

/* Steps 4-5: visibility union and exact attention [HGA-it, Meccanismo Core,
 * item 2 third bullet, item 4].  A query at position t in chunk j attends, with
 * a plain softmax of q.k/sqrt(d), to exactly the tokens u <= t of the set union
 * of the sink chunks [0, n_sink), the local chunks [j - n_local, j), chunk j and
 * the groups listed in group_idx for its unit.  The list may be in any order;
 * -1 holes, ids outside [0, n_cap/G), a group listed twice, a group inside a
 * forced chunk and a group after chunk j add no token (each token counts
 * once).  Putting a list in that form costs O(top_g^2) per unit, done on the
 * device.  No summary enters the output.  O: [B, Hq, nq, d] of out_dtype;
 * lse_out (nullable): [B, Hq, nq] float32 natural-log sum of exp of the scaled
 * scores. */
hga_status hga_attend(const hga_params* p, const void* Q, int64_t nq, const int32_t* q_pos,
                      const void* K, const void* V, int64_t n_cap, const int32_t* group_idx,
                      void* O, float* lse_out, void* ws, size_t ws_bytes, void* stream);

/* Steps 1-5 for a full causal prefill of n tokens (q_pos = 0 for every
 * sequence): builds chunk_sum/group_sum for every complete chunk, routes every
 * query chunk, attends.  Q: [B, Hq, n, d]; K, V: [B, Hkv, n, d]; n a multiple
 * of C.  chunk_idx / group_idx (nullable) receive the routing of every unit. */
hga_status hga_prefill(const hga_params* p, const void* Q, const void* K, const void* V,
                       int64_t n, float* chunk_sum, float* group_sum, void* O,
                       int32_t* chunk_idx, int32_t* group_idx,
                       void* ws, size_t ws_bytes, void* stream);

/* One decode step.  Query b (Q: [B, Hq, 1, d]) sits at position
 * seq_len[b] - 1 and its K/V row is already in the cache.  Routes against
 * chunk_sum/group_sum (which must hold every chunk before
 * (seq_len-1)/C - n_local), then attends.  When seq_len[b] is a multiple of C
 * the step also writes the summaries of the chunk it completes, so a decode
 * loop keeps the tables current without separate build calls.
 * seq_len: [B] int32 device, 1 <= seq_len[b] <= n_cap.  chunk_idx/group_idx
 * (nullable): [B, Hkv, 1, top_k|top_g]. */
hga_status hga_decode(const hga_params* p, const void* Q, const void* K, const void* V,
                      int64_t n_cap, const int32_t* seq_len, float* chunk_sum, float* group_sum,
                      void* O, int32_t* chunk_idx, int32_t* group_idx,
                      void* ws, size_t ws_bytes, void* stream);

/* hga_decode without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, results and launch as hga_decode, minus
 * ws / ws_bytes: the scratch (per-unit arrival counters, partial softmax
 * results, and the index lists when chunk_idx / group_idx are null) lives in
 * a static device array of 16 MiB that the library holds on every device it
 * runs on until the process ends.  Limits: the shapes of hga_decode's
 * one-launch kernel (Hq/Hkv in {1, 2, 4}, d in {64, 128}, C and G powers of
 * two, top_g <= 256), B * Hkv <= 1024 and the scratch size; anything else
 * returns HGA_ERR_UNSUPPORTED or HGA_ERR_SHAPE before any launch.  The first
 * call on a device also enqueues, ahead of its step, a small kernel that
 * clears the array's counters (make it outside graph capture, or replay the
 * captured graph before other calls); every call leaves them cleared again.
 * Calls on one device share the array: calls that overlap in time on one
 * device (different streams, no ordering) race and give wrong results. */
hga_status hga_decode_static(const hga_params* p, const void* Q, const void* K, const void* V,
                             int64_t n_cap, const int32_t* seq_len, float* chunk_sum,
                             float* group_sum, void* O, int32_t* chunk_idx, int32_t* group_idx,
                             void* stream);

/* Decode with the cold tier in host memory [HGA-it, Architettura della
 * Memoria: hot / warm / cold tiers; Meccanismo Core item 4: routed K/V fetched
 * from host RAM into device memory].  K_host, V_host: [B, Hkv, n_cap, d] in
 * pinned host memory allocated with hipHostMalloc (mapped).  K_hot, V_hot:
 * device [B, Hkv, (n_sink + n_local + 1) * C, d] hot windows: slot s holds
 * chunk s for s < n_sink; the recent chunks live in a ring: chunk c >= n_sink
 * sits in slot n_sink + (c - n_sink) % (n_local + 1).  The hot windows must
 * hold the sink chunks, the n_local chunks before the current one and the
 * current chunk's tokens up to the query.  Routing runs on device-resident
 * summaries; the routed groups are then copied from host into `staging`
 * (device, >= 2*B*Hkv*top_g*G*d*elem bytes: K rows, then V rows) by a copy
 * kernel on `copy_stream`,
 * ordered after routing and before attention by events; attention reads only
 * device memory (the hot-window part of it overlaps the copy).  Like
 * hga_decode, a step whose query completes its chunk also writes that chunk's
 * summaries, read from the hot window.
 * The two events are the one resource the library creates itself: a pair per
 * calling thread and device, made (hipEventCreateWithFlags, timing disabled)
 * by that thread's first offload call on the device and kept until the process
 * ends.  A failure to create them returns HGA_ERR_HIP before any launch. */
hga_status hga_decode_offload(const hga_params* p, const void* Q, const void* K_host,
                              const void* V_host, const void* K_hot, const void* V_hot,
                              int64_t n_cap, const int32_t* seq_len, float* chunk_sum,
                              float* group_sum, void* O, int32_t* chunk_idx,
                              int32_t* group_idx, void* staging, size_t staging_bytes,
                              void* ws, size_t ws_bytes, void* stream, void* copy_stream);

/* Backward of hga_prefill's attention [HGA-it, Meccanismo Core, item 4: the
 * output is an exact softmax over the selected tokens].  Gradients of O with
 * respect to Q, K and V for an upstream gradient dO, with the routing held
 * fixed: the selection is a piecewise-constant function of the inputs, so no
 * gradient flows through it (nor into the summaries).  The visible sets are
 * those of the forward: the sink, local and current chunks plus the groups of
 * group_idx (as hga_prefill returned it, or any list, read as hga_attend
 * reads it), causal.  Q, K, V as in
 * hga_prefill (C = 64); dO: [B, Hq, n, d] float32; dQ: [B, Hq, n, d] float32,
 * dK, dV: [B, Hkv, n, d] float32, all written.  Workspace:
 * hga_workspace_size(p, HGA_OP_PREFILL_BACKWARD, n, n).  Float atomics sum
 * the key-side partials, so dK and dV may differ in the last bits from run to
 * run. */
hga_status hga_prefill_backward(const hga_params* p, const void* Q, const void* K, const void* V,
                                int64_t n, const int32_t* group_idx, const float* dO, float* dQ,
                                float* dK, float* dV, void* ws, size_t ws_bytes, void* stream);

/* Warm tier of hga_decode_offload_warm [HGA-it, Architettura della Memoria:
 * a bounded LRU cache in device memory holds the recently routed chunks].
 * The cached unit is the routed group, the unit the cold tier copies.  Every
 * buffer is device memory owned by the caller and kept from step to step:
 *   K, V:    [B, Hkv, slots, G, d] (qkv dtype): the cached groups' rows;
 *   tags:    [B, Hkv, slots] int32: the group each slot holds, -1 if empty;
 *   stamps:  [B, Hkv, slots] int32: the last step that used each slot;
 *   clock:   [B, Hkv] int32: steps taken.
 * Before the first step tags must be all -1 and stamps and clock all 0 (K and
 * V may hold anything).  hits, misses (nullable) [B, Hkv] int32 receive, per
 * step, the routed groups found cached and the ones copied in from host. */
typedef struct hga_warm {
  void* K;
  void* V;
  int32_t* tags;
  int32_t* stamps;
  int32_t* clock;
  int32_t* hits;
  int32_t* misses;
  int32_t slots;  /* slots per (b, kv head), top_g <= slots <= 1024 */
} hga_warm;

/* hga_decode_offload with the warm tier in place of the staging buffer.
 * After routing, a lookup kernel maps each routed group of a (b, kv head) to a
 * slot: a group already cached keeps its slot (a hit, the slot's stamp is
 * renewed); the missing groups take the least recently used slots that this
 * step does not use (smallest stamp first, the lower slot on equal stamps; the
 * j-th missing group in list order gets the j-th of those slots in slot
 * order).  Attention reads the cached groups' rows from their slots and the
 * missing groups' rows from host memory, and writes the latter into the
 * slots the lookup chose, so only the missing groups cross the host link and
 * their copy overlaps the attention of the cached ones.  Everything runs on
 * `stream`: `copy_stream` is not used (it may be null) and no event is
 * created.  The output equals hga_decode_offload's bit for bit (the
 * attention splits its work and merges the parts the same way).  Steps that
 * share one `warm` must be ordered (same stream or events). */
hga_status hga_decode_offload_warm(const hga_params* p, const void* Q, const void* K_host,
                                   const void* V_host, const void* K_hot, const void* V_hot,
                                   int64_t n_cap, const int32_t* seq_len, float* chunk_sum,
                                   float* group_sum, void* O, int32_t* chunk_idx,
                                   int32_t* group_idx, const hga_warm* warm, void* ws,
                                   size_t ws_bytes, void* stream, void* copy_stream);

/* Message of the last failed call on this thread ("" if none). */
const char* hga_last_error(void);

/* Library version string. */
const char* hga_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HGA_H */
