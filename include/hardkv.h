/*
 * hardkv.h -- C ABI of the HARD-KV decode-step library for MI355X (gfx950).
 *
 * The method is "HARD-KV: Head-Adaptive Regularization for Decoding-time KV
 * Compression" (arXiv abstract on mlsanity.com; gist.science technical
 * summary, section 2 "Methodology").  Per KV head, one decode step:
 *   score      q.K importance of every aged token            (section 2.B, Goal)
 *   calibrate  per-head softmax into one probability space  (section 2.B, Mechanism)
 *   top-p      smallest calibrated set with mass >= p       (section 2.A, Tier 2)
 *   compact    rewrite the selection into contiguous slots  (section 2.C, Rewrite
 *              Cache + Flatten Index) and pool the evicted
 *              tokens into condensed chunks                 (section 2.A, Tier 3)
 *   attention  over dense + sparse + condensed tiers        (abstract; section 3)
 * hardkv_step chains all of them; hardkv_step_inplace runs the multi-step
 * token lifecycle (section 2.A four-step pipeline) on persistent tiers.
 * hardkv_plan and hardkv_step_policy choose per head between rewriting the
 * selection and loading it in place (section 2.C: Sparse Loading, and the
 * Memory-Time Integral with budget thresholds under "Trade-off Management").
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a caller-owned DEVICE pointer unless it is a
 *     `const hardkv_*` descriptor struct, which lives in HOST memory and is
 *     read only during the call.  The library never allocates, frees or
 *     retains caller memory; kernels use the buffers until they complete on
 *     the given stream.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work: no host synchronisation, no device-to-host reads, no
 *     allocation, so every call can be captured into a HIP graph.
 *   - Every argument is validated on the host before the first launch; a call
 *     that returns an error has enqueued nothing.  Faults inside kernels show
 *     up at the caller's next synchronisation of the stream.  No C++
 *     exception crosses the ABI.
 *   - Device-resident sizes (ctx_len, counts) are clamped by the kernels to
 *     the capacities in the descriptor, so a bad value cannot make a kernel
 *     read or write out of bounds.
 *   - Shapes: B sequences, Hq query heads, Hkv KV heads, G = Hq / Hkv query
 *     heads per KV head (query head g belongs to KV head g / G), d head dim,
 *     T_b context length of sequence b (current token included), W dense
 *     window, S sink tokens, C chunk size, A_b = max(T_b - W - S, 0) aged
 *     tokens (the candidates, positions [S, S + A_b)).
 *   - Thread safety: the only global state is the optional launch observer;
 *     calls on distinct streams with distinct buffers may run concurrently.
 */
#ifndef HARDKV_H
#define HARDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hardkv_stream_t; /* same type as hipStream_t */

/* Return codes. */
#define HARDKV_OK 0
#define HARDKV_ERR_INVALID_ARG -1  /* null pointer, Hq % Hkv != 0, top_p not in (0,1], W < 0, C < 1, ... */
#define HARDKV_ERR_UNSUPPORTED -2  /* head_dim not 64/128, dtype, G not in {1,2,4,8} */
#define HARDKV_ERR_CAPACITY -3     /* sparse_cap / chunk_cap smaller than the aged capacity */
#define HARDKV_ERR_WORKSPACE -4    /* workspace missing or smaller than hardkv_workspace_size() */
#define HARDKV_ERR_HIP -5          /* a kernel launch failed (hipGetLastError) */

/* Element types of q, K and V (the compacted K/V use the cache's type). */
#define HARDKV_F32 0
#define HARDKV_BF16 1

/* Importance metric per KV head. */
#define HARDKV_METRIC_QK 0 /* max over the GQA group of q.k / sqrt(d) ("max-pooled logits") */
#define HARDKV_METRIC_L2 1 /* key L2 norm, calibrated onto the head's logit spread */
#define HARDKV_METRIC_WINDOW 2 /* observation window: max over the last obs_window queries and
                                  the GQA group of q.k / sqrt(d), max-pooled over positions
                                  [t - pool_radius, t + pool_radius]; calibrated like L2
                                  (section 2.B: SnapKV-style strategies) */
#define HARDKV_METRIC_KEYDIFF 3 /* key dissimilarity: -(k_t . mu) / (||k_t|| ||mu||), mu the
                                   sum of the head's candidate keys (0 for a zero vector),
                                   float64, one rounding; calibrated like L2 (section 2.B:
                                   similarity scores among the importance metrics) */
#define HARDKV_METRIC_RKV 4 /* R-KV redundancy: -(u_t . nu - [k_t != 0]) / (A - 1), the minus
                               mean cosine similarity to the other candidates, u the unit keys
                               (0 for a zero key), nu their sum over the head's candidates; 0
                               when A = 1; float64, one rounding; calibrated like L2
                               (section 2.B, "Mechanism": strategies such as R-KV) */

/* How L2 and window heads are calibrated (hardkv_desc.calibration); QK heads
 * always keep temperature 1 (section 2.B, Mechanism: a temperature maps a
 * metric onto the raw attention distribution). */
#define HARDKV_CALIB_SPREAD 0  /* c = (x - mean x) * std(logit) / std(x) */
#define HARDKV_CALIB_ENTROPY 1 /* c = (x - max x) * beta, softmax(beta x) with the entropy of
                                  softmax(logit) (section 2.A Tier 2: budgets from attention
                                  entropy); beta from a fixed 32-step float64 bisection */

/* How evicted tokens are merged into a condensed chunk (hardkv_desc.merge). */
#define HARDKV_MERGE_MEAN 0     /* plain mean of the chunk's evicted tokens */
#define HARDKV_MERGE_WEIGHTED 1 /* mean weighted by each token's calibrated attention weight */

/* How a head's selection is served (per head, device byte). */
#define HARDKV_MODE_REWRITE 0 /* kept rows copied into the tier's contiguous slots */
#define HARDKV_MODE_SPARSE 1  /* kept rows left in the cache, loaded through the tier's positions */

/* Policy kinds (hardkv_policy.kind). */
#define HARDKV_POLICY_REWRITE 0 /* every head rewritten */
#define HARDKV_POLICY_SPARSE 1  /* every head sparse-loaded */
#define HARDKV_POLICY_MTI 2     /* budget thresholds, then the memory-time integral */

/* Rewrite-versus-sparse-loading policy (host memory; section 2.C, "Trade-off
 * Management").  For a head with A aged tokens of which k are kept, window W:
 *   k <= l_lower -> rewrite; else k >= l_upper -> sparse loading; else the
 *   smaller memory-time integral over `horizon` steps (the selection step
 *   and horizon - 1 steps that reuse its tiers), in units of K/V rows:
 *     sparse  = (A + W)(3A + 2W) + (horizon - 1)(A + W) * 2(k + W)
 *     rewrite = (A + W + k)(3A + 2W + 2k) + (horizon - 1)(k + W) * 2(k + W)
 *   rewrite only if strictly smaller; computed in exact 128-bit integers. */
typedef struct hardkv_policy {
  int32_t kind;    /* HARDKV_POLICY_* */
  int32_t horizon; /* >= 1 */
  int32_t l_lower; /* budgets k <= l_lower are rewritten (e.g. 0) */
  int32_t l_upper; /* budgets k >= l_upper are sparse-loaded (e.g. INT32_MAX) */
} hardkv_policy;

/* Shapes and policy of one decode step (host memory). */
typedef struct hardkv_desc {
  int32_t batch;        /* B >= 1 */
  int32_t num_q_heads;  /* Hq, a multiple of Hkv */
  int32_t num_kv_heads; /* Hkv >= 1; G = Hq / Hkv must be 1, 2, 4 or 8 */
  int32_t head_dim;     /* d: 64 or 128 */
  int32_t dtype;        /* HARDKV_F32 or HARDKV_BF16 for q, K, V and the compacted tier */
  int32_t dense_window; /* W >= 0: the last W tokens form the dense tier */
  int32_t chunk;        /* C >= 1: condensed chunk j pools evicted positions [jC, (j+1)C) */
  int32_t block_size;   /* 0: contiguous cache; > 0: paged cache with this many tokens per block */
  int32_t ctx_cap;      /* largest allowed T_b; contiguous: token stride of the cache per (b, h) */
  int32_t max_blocks;   /* paged: entries per block-table row; ctx_cap <= max_blocks * block_size */
  int32_t sparse_cap;   /* sparse slots per (b, h); >= max(ctx_cap - W - S, 0) */
  int32_t chunk_cap;    /* chunk slots per (b, h); >= ceil(max(ctx_cap - W - S, 0) / C) */
  float top_p;          /* p in (0, 1]; p = 1 keeps every aged token */
  int32_t sinks;        /* S >= 0: positions [0, S) stay in the dense tier (attention sinks,
                           section 2.A Tier 1); candidates are [S, T - W) and chunk j pools
                           evicted positions [S + jC, S + (j+1)C).  0 = none */
  int32_t merge;        /* HARDKV_MERGE_*: condensed chunks (section 2.A Tier 3) store
                           n times the mean of their evicted keys / values, plain or weighted
                           by a = exp(max(c - m, -60)), c the token's calibrated value and m
                           the head's largest (float32); attention uses sum / n either way */
  int32_t packed_rows;  /* 0: the rewritten tier has a region of sparse_cap rows per head
                           (Flatten Index to the maximum length).  > 0: one region of this many
                           rows shared by all heads, laid end to end in (b, h) order (Flatten
                           Index to the sum; section 2.C, head-wise allocation under static
                           shapes); needs tiers->offset and tiers->mode, and
                           B * Hkv * sparse_cap < 2^31 */
  int32_t obs_window;   /* HARDKV_METRIC_WINDOW heads: queries in the observation window,
                           0..64 (0 or 1 = this step's query only; > 1 needs cache->q_hist) */
  int32_t pool_radius;  /* HARDKV_METRIC_WINDOW heads: max-pooling radius, 0..512 */
  int32_t calibration;  /* HARDKV_CALIB_*: the temperature rule of L2 and window heads */
  int32_t select_block; /* 0: top-p over tokens; a power of two bs in 1..1024: top-p over
                           whole blocks of positions [j bs, (j + 1) bs), each ranked by its
                           calibrated mass (section 2.C: selected blocks moved into contiguous
                           ranges); at most 4096 blocks per head (ceil(max aged / bs) + 1);
                           single-step calls only */
  int32_t tier_block;   /* 0: no block manager.  A power of two tb in 16..1024: the rewritten
                           tier lives in a shared pool of tier_blocks blocks of tb rows
                           (tiers->k, v = [tier_blocks][tb][d]); slot j of (b, h) is row
                           j % tb of block tiers->table[b][h][j / tb] (section 2.C, a
                           head-wise block manager for head-adaptive budgets under static
                           shapes); needs tiers->table, held, free_ids, free_top and mode;
                           excludes packed_rows; single-step calls only */
  int32_t tier_blocks;  /* blocks in that pool, 1 .. 2^31 / tb (tier_block > 0) */
} hardkv_desc;

/* The KV cache of one layer.
 *   contiguous: k, v = [B][Hkv][ctx_cap][d]
 *   paged:      k, v = [num_blocks][Hkv][block_size][d]; token t of sequence b,
 *               head h is row (t % block_size) of block block_table[b][t / block_size];
 *               the entries covering t < T_b must be block ids of k and v (they are
 *               read on the device and not checked: the pool's size is not passed)
 *   ctx_len:    [B] int32, 1 <= T_b <= ctx_cap (clamped on the device). */
typedef struct hardkv_cache {
  const void* k;
  const void* v;
  const int32_t* block_table; /* [B][max_blocks]; NULL for a contiguous cache */
  const int32_t* ctx_len;
  const void* q_hist;         /* [B][obs_window - 1][Hq][d] in desc->dtype: the previous
                                 decode queries, most recent first; NULL if obs_window <= 1 */
} hardkv_cache;

/* Sparse (rewritten) and condensed tiers.
 *   k, v:   [B][Hkv][sparse_cap][d] in the cache dtype; slots 0..count-1 hold the
 *           selected tokens as bit copies, ascending position; later slots unspecified
 *   pos:    [B][Hkv][sparse_cap] int32 original positions of those slots
 *   count:  [B][Hkv] int32 selected tokens (the head's budget k_{b,h})
 *   ksum, vsum: [B][Hkv][chunk_cap][d] float32 sums of the evicted keys / values
 *   ccount: [B][Hkv][chunk_cap] int32 evicted tokens per chunk (0 = empty chunk)
 *   mode:   [B][Hkv] uint8 HARDKV_MODE_* per head, or NULL (every head rewritten).
 *           A HARDKV_MODE_SPARSE head's k / v slots are neither written nor read:
 *           attention loads its kept rows from the cache at pos (Sparse Loading,
 *           section 2.C), so that cache must stay unchanged while the tiers are used.
 *   offset: [B][Hkv] int32, packed layout only (desc->packed_rows > 0; else may be
 *           NULL): k, v are then [packed_rows][d] and slot j of head (b, h) is row
 *           offset[b][h] + j (hardkv_pack).
 * Single-step calls write chunk slots [0, ceil(A_b / C)); the rest is unspecified. */
typedef struct hardkv_tiers {
  void* k;
  void* v;
  int32_t* pos;
  int32_t* count;
  float* ksum;
  float* vsum;
  int32_t* ccount;
  uint8_t* mode;
  int32_t* offset;
  /* block manager of the rewritten tier (desc->tier_block > 0; else may be NULL):
   *   table:    [B][Hkv][ceil(sparse_cap / tier_block)] int32 block ids, entries
   *             0 .. held - 1 valid
   *   held:     [B][Hkv] int32 blocks the head holds
   *   free_ids: [tier_blocks] int32 stack of free block ids, entries 0 .. *free_top - 1
   *   free_top: [1] int32
   * Set up once with hardkv_tier_init; every selection then returns each head's
   * blocks and hands out new ones (hardkv_tier_alloc).  The pool and this state
   * may be shared by several layers' tiers (one table and held array each). */
  int32_t* table;
  int32_t* held;
  int32_t* free_ids;
  int32_t* free_top;
} hardkv_tiers;

/* Persistent state of the multi-step lifecycle (one layer).
 *   ring_k, ring_v: [B][Hkv][W][d] dense window; position t lives in slot t % W
 *   tiers: sparse pool (positions ascending, `count` residents) and running chunk sums;
 *          tiers.mode must be NULL (the pool is always compacted in place)
 *   seq_len: [B] int32 tokens seen so far; must be >= W; advanced by one per step
 *
 * Head-wise block manager (section 2.C: a head-wise block manager allocates
 * head-adaptive budgets under static shapes).  pool_block = 0: every (b, h)
 * owns a region of sparse_cap pool rows (tiers.k / tiers.v = [B][Hkv][sparse_cap][d]).
 * pool_block > 0 (a power of two, at most 4096): pool row r of (b, h) lives in
 * row r % pool_block of block pool_table[b][h][r / pool_block] of a shared pool,
 * tiers.k / tiers.v = [pool_blocks][pool_block][d] (one head per block); tiers.pos
 * stays [B][Hkv][sparse_cap].  A head holds exactly ceil(count / pool_block)
 * blocks (table entries beyond are -1).  Every step, before the append, each
 * head whose next row starts a block takes one from the free stack
 * free_ids[0 .. *free_top) (top first, heads served in (b, h) order); after the
 * compaction every head returns the blocks it no longer needs (pushed in (b, h)
 * order, each head's in ascending table index).  Deterministic.  When the stack
 * is empty, the token leaving the window goes straight into its condensed
 * chunk instead of the pool.  The caller sets up the tables, the stack and the
 * pool rows (e.g. after prefill) so that these invariants hold. */
typedef struct hardkv_state {
  void* ring_k;
  void* ring_v;
  hardkv_tiers tiers;
  int32_t* seq_len;
  int32_t* pool_table;  /* [B][Hkv][ceil(sparse_cap / pool_block)] block ids or -1 */
  int32_t* free_ids;    /* [pool_blocks] stack of free block ids */
  int32_t* free_top;    /* [1] free ids on the stack */
  int32_t pool_block;   /* rows per block; 0 = per-head regions (the fields above unused) */
  int32_t pool_blocks;  /* blocks in the shared pool */
} hardkv_state;

/* Library version (major * 10000 + minor * 100 + patch). */
int hardkv_version(void);

/* Profiling hook.  When installed, `fn` is called on the calling thread right
 * before every kernel launch the library makes, with the kernel's name, the
 * stream it goes to and `user`, so a profiler can record stream events
 * between launches (per-kernel durations of one hardkv_step, say).  NULL
 * (the default) disables it.  The observer is process-wide: install or
 * remove it while no other thread is calling the library. */
typedef void (*hardkv_launch_observer)(const char* kernel, hardkv_stream_t stream, void* user);
void hardkv_set_launch_observer(hardkv_launch_observer fn, void* user);

/* Static text for a return code. */
const char* hardkv_strerror(int code);

/* Checks a descriptor.  Returns HARDKV_OK or the error any entry point would
 * return for it. */
int hardkv_validate(const hardkv_desc* desc);

/* Bytes of device workspace every entry point below needs for `desc`
 * (one buffer serves all of them).  0 if the descriptor is invalid.
 * The workspace is scratch: its contents are not preserved between calls,
 * and two calls that run at the same time need separate workspaces. */
size_t hardkv_workspace_size(const hardkv_desc* desc);

/* Importance scores of the aged tokens [0, A_b) of every (b, h)
 * (section 2.B, Goal: max-pooled logits and other similarity metrics).
 *   q:      [B][Hq][d] in desc->dtype
 *   metric: [Hkv] int8 HARDKV_METRIC_*, NULL = all QK
 *   logit:  [B][Hkv][sparse_cap] float32, logit[t] = fl32(max_g q_g.k_t / sqrt(d)),
 *           the dot product accumulated in float64
 *   l2:     [B][Hkv][sparse_cap] float32 second metric: key norms for HARDKV_METRIC_L2
 *           heads, the pooled window metric for HARDKV_METRIC_WINDOW heads (float64
 *           dots, one rounding, exact max-pooling), the key dissimilarity for
 *           HARDKV_METRIC_KEYDIFF heads and the redundancy for HARDKV_METRIC_RKV heads
 *           (the sum of the keys, or of the unit keys, is formed first, in float64 and
 *           in a fixed order, in the workspace); must be non-NULL whenever metric is
 *           non-NULL
 * Entries at t >= A_b are unspecified. */
int hardkv_score(const hardkv_desc* desc, const void* q, const hardkv_cache* cache,
                 const int8_t* metric, float* logit, float* l2, void* ws, size_t ws_bytes,
                 hardkv_stream_t stream);

/* Logits Calibration (section 2.B, Mechanism; section 3, second contribution).
 * For each (b, h) maps the aged tokens' metric x into calibrated values
 *   c_t = fl32((x_t - shift) * scale)
 * QK heads: x = logit, shift 0, scale 1 (the raw attention distribution).
 * L2 and window heads, x = l2:
 *   HARDKV_CALIB_SPREAD:  shift = mean(l2), scale = std(logit) / std(l2)
 *                         (population moments over the aged tokens; 0 if either
 *                         spread is 0)
 *   HARDKV_CALIB_ENTROPY: shift = max(l2), scale = beta with
 *                         H(softmax(beta l2)) = H(softmax(logit)), H the entropy:
 *                         the bracket [0, 1024 / (max l2 - min l2)] is halved 32
 *                         times (midpoint entropy above the target raises the lower
 *                         end) and beta is the final midpoint; 0 if l2 is constant.
 *                         Costs 32 float64 passes over the head's values.
 *   stats: [B][Hkv][4] float64 {shift, scale, m = max c, Z = sum exp(c - m)}. */
int hardkv_calibrate(const hardkv_desc* desc, const int32_t* ctx_len, const int8_t* metric,
                     const float* logit, const float* l2, double* stats, void* ws,
                     size_t ws_bytes, hardkv_stream_t stream);

/* Calibrated Top-p selection (section 2.A, Tier 2; section 2.B, Outcome).
 * Ranks the aged tokens by c (highest first, equal values lower position first)
 * and keeps the smallest prefix whose mass sum exp(c - m) reaches top_p * Z.
 * Masses are accumulated exactly in fixed point: 2^-47 units for heads of up to
 * 65536 candidates, 2^-(63 - ceil(log2 n)) for a larger candidate capacity n.
 *   mask:  [B][Hkv][sparse_cap] uint8, 1 = kept, for t < A_b (later bytes unspecified)
 *   count: [B][Hkv] int32 kept tokens. */
int hardkv_topp_select(const hardkv_desc* desc, const int32_t* ctx_len, const int8_t* metric,
                       const float* logit, const float* l2, const double* stats,
                       uint8_t* mask, int32_t* count, void* ws, size_t ws_bytes,
                       hardkv_stream_t stream);

/* Index Regularization (section 2.C: Rewrite Cache, Flatten Index to the
 * maximum length) and the condensed tier (section 2.A, Tier 3).  For every
 * (b, h): the tokens t < A_b with mask[t] = 1 are copied bit for bit into
 * out->k / out->v slots 0..count-1 in ascending position order with their
 * positions; every other aged token is added to the float32 sums of chunk
 * t / C.  Writes every field of *out (count = number of mask bytes set),
 * except the k / v slots of heads whose out->mode byte is HARDKV_MODE_SPARSE
 * (out->mode is read, e.g. as written by hardkv_plan).
 * The tiers must not alias the cache.  desc->merge must be HARDKV_MERGE_MEAN
 * (weighted merging needs the scores: hardkv_compact_scored). */
int hardkv_compact(const hardkv_desc* desc, const hardkv_cache* cache, const uint8_t* mask,
                   const hardkv_tiers* out, void* ws, size_t ws_bytes,
                   hardkv_stream_t stream);

/* hardkv_compact with the scores and statistics of the selection at hand
 * (as written by hardkv_score and hardkv_calibrate), which weighted merging
 * needs; for HARDKV_MERGE_MEAN it equals hardkv_compact. */
int hardkv_compact_scored(const hardkv_desc* desc, const hardkv_cache* cache,
                          const int8_t* metric, const float* logit, const float* l2,
                          const double* stats, const uint8_t* mask, const hardkv_tiers* out,
                          void* ws, size_t ws_bytes, hardkv_stream_t stream);

/* Decode attention over the three tiers (abstract; section 3, third
 * contribution).  For every query head g of (b, h = g / G): softmax over
 *   dense tokens [0, S) and [S + A_b, T_b)    logit q.k / sqrt(d), value v
 *   sparse slots 0..count-1 of the tiers      logit q.k / sqrt(d), value v
 *     (HARDKV_MODE_SPARSE heads: cache rows at pos[0..count-1] instead)
 *   chunks j < ceil(A_b / C) with n = ccount > 0: logit q.(ksum / n) / sqrt(d) + ln n,
 *                                             value vsum / n
 *   out: [B][Hq][d] float32.  Split-K partials live in the workspace.
 * Reusing a selection on later steps: after a step at length T with window W
 * wrote the tiers, a call with ctx_len T + i and dense_window W + i attends
 * the same sparse and condensed tiers plus every token that aged since,
 * densely (A_b stays that of the selection). */
int hardkv_decode_attn(const hardkv_desc* desc, const void* q, const hardkv_cache* cache,
                       const hardkv_tiers* tiers, float* out, void* ws, size_t ws_bytes,
                       hardkv_stream_t stream);

/* One complete decode step (section 2.A four-step pipeline for a single
 * step): score -> calibrate -> top-p -> compact -> attention, on one stream,
 * with intermediate scores, statistics and masks in the workspace.  When C
 * is a multiple of 64, attention over the rewritten rows is folded into the
 * compaction pass (the rows are attended while they are copied), so the
 * sparse tier is not read back; results equal hardkv_compact followed by
 * hardkv_decode_attn up to float32 summation order in the attention.
 *   metric: as in hardkv_score; tiers: written as by hardkv_compact, every
 *   head rewritten (tiers->mode, when given, is set to HARDKV_MODE_REWRITE;
 *   with a packed tier, heads that do not fit are sparse-loaded, hardkv_pack);
 *   out: [B][Hq][d] float32 attention output. */
int hardkv_step(const hardkv_desc* desc, const void* q, const hardkv_cache* cache,
                const int8_t* metric, const hardkv_tiers* tiers, float* out, void* ws,
                size_t ws_bytes, hardkv_stream_t stream);

/* Rewrite or sparse loading per head (section 2.C, "Trade-off Management"):
 *   count: [B][Hkv] int32 kept tokens k (as written by hardkv_topp_select)
 *   mode:  [B][Hkv] uint8 output, HARDKV_MODE_* from *policy with A = A_b. */
int hardkv_plan(const hardkv_desc* desc, const hardkv_policy* policy, const int32_t* ctx_len,
                const int32_t* count, uint8_t* mode, hardkv_stream_t stream);

/* Head-wise allocation of the packed rewritten tier (desc->packed_rows > 0;
 * section 2.C, "Metadata" and Flatten Index to the sum).  With need = count
 * for a HARDKV_MODE_REWRITE head and 0 for a sparse-loaded one, head i in
 * (b, h) order gets tiers->offset[i] = the sum of the needs before it; a
 * rewritten head whose rows would end past packed_rows is switched to
 * HARDKV_MODE_SPARSE (its attention is unchanged, its rows stay in the cache).
 * Reads count and tiers->mode, writes tiers->offset and tiers->mode.  Run it
 * after hardkv_plan and before hardkv_compact; the steps run it themselves. */
int hardkv_pack(const hardkv_desc* desc, const int32_t* count, const hardkv_tiers* tiers,
                hardkv_stream_t stream);

/* Set-up of the rewritten tier's block manager (desc->tier_block > 0): every
 * block free (free_ids[i] = i, *free_top = tier_blocks), every head holding
 * none (held = 0, table = -1).  A kernel launch (no memset), so it can be
 * captured.  Run it once before the first selection on a fresh pool; with a
 * pool shared by several tiers, once per tier before any of them selects
 * (each call also refills the shared stack). */
int hardkv_tier_init(const hardkv_desc* desc, const hardkv_tiers* tiers, hardkv_stream_t stream);

/* Head-wise block allocation of the rewritten tier (desc->tier_block > 0;
 * section 2.C, "Metadata": a head-wise block manager for head-adaptive
 * budgets under static shapes).  One workgroup, deterministic:
 *   1. every head, in (b, h) order, pushes its held blocks (table order) onto
 *      the free stack and then holds none;
 *   2. every HARDKV_MODE_REWRITE head, in (b, h) order, needs ceil(k / tier_block)
 *      blocks for its k = count kept rows (clamped to [0, max aged]) and pops them
 *      from the top of the stack into table entries 0, 1, ...; a head whose need
 *      exceeds what the heads before it left on the stack takes none and is
 *      switched to HARDKV_MODE_SPARSE (its rows stay in the cache; its attention
 *      is unchanged), and so is every head after it.
 * Reads count and tiers->mode; writes tiers->table, held, free_ids, free_top and
 * mode.  Run it after the selection (and hardkv_plan) and before hardkv_compact;
 * the steps run it themselves. */
int hardkv_tier_alloc(const hardkv_desc* desc, const int32_t* count, const hardkv_tiers* tiers,
                      hardkv_stream_t stream);

/* hardkv_step with a per-head choice between rewriting the selection and
 * loading it in place: the policy is evaluated right after the top-p
 * selection, tiers->mode (required) receives each head's choice, and
 * HARDKV_MODE_SPARSE heads skip the row copies.  The attention output is
 * the same function of the inputs for every choice (the selection, the
 * chunks and the positions do not depend on it). */
int hardkv_step_policy(const hardkv_desc* desc, const hardkv_policy* policy, const void* q,
                       const hardkv_cache* cache, const int8_t* metric,
                       const hardkv_tiers* tiers, float* out, void* ws, size_t ws_bytes,
                       hardkv_stream_t stream);

/* One decode step of the multi-step token lifecycle on persistent tiers
 * (section 2.A: tokens move dense -> sparse -> condensed as they age; the
 * sparse tier is re-selected every step).  For every (b, h), with P = seq_len[b]:
 *   0. (block manager) heads whose next pool row starts a block take one;
 *   1. append: the token in ring slot P % W (position P - W) moves to the end of
 *      the sparse pool (or, with the block manager out of blocks, into its
 *      chunk); k_new / v_new ([B][Hkv][d]) take its ring slot;
 *   2. score, calibrate and top-p over the pool residents;
 *   3. the kept residents are compacted in place (stable, positions ascending);
 *   4. every dropped resident is added to the running sums of chunk pos / C
 *      (block manager: blocks past the new count go back to the free stack);
 *   5. attention over the ring, the pool and the chunks -> out [B][Hq][d] f32;
 *   6. seq_len[b] += 1.
 * desc->block_size, sinks, merge, packed_rows, pool_radius and calibration must be 0 and obs_window
 * at most 1 (the pool has no position-ordered neighbours to pool or old queries to keep); ctx_cap bounds P + 1 and sizes the pool
 * (sparse_cap >= ctx_cap - W) and the chunks (chunk_cap >= ceil((ctx_cap - W) / C)).
 * With state->pool_block > 0: pool_table, free_ids and free_top non-NULL, pool_blocks >= 1,
 * B * Hkv * ceil(sparse_cap / pool_block) < 2^31 and pool_blocks * pool_block < 2^31. */
int hardkv_step_inplace(const hardkv_desc* desc, const void* q, const void* k_new,
                        const void* v_new, const int8_t* metric, const hardkv_state* state,
                        float* out, void* ws, size_t ws_bytes, hardkv_stream_t stream);

/* Bytes of the library-held workspace of hardkv_step_noalloc, per device. */
#define HARDKV_SCRATCH_BYTES ((size_t)64 << 20)

/* hardkv_step for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same launches as hardkv_step, with the workspace taken from a library-held
 * array of HARDKV_SCRATCH_BYTES on the current device (hipGetDevice; the
 * stream must belong to that device).  Each device's copy is set up on the
 * first call with that device current and lives until the process ends;
 * nothing is allocated or freed by any call.
 *   Arguments, layouts and results: as hardkv_step (the caller still owns q,
 *   the cache, the tiers and out).
 *   Errors: as hardkv_step, and HARDKV_ERR_WORKSPACE when
 *   hardkv_workspace_size(desc) exceeds HARDKV_SCRATCH_BYTES (the headline
 *   shape, 32 sequences x 8 KV heads x 16k tokens, needs 54 MiB);
 *   HARDKV_ERR_HIP when the device or the array's address cannot be queried.
 * Every call on one device shares that device's array, which keeps the last
 * call's contents (the step needs none of them: each kernel writes what it
 * reads later in the same call).  Calls that overlap on one device (two
 * streams, two threads) race on the array and must be serialised by the
 * caller. */
int hardkv_step_noalloc(const hardkv_desc* desc, const void* q, const hardkv_cache* cache,
                        const int8_t* metric, const hardkv_tiers* tiers, float* out,
                        hardkv_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* HARDKV_H */
