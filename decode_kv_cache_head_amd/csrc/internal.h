// Host-side launch interfaces between the C ABI and the kernels.
#pragma once

#include "common.h"

namespace hk {

// Dispatch on element type, head dim and GQA group size (compile-time
// specialisations for every supported combination).
#define HK_DISPATCH_G(T, D, G, FN, ...)               \
  do {                                                \
    switch (G) {                                      \
      case 1: FN<T, D, 1>(__VA_ARGS__); break;        \
      case 2: FN<T, D, 2>(__VA_ARGS__); break;        \
      case 4: FN<T, D, 4>(__VA_ARGS__); break;        \
      default: FN<T, D, 8>(__VA_ARGS__); break;       \
    }                                                 \
  } while (0)
#define HK_DISPATCH_D(T, D, G, FN, ...)                       \
  do {                                                        \
    if ((D) == 64) HK_DISPATCH_G(T, 64, G, FN, __VA_ARGS__);  \
    else HK_DISPATCH_G(T, 128, G, FN, __VA_ARGS__);           \
  } while (0)
#define HK_DISPATCH(DT, D, G, FN, ...)                                  \
  do {                                                                  \
    if ((DT) == HARDKV_F32) HK_DISPATCH_D(float, D, G, FN, __VA_ARGS__); \
    else HK_DISPATCH_D(bf16_t, D, G, FN, __VA_ARGS__);                  \
  } while (0)
// ... and on the cache layout (paged or contiguous rows) as a fourth parameter.
#define HK_DISPATCH_GP(T, D, G, P, FN, ...)                  \
  do {                                                       \
    switch (G) {                                             \
      case 1: FN<T, D, 1, P>(__VA_ARGS__); break;            \
      case 2: FN<T, D, 2, P>(__VA_ARGS__); break;            \
      case 4: FN<T, D, 4, P>(__VA_ARGS__); break;            \
      default: FN<T, D, 8, P>(__VA_ARGS__); break;           \
    }                                                        \
  } while (0)
#define HK_DISPATCH_DP(T, D, G, P, FN, ...)                              \
  do {                                                                   \
    if ((D) == 64) HK_DISPATCH_GP(T, 64, G, P, FN, __VA_ARGS__);         \
    else HK_DISPATCH_GP(T, 128, G, P, FN, __VA_ARGS__);                  \
  } while (0)
#define HK_DISPATCH_TP(T, D, G, PAGED, FN, ...)                            \
  do {                                                                     \
    if (PAGED) HK_DISPATCH_DP(T, D, G, true, FN, __VA_ARGS__);             \
    else HK_DISPATCH_DP(T, D, G, false, FN, __VA_ARGS__);                  \
  } while (0)
#define HK_DISPATCH_P(DT, D, G, PAGED, FN, ...)                                   \
  do {                                                                          \
    if ((DT) == HARDKV_F32) HK_DISPATCH_TP(float, D, G, PAGED, FN, __VA_ARGS__); \
    else HK_DISPATCH_TP(bf16_t, D, G, PAGED, FN, __VA_ARGS__);                  \
  } while (0)

// Profiling hook: reports every kernel launch (name, stream) just before it
// is enqueued when an observer is installed through the C ABI.
void observe(const char* kernel, hipStream_t st);

struct ScoreArgs {
  int dtype, D, G, B, hq, hkv;
  const void* q;
  const void* q_hist;  // [B][window - 1][Hq][D] previous queries (window metric)
  int window;          // queries in the observation window (>= 1)
  int radius;          // max-pooling radius of the window metric
  float* wx;           // workspace [B][Hkv][cap_stride]: window metric before pooling
  double* q64;        // workspace [B][window][Hq][D]
  double* kmu;        // workspace [B][Hkv][D + 1]: key sum and its norm (key-dissimilarity heads)
  bool q_ready;       // q64 already holds this step's queries (the lifecycle's append widens them)
  Rows rows;          // candidate key rows
  Cand cand;
  int max_cand;       // upper bound of any (b, h)'s candidate count
  const int8_t* metric;
  float* logit;
  float* l2;
  int64_t cap_stride; // elements per (b, h) in logit / l2
  double scale;       // 1 / sqrt(D)
};
void launch_score(const ScoreArgs& a, hipStream_t st);

struct SelectArgs {
  int B, hkv;
  Cand cand;
  const int8_t* metric;
  const float* logit;
  const float* l2;
  int64_t cap_stride;
  double* stats;        // [B][Hkv][4] {shift, scale, max, Z}
  float top_p;
  uint8_t* mask;        // [B][Hkv][cap_stride]
  int32_t* count;       // [B][Hkv]
  uint8_t* mode;        // [B][Hkv] rewrite / sparse choice, written with count; may be null
  hardkv_policy policy;
  int calib;            // HARDKV_CALIB_* for heads on the second score array
  int block;            // > 0: block-granular selection, blocks of this many positions
  // the steps' own statistics: calibrate leaves Z out and the select records
  // it as its fixed-point total (nothing downstream reads Z)
  bool z_from_select;
  // kept tokens per kKeptBlk-token block of each head, [B][Hkv][kept_stride]
  // (for the compaction's tile offsets); null = not emitted
  int32_t* kept_blk;
  int kept_stride;
};
void launch_calibrate(const SelectArgs& a, hipStream_t st);
// top-p over position-aligned blocks ranked by calibrated mass (after calibrate)
constexpr int kBlockSelMax = 4096;  // blocks per head
void launch_blocksel(const SelectArgs& a, hipStream_t st);
void launch_select(const SelectArgs& a, hipStream_t st);
// calibrate + select in one launch, scores in registers (max_cand <= 16384)
bool calsel_fits(int max_cand);
void launch_calsel(const SelectArgs& a, int max_cand, hipStream_t st);
// mode[b][h] from count[b][h] and the candidate count
void launch_plan(const SelectArgs& a, hipStream_t st);
// offsets of the packed rewritten tier (and overflow -> sparse loading)
// Block manager of the rewritten tier (tier_block rows per block).
struct TierBlocks {
  int32_t* table;     // [n_heads][maxb]
  int32_t* held;      // [n_heads]
  int32_t* free_ids;  // [nblocks]
  int32_t* free_top;  // [1]
  int lbs;            // log2(rows per block)
  int maxb;           // table entries per head
  int nblocks;
};
constexpr int kTierMaxHeads = 16384;  // heads one allocation handles (its scans live in LDS)
void launch_tier_init(const TierBlocks& tb, int n_heads, hipStream_t st);
void launch_tier_alloc(const TierBlocks& tb, int n_heads, const int32_t* count, int cap,
                       uint8_t* mode, hipStream_t st);
void launch_pack(int n_heads, const int32_t* count, int cap, uint8_t* mode, int32_t* offset,
                 int packed_rows, hipStream_t st);

// Tile of the single-step compaction: whole chunks, about 1024 tokens
// (one chunk when a chunk is longer), processed in 64-row sub-tiles.
// Candidate rows per compaction tile: whole chunks, ~1024 rows.  Capacities
// of 16385 to 32768 candidates take 512-row tiles when C divides 512: on a
// batch of uneven heads of that length the shorter tiles end with a shorter
// tail (measured: 8k-32k ragged batch -4 %, uniform 64k heads +2 %, so
// longer capacities keep 1024).
inline int compact_tile(int C, int max_cand) {
  if (max_cand > 16384 && max_cand <= 32768 && 512 % C == 0) return 512;
  return C >= 1024 ? C : C * (1024 / C);
}
// Chunks of whole 64-row sub-tiles take the register-streaming compaction,
// which can also fold attention over the kept rows into the same pass.
inline bool compact_fusable(int C) { return C % 64 == 0 && compact_tile(C, 0) <= 1024; }

// Head-wise block manager of the lifecycle pool: table == nullptr means
// per-head regions of sparse_cap rows.
struct PoolPaging {
  int32_t* table;     // [B * Hkv][maxb] block ids or -1
  int32_t* free_ids;  // [nblocks] stack
  int32_t* free_top;  // [1]
  int lbs;            // log2(rows per block)
  int maxb;           // table entries per head
  int nblocks;
};

// Kept-token counts per block of candidates, from the select kernels: a
// compaction tile starts at the sum of the counts before it instead of
// counting the mask bytes before it.
constexpr int kKeptBlk = 512;
constexpr int kKeptMaxBlks = 256;  // blocks a select kernel counts in LDS (131072 candidates)
inline int kept_stride(int max_cand) { return ceil_div(max_cand, kKeptBlk); }

struct CompactArgs {
  int dtype, D, B, hkv, C;
  Rows krows, vrows;    // candidate rows
  Cand cand;
  int max_cand;
  const uint8_t* mask;
  int64_t cap_stride;   // mask / tier slots per (b, h)
  char* out_k;          // [B][Hkv][cap_stride][D]
  char* out_v;
  int32_t* out_pos;
  int32_t* out_count;
  float* ksum;          // [B][Hkv][chunk_stride][D]
  float* vsum;
  int32_t* ccount;
  int chunk_stride;
  const uint8_t* mode;  // [B][Hkv]; HARDKV_MODE_SPARSE heads skip the row copies; may be null
  const int32_t* offset;  // packed tier: head (b, h)'s slot 0 is row offset[b][h]; may be null
  const int32_t* kept_blk;  // kept tokens per kKeptBlk block ([B][Hkv][kept_stride]); may be null
  int kept_stride;
  // block manager of the rewritten tier: slot j of head i is row
  // (tier_table[i][j >> tier_lbs] << tier_lbs) + (j & mask) of out_k / out_v; may be null
  const int32_t* tier_table;
  int tier_lbs, tier_maxb, tier_nblocks;
  // -1: the slot's block id lies outside the pool (nothing is stored)
  __device__ inline int64_t tier_slot(int64_t bh, int j) const {
    const int id = tier_table[bh * tier_maxb + (j >> tier_lbs)];
    if (id < 0 || id >= tier_nblocks) return -1;
    return ((int64_t)id << tier_lbs) + (j & ((1 << tier_lbs) - 1));
  }
  int pos_off;          // position of candidate 0 (the sink count)
  // weighted merging (merge == HARDKV_MERGE_WEIGHTED): per-token weights from
  // the selection's scores and statistics
  int merge;
  const int8_t* metric;
  const float* logit;
  const float* l2;
  const double* stats;  // [B][Hkv][4] {shift, scale, max, Z}
  PoolPaging pg;         // in place: pool rows through per-head block tables
  // fused attention over the kept rows (launch_compact_attn only)
  int G, hq;
  const void* q;        // [B][Hq][D]
  float* part;          // partials [B][Hkv][max_tiles][G][D + 2]; tile j -> slot j
  int max_tiles;
  float scale;
};
void launch_compact(const CompactArgs& a, hipStream_t st);
void launch_compact_attn(const CompactArgs& a, hipStream_t st);
void launch_compact_inplace(const CompactArgs& a, hipStream_t st);

struct AttnArgs {
  int dtype, D, G, B, hkv, hq;
  const void* q;
  // dense tier: single step = cache positions [A_b, T_b); lifecycle = ring of W slots
  Rows dk, dv;
  const int32_t* ctx_len;  // single step
  int ctx_cap, W;
  int sinks;               // single step: dense = [0, sinks) and [sinks + A, T)
  bool ring;
  // sparse tier
  Rows sk, sv;
  const int32_t* count;
  int sparse_cap;
  // sparse loading: heads whose mode byte is HARDKV_MODE_SPARSE read their
  // kept rows from the dense-tier rows (the cache) at pos; may be null
  const uint8_t* mode;
  const int32_t* pos;
  const int32_t* offset;   // packed tier (see CompactArgs); may be null
  // condensed tier
  const float* ksum;
  const float* vsum;
  const int32_t* ccount;
  int chunk_cap, C;
  float* part;             // workspace partials
  int max_tiles;
  float* out;
  double scale;
  // > 0: the sparse and condensed tiers were attended by the fused
  // compaction (its tiles of fused_tt candidates own partial slots 0..);
  // only dense tiles here
  int fused_tt;
  // lifecycle: advance[b] += 1 for every sequence once the outputs are
  // written (by the merge); null elsewhere
  int32_t* advance;
  // set by the launcher: the chunk launch holds one tile per head, which
  // joins the head's partials itself (no merge launch follows)
  bool merge_chunks;
};
int attn_max_tiles(int W, int sparse_cap, int chunk_cap);
void launch_attn(const AttnArgs& a, hipStream_t st);

struct AppendArgs {
  int dtype, D, B, hkv, W, sparse_cap, ctx_cap;
  const void* k_new;
  const void* v_new;
  char* ring_k;
  char* ring_v;
  char* pool_k;
  char* pool_v;
  int32_t* pool_pos;
  int32_t* pool_count;
  const int32_t* seq_len;
  PoolPaging pg;
  // condensed tier, for a token that finds no free block
  float* ksum;
  float* vsum;
  int32_t* ccount;
  int C, chunk_cap;
  // this step's queries widened to float64 for the score: head h's block
  // writes q64[b][hG .. hG + G)[:] from q (hq query heads)
  const void* q;
  double* q64;
  int hq;
};
void launch_append(const AppendArgs& a, hipStream_t st);

// The lifecycle step's append, score, calibrate + select and in-place
// compaction in one workgroup per (b, h) (launches with every head on the
// logit and per-head pool regions).
struct LifeArgs {
  AppendArgs ap;        // ring, pool, lengths, the new token (q64 unused)
  CompactArgs ca;       // in-place compaction of the pool (mask in the workspace)
  const void* q;        // [B][Hq][D]
  float* logit;         // workspace [B][Hkv][cap_stride]
  uint8_t* mask;        // workspace [B][Hkv][cap_stride] (ca.mask, written here)
  int64_t cap_stride;
  double* stats;        // workspace [B][Hkv][4]
  float top_p;
  double wscale;        // fixed-point scale of the selection masses
  double scale;         // 1 / sqrt(D)
};
void launch_life(const LifeArgs& a, hipStream_t st);
// block manager: blocks for the rows the append is about to write, and the
// return of blocks past each head's count after the compaction
void launch_pool_grow(const AppendArgs& a, hipStream_t st);
void launch_pool_shrink(const PoolPaging& pg, const int32_t* count, int n_heads, hipStream_t st);

}  // namespace hk
