// C ABI of the HARD-KV decode-step library: argument validation, workspace
// layout and the launch sequences.  Declarations and contracts: hardkv.h.
#include <math.h>
#include <string.h>

#include <mutex>

#include "internal.h"

using namespace hk;

// Workspace of hardkv_step_noalloc.  Host code never names this array past
// set-up: its host-side symbol is a stand-in, not a device address; the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[HARDKV_SCRATCH_BYTES];

namespace {
hardkv_launch_observer g_observer = nullptr;
void* g_observer_user = nullptr;
}  // namespace

void hk::observe(const char* kernel, hipStream_t st) {
  if (g_observer) g_observer(kernel, (hardkv_stream_t)st, g_observer_user);
}

namespace {

constexpr int kVersion = 10900;  // 1.9.0

// Device address of `scratch` on each device, looked up on the first
// hardkv_step_noalloc call with that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return HARDKV_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
      return HARDKV_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HARDKV_OK;
}

int log2i(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

// candidates per (b, h) at most: positions [S, ctx_cap - W)
int max_aged(const hardkv_desc* d) {
  const int64_t a = (int64_t)d->ctx_cap - d->dense_window - d->sinks;
  return a > 0 ? (int)a : 0;
}

int validate(const hardkv_desc* d) {
  if (!d) return HARDKV_ERR_INVALID_ARG;
  if (d->batch < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1) return HARDKV_ERR_INVALID_ARG;
  if (d->num_q_heads % d->num_kv_heads) return HARDKV_ERR_INVALID_ARG;
  const int G = d->num_q_heads / d->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return HARDKV_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return HARDKV_ERR_UNSUPPORTED;
  if (d->dtype != HARDKV_F32 && d->dtype != HARDKV_BF16) return HARDKV_ERR_UNSUPPORTED;
  if (d->dense_window < 0 || d->chunk < 1 || d->block_size < 0 || d->ctx_cap < 1)
    return HARDKV_ERR_INVALID_ARG;
  if (d->block_size > 0) {
    if (d->block_size & (d->block_size - 1)) return HARDKV_ERR_UNSUPPORTED;
    if (d->max_blocks < 1 || (int64_t)d->max_blocks * d->block_size < d->ctx_cap)
      return HARDKV_ERR_INVALID_ARG;
  }
  if (!(d->top_p > 0.0f && d->top_p <= 1.0f)) return HARDKV_ERR_INVALID_ARG;  // NaN fails too
  if (d->sinks < 0 || (d->merge != HARDKV_MERGE_MEAN && d->merge != HARDKV_MERGE_WEIGHTED))
    return HARDKV_ERR_INVALID_ARG;
  if ((int64_t)d->dense_window + d->sinks > INT32_MAX / 2) return HARDKV_ERR_INVALID_ARG;
  if (d->packed_rows < 0) return HARDKV_ERR_INVALID_ARG;
  if (d->obs_window < 0 || d->obs_window > 64 || d->pool_radius < 0 || d->pool_radius > 512)
    return HARDKV_ERR_INVALID_ARG;
  if (d->calibration != HARDKV_CALIB_SPREAD && d->calibration != HARDKV_CALIB_ENTROPY)
    return HARDKV_ERR_INVALID_ARG;
  if (d->select_block < 0 || d->select_block > 1024 ||
      (d->select_block & (d->select_block - 1)))
    return HARDKV_ERR_INVALID_ARG;
  if (d->packed_rows > 0 &&
      (int64_t)d->batch * d->num_kv_heads * (int64_t)d->sparse_cap >= ((int64_t)1 << 31))
    return HARDKV_ERR_INVALID_ARG;
  if (d->tier_block != 0) {
    if (d->tier_block < 16 || d->tier_block > 1024 || (d->tier_block & (d->tier_block - 1)) ||
        d->tier_blocks < 1 || (int64_t)d->tier_blocks * d->tier_block >= ((int64_t)1 << 31) ||
        d->packed_rows != 0)
      return HARDKV_ERR_INVALID_ARG;
    if ((int64_t)d->batch * d->num_kv_heads > kTierMaxHeads) return HARDKV_ERR_UNSUPPORTED;
  }
  if (d->sparse_cap < 0 || d->chunk_cap < 0) return HARDKV_ERR_INVALID_ARG;
  const int A = max_aged(d);
  if (d->select_block > 0 && ceil_div(A, d->select_block) + 1 > kBlockSelMax)
    return HARDKV_ERR_UNSUPPORTED;
  if (d->sparse_cap < A) return HARDKV_ERR_CAPACITY;
  if ((int64_t)d->chunk_cap * d->chunk < A) return HARDKV_ERR_CAPACITY;
  // launch grids: the batch and the KV heads are grid dimensions of their own
  if (d->batch > 65535 || d->num_kv_heads > 65535) return HARDKV_ERR_UNSUPPORTED;
  // every element offset must fit comfortably in 63 bits
  const double elems = (double)d->batch * d->num_kv_heads *
                       ((double)d->sparse_cap + d->ctx_cap + d->chunk_cap) * d->head_dim * 8.0;
  if (elems > 4.0e18) return HARDKV_ERR_INVALID_ARG;
  return HARDKV_OK;
}

struct Layout {
  size_t q64, kmu, logit, l2, wx, stats, mask, count, kept, part, total;
  int max_tiles;
};

// queries in the observation window (0 and 1 both mean this step's only)
int window_of(const hardkv_desc* d) { return d->obs_window > 1 ? d->obs_window : 1; }

Layout layout(const hardkv_desc* d) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  const size_t B = d->batch, Hq = d->num_q_heads, Hkv = d->num_kv_heads, D = d->head_dim;
  const size_t G = Hq / Hkv, cap = d->sparse_cap;
  L.q64 = take(B * (size_t)window_of(d) * Hq * D * 8);
  L.kmu = take(B * Hkv * (D + 1) * 8);
  L.logit = take(B * Hkv * cap * 4);
  L.l2 = take(B * Hkv * cap * 4);
  L.wx = take(d->pool_radius > 0 ? B * Hkv * cap * 4 : 0);
  L.stats = take(B * Hkv * 4 * 8);
  L.mask = take(B * Hkv * cap);
  L.count = take(B * Hkv * 4);
  L.kept = take(B * Hkv * (size_t)kept_stride(d->sparse_cap) * 4);
  L.max_tiles = attn_max_tiles(d->dense_window + d->sinks, d->sparse_cap, d->chunk_cap);
  L.part = take(B * Hkv * (size_t)L.max_tiles * G * (D + 2) * 4);
  L.total = off;
  return L;
}

Rows cache_rows(const hardkv_desc* d, const void* base, const int32_t* table) {
  Rows r{};
  r.base = (const char*)base;
  r.table = d->block_size > 0 ? table : nullptr;
  r.region = d->ctx_cap;
  r.hkv = d->num_kv_heads;
  r.lbs = d->block_size > 0 ? log2i(d->block_size) : 0;
  r.max_blocks = d->max_blocks;
  r.row_bytes = d->head_dim * (d->dtype == HARDKV_F32 ? 4 : 2);
  return r;
}

// candidate rows: position t of the candidates is cache position sinks + t
Rows cand_rows(const hardkv_desc* d, const void* base, const int32_t* table) {
  Rows r = cache_rows(d, base, table);
  r.off = d->sinks;
  return r;
}

Rows region_rows(const hardkv_desc* d, const void* base, int64_t region) {
  Rows r{};
  r.base = (const char*)base;
  r.table = nullptr;
  r.region = region;
  r.hkv = d->num_kv_heads;
  r.row_bytes = d->head_dim * (d->dtype == HARDKV_F32 ? 4 : 2);
  return r;
}

// block manager of the rewritten tier
int tier_maxb(const hardkv_desc* d) { return ceil_div(d->sparse_cap, d->tier_block); }
TierBlocks tier_blocks(const hardkv_desc* d, const hardkv_tiers* t) {
  TierBlocks b{};
  b.table = t->table;
  b.held = t->held;
  b.free_ids = t->free_ids;
  b.free_top = t->free_top;
  b.lbs = log2i(d->tier_block);
  b.maxb = tier_maxb(d);
  b.nblocks = d->tier_blocks;
  return b;
}
// rows of the rewritten tier under its block manager: head (b, h) uses
// table row b * Hkv + h, blocks of tier_block rows of one head each
Rows tier_rows(const hardkv_desc* d, const void* base, const int32_t* table) {
  Rows r{};
  r.base = (const char*)base;
  r.table = table;
  r.region = 0;
  r.hkv = 1;
  r.lbs = log2i(d->tier_block);
  r.max_blocks = tier_maxb(d);
  r.row_bytes = d->head_dim * (d->dtype == HARDKV_F32 ? 4 : 2);
  r.headtab = d->num_kv_heads;
  return r;
}

Cand aged_cand(const hardkv_desc* d, const int32_t* ctx_len) {
  return Cand{ctx_len, nullptr, d->dense_window, d->ctx_cap, max_aged(d), d->num_kv_heads,
              d->sinks};
}

// Drops an error left by an earlier, unrelated launch on this thread, so
// launched() reports only this call's launches.
void clear_launch_error() { (void)hipGetLastError(); }

int launched() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? HARDKV_OK : HARDKV_ERR_HIP;
}

// ---------------------------------------------------------- launch steps --
// q_ready: an earlier launch of the same step has widened q into q64.
void do_score(const hardkv_desc* d, const Layout& L, char* ws, const void* q, const void* q_hist,
              const Rows& rows, const Cand& cand, int max_cand, const int8_t* metric,
              float* logit, float* l2, hipStream_t st, bool q_ready = false) {
  ScoreArgs a{};
  a.q_ready = q_ready;
  a.dtype = d->dtype;
  a.D = d->head_dim;
  a.G = d->num_q_heads / d->num_kv_heads;
  a.B = d->batch;
  a.hq = d->num_q_heads;
  a.hkv = d->num_kv_heads;
  a.q = q;
  a.q_hist = q_hist;
  a.window = window_of(d);
  a.radius = d->pool_radius;
  a.wx = (float*)(ws + L.wx);
  a.q64 = (double*)(ws + L.q64);
  a.kmu = (double*)(ws + L.kmu);
  a.rows = rows;
  a.cand = cand;
  a.max_cand = max_cand;
  a.metric = metric;
  a.logit = logit;
  a.l2 = l2;
  a.cap_stride = d->sparse_cap;
  a.scale = 1.0 / sqrt((double)d->head_dim);
  launch_score(a, st);
}

SelectArgs select_args(const hardkv_desc* d, const Cand& cand, const int8_t* metric,
                       const float* logit, const float* l2, double* stats, uint8_t* mask,
                       int32_t* count) {
  SelectArgs a{};
  a.B = d->batch;
  a.hkv = d->num_kv_heads;
  a.cand = cand;
  a.metric = metric;
  a.logit = logit;
  a.l2 = l2;
  a.cap_stride = d->sparse_cap;
  a.stats = stats;
  a.top_p = d->top_p;
  a.mask = mask;
  a.count = count;
  a.mode = nullptr;
  a.policy = hardkv_policy{HARDKV_POLICY_REWRITE, 1, 0, 0};
  a.calib = d->calibration;
  a.block = d->select_block;
  return a;
}

CompactArgs compact_args(const hardkv_desc* d, const Layout& L, char* ws, const Rows& kr,
                         const Rows& vr, const Cand& cand, int max_cand, const uint8_t* mask,
                         const hardkv_tiers* t) {
  CompactArgs a{};
  a.dtype = d->dtype;
  a.D = d->head_dim;
  a.B = d->batch;
  a.hkv = d->num_kv_heads;
  a.C = d->chunk;
  a.krows = kr;
  a.vrows = vr;
  a.cand = cand;
  a.max_cand = max_cand;
  a.mask = mask;
  a.cap_stride = d->sparse_cap;
  a.out_k = (char*)t->k;
  a.out_v = (char*)t->v;
  a.out_pos = t->pos;
  a.out_count = t->count;
  a.ksum = t->ksum;
  a.vsum = t->vsum;
  a.ccount = t->ccount;
  a.chunk_stride = d->chunk_cap;
  a.mode = t->mode;
  a.offset = d->packed_rows > 0 ? t->offset : nullptr;
  if (d->tier_block > 0) {
    a.tier_table = t->table;
    a.tier_lbs = log2i(d->tier_block);
    a.tier_maxb = tier_maxb(d);
    a.tier_nblocks = d->tier_blocks;
  }
  a.pos_off = d->sinks;
  a.merge = d->merge;
  a.G = d->num_q_heads / d->num_kv_heads;
  a.hq = d->num_q_heads;
  a.q = nullptr;
  a.part = (float*)(ws + L.part);
  a.max_tiles = L.max_tiles;
  a.scale = (float)(1.0 / sqrt((double)d->head_dim));
  return a;
}

AttnArgs attn_args(const hardkv_desc* d, const Layout& L, char* ws, const void* q,
                   const hardkv_tiers* t, float* out) {
  AttnArgs a{};
  a.dtype = d->dtype;
  a.D = d->head_dim;
  a.G = d->num_q_heads / d->num_kv_heads;
  a.B = d->batch;
  a.hkv = d->num_kv_heads;
  a.hq = d->num_q_heads;
  a.q = q;
  a.ctx_cap = d->ctx_cap;
  a.W = d->dense_window;
  a.sinks = d->sinks;
  if (d->tier_block > 0) {
    a.sk = tier_rows(d, t->k, t->table);
    a.sv = tier_rows(d, t->v, t->table);
  } else {
    a.sk = region_rows(d, t->k, d->sparse_cap);
    a.sv = region_rows(d, t->v, d->sparse_cap);
  }
  a.count = t->count;
  a.sparse_cap = d->sparse_cap;
  a.mode = t->mode;
  a.pos = t->pos;
  a.offset = d->packed_rows > 0 ? t->offset : nullptr;
  a.ksum = t->ksum;
  a.vsum = t->vsum;
  a.ccount = t->ccount;
  a.chunk_cap = d->chunk_cap;
  a.C = d->chunk;
  a.part = (float*)(ws + L.part);
  a.max_tiles = L.max_tiles;
  a.out = out;
  a.scale = 1.0 / sqrt((double)d->head_dim);
  a.fused_tt = 0;
  return a;
}

bool tiers_ok(const hardkv_tiers* t) {
  return t && t->k && t->v && t->pos && t->count && t->ksum && t->vsum && t->ccount;
}
// ... and, for a packed rewritten tier, the offsets and the per-head modes;
// under the tier's block manager, its state and the per-head modes
bool tiers_ok(const hardkv_desc* d, const hardkv_tiers* t) {
  return tiers_ok(t) && (d->packed_rows == 0 || (t->mode && t->offset)) &&
         (d->tier_block == 0 ||
          (t->mode && t->table && t->held && t->free_ids && t->free_top));
}
bool cache_ok(const hardkv_desc* d, const hardkv_cache* c) {
  return c && c->k && c->v && c->ctx_len && (d->block_size == 0 || c->block_table);
}
// ... and, when the window metric looks back, the earlier queries
bool scored_cache_ok(const hardkv_desc* d, const hardkv_cache* c) {
  return cache_ok(d, c) && (window_of(d) == 1 || c->q_hist);
}

bool policy_ok(const hardkv_policy* p) {
  return p && (p->kind == HARDKV_POLICY_REWRITE || p->kind == HARDKV_POLICY_SPARSE ||
               p->kind == HARDKV_POLICY_MTI) &&
         p->horizon >= 1;
}

int common_checks(const hardkv_desc* d, void* ws, size_t ws_bytes) {
  const int rc = validate(d);
  if (rc != HARDKV_OK) return rc;
  if (!ws || ws_bytes < layout(d).total) return HARDKV_ERR_WORKSPACE;
  return HARDKV_OK;
}

// score -> calibrate + select (+ plan) -> compact (+ attention over the kept
// rows) -> attention.  Each head's choice goes to tiers->mode when that is
// given.
void run_step(const hardkv_desc* d, const hardkv_policy* policy, const void* q,
              const hardkv_cache* cache, const int8_t* metric, const hardkv_tiers* tiers,
              float* out, void* ws, hipStream_t st) {
  const Layout L = layout(d);
  char* w = (char*)ws;
  const hardkv_tiers& t = *tiers;
  const Rows kr = cand_rows(d, cache->k, cache->block_table);
  const Rows vr = cand_rows(d, cache->v, cache->block_table);
  const Cand cand = aged_cand(d, cache->ctx_len);
  float* logit = (float*)(w + L.logit);
  float* l2 = (float*)(w + L.l2);
  double* stats = (double*)(w + L.stats);
  uint8_t* mask = (uint8_t*)(w + L.mask);
  int32_t* count = (int32_t*)(w + L.count);
  clear_launch_error();
  do_score(d, L, w, q, cache->q_hist, kr, cand, max_aged(d), metric, logit, l2, st);
  SelectArgs sa = select_args(d, cand, metric, logit, l2, stats, mask, count);
  sa.mode = t.mode;
  sa.policy = *policy;
  if (d->select_block > 0) {
    launch_calibrate(sa, st);
    launch_blocksel(sa, st);
  } else {
    // the select kernels count the kept tokens of every block of candidates
    // for the compaction tiles' offsets (whole blocks per tile)
    if (compact_fusable(d->chunk) &&
        compact_tile(d->chunk, max_aged(d)) % kKeptBlk == 0 &&
        kept_stride(max_aged(d)) <= kKeptMaxBlks) {
      sa.kept_blk = (int32_t*)(w + L.kept);
      sa.kept_stride = kept_stride(max_aged(d));
    }
    if (calsel_fits(max_aged(d))) {
      launch_calsel(sa, max_aged(d), st);
    } else {
      sa.z_from_select = true;
      launch_calibrate(sa, st);
      launch_select(sa, st);
    }
  }
  if (d->packed_rows > 0)
    launch_pack(d->batch * d->num_kv_heads, count, max_aged(d), t.mode, t.offset,
                d->packed_rows, st);
  if (d->tier_block > 0)
    launch_tier_alloc(tier_blocks(d, &t), d->batch * d->num_kv_heads, count, max_aged(d), t.mode,
                      st);
  CompactArgs ca = compact_args(d, L, w, kr, vr, cand, max_aged(d), mask, &t);
  ca.kept_blk = sa.kept_blk;
  ca.kept_stride = sa.kept_stride;
  ca.metric = metric;
  ca.logit = logit;
  ca.l2 = l2;
  ca.stats = stats;
  AttnArgs a = attn_args(d, L, w, q, &t, out);
  a.dk = cache_rows(d, cache->k, cache->block_table);
  a.dv = cache_rows(d, cache->v, cache->block_table);
  a.ctx_len = cache->ctx_len;
  a.ring = false;
  if (compact_fusable(d->chunk)) {
    // attention over the kept rows happens inside the compaction pass; the
    // attention launch then covers the dense and condensed tiers only
    ca.q = q;
    launch_compact_attn(ca, st);
    a.fused_tt = compact_tile(d->chunk, max_aged(d));
  } else {
    launch_compact(ca, st);
  }
  launch_attn(a, st);
}

}  // namespace

extern "C" {

int hardkv_version(void) { return kVersion; }

const char* hardkv_strerror(int code) {
  switch (code) {
    case HARDKV_OK: return "ok";
    case HARDKV_ERR_INVALID_ARG: return "invalid argument";
    case HARDKV_ERR_UNSUPPORTED: return "unsupported head_dim, dtype or GQA group size";
    case HARDKV_ERR_CAPACITY: return "sparse_cap or chunk_cap below the aged capacity";
    case HARDKV_ERR_WORKSPACE: return "workspace missing or too small";
    case HARDKV_ERR_HIP: return "HIP launch failure";
    default: return "unknown error";
  }
}

int hardkv_validate(const hardkv_desc* desc) { return validate(desc); }

void hardkv_set_launch_observer(hardkv_launch_observer fn, void* user) {
  g_observer = fn;
  g_observer_user = user;
}

size_t hardkv_workspace_size(const hardkv_desc* desc) {
  if (validate(desc) != HARDKV_OK) return 0;
  return layout(desc).total;
}

int hardkv_score(const hardkv_desc* d, const void* q, const hardkv_cache* cache,
                 const int8_t* metric, float* logit, float* l2, void* ws, size_t ws_bytes,
                 hardkv_stream_t stream) {
  int rc = common_checks(d, ws, ws_bytes);
  if (rc) return rc;
  if (!q || !scored_cache_ok(d, cache) || !logit || (metric && !l2)) return HARDKV_ERR_INVALID_ARG;
  const Layout L = layout(d);
  clear_launch_error();
  do_score(d, L, (char*)ws, q, cache->q_hist, cand_rows(d, cache->k, cache->block_table),
           aged_cand(d, cache->ctx_len), max_aged(d), metric, logit, l2, (hipStream_t)stream);
  return launched();
}

int hardkv_calibrate(const hardkv_desc* d, const int32_t* ctx_len, const int8_t* metric,
                     const float* logit, const float* l2, double* stats, void* ws,
                     size_t ws_bytes, hardkv_stream_t stream) {
  int rc = common_checks(d, ws, ws_bytes);
  if (rc) return rc;
  if (!ctx_len || !logit || !stats || (metric && !l2)) return HARDKV_ERR_INVALID_ARG;
  clear_launch_error();
  launch_calibrate(select_args(d, aged_cand(d, ctx_len), metric, logit, l2, stats, nullptr, nullptr),
                   (hipStream_t)stream);
  return launched();
}

int hardkv_topp_select(const hardkv_desc* d, const int32_t* ctx_len, const int8_t* metric,
                       const float* logit, const float* l2, const double* stats, uint8_t* mask,
                       int32_t* count, void* ws, size_t ws_bytes, hardkv_stream_t stream) {
  int rc = common_checks(d, ws, ws_bytes);
  if (rc) return rc;
  if (!ctx_len || !logit || !stats || !mask || !count || (metric && !l2))
    return HARDKV_ERR_INVALID_ARG;
  clear_launch_error();
  const SelectArgs sa = select_args(d, aged_cand(d, ctx_len), metric, logit, l2, (double*)stats,
                                    mask, count);
  if (d->select_block > 0)
    launch_blocksel(sa, (hipStream_t)stream);
  else
    launch_select(sa, (hipStream_t)stream);
  return launched();
}

int hardkv_compact_scored(const hardkv_desc* d, const hardkv_cache* cache,
                          const int8_t* metric, const float* logit, const float* l2,
                          const double* stats, const uint8_t* mask, const hardkv_tiers* out,
                          void* ws, size_t ws_bytes, hardkv_stream_t stream) {
  int rc = common_checks(d, ws, ws_bytes);
  if (rc) return rc;
  if (!cache_ok(d, cache) || !mask || !tiers_ok(d, out)) return HARDKV_ERR_INVALID_ARG;
  if (d->merge == HARDKV_MERGE_WEIGHTED && (!logit || !stats || (metric && !l2)))
    return HARDKV_ERR_INVALID_ARG;
  const Layout L = layout(d);
  CompactArgs a = compact_args(d, L, (char*)ws, cand_rows(d, cache->k, cache->block_table),
                               cand_rows(d, cache->v, cache->block_table),
                               aged_cand(d, cache->ctx_len), max_aged(d), mask, out);
  a.metric = metric;
  a.logit = logit;
  a.l2 = l2;
  a.stats = stats;
  clear_launch_error();
  launch_compact(a, (hipStream_t)stream);
  return launched();
}

int hardkv_compact(const hardkv_desc* d, const hardkv_cache* cache, const uint8_t* mask,
                   const hardkv_tiers* out, void* ws, size_t ws_bytes, hardkv_stream_t stream) {
  const int rc = validate(d);
  if (rc) return rc;
  if (d->merge != HARDKV_MERGE_MEAN) return HARDKV_ERR_INVALID_ARG;
  return hardkv_compact_scored(d, cache, nullptr, nullptr, nullptr, nullptr, mask, out, ws,
                               ws_bytes, stream);
}

int hardkv_decode_attn(const hardkv_desc* d, const void* q, const hardkv_cache* cache,
                       const hardkv_tiers* tiers, float* out, void* ws, size_t ws_bytes,
                       hardkv_stream_t stream) {
  int rc = common_checks(d, ws, ws_bytes);
  if (rc) return rc;
  if (!q || !cache_ok(d, cache) || !tiers_ok(d, tiers) || !out) return HARDKV_ERR_INVALID_ARG;
  const Layout L = layout(d);
  AttnArgs a = attn_args(d, L, (char*)ws, q, tiers, out);
  a.dk = cache_rows(d, cache->k, cache->block_table);
  a.dv = cache_rows(d, cache->v, cache->block_table);
  a.ctx_len = cache->ctx_len;
  a.ring = false;
  clear_launch_error();
  launch_attn(a, (hipStream_t)stream);
  return launched();
}

int hardkv_plan(const hardkv_desc* d, const hardkv_policy* policy, const int32_t* ctx_len,
                const int32_t* count, uint8_t* mode, hardkv_stream_t stream) {
  const int rc = validate(d);
  if (rc) return rc;
  if (!policy_ok(policy) || !ctx_len || !count || !mode) return HARDKV_ERR_INVALID_ARG;
  SelectArgs a = select_args(d, aged_cand(d, ctx_len), nullptr, nullptr, nullptr, nullptr,
                             nullptr, (int32_t*)count);
  a.mode = mode;
  a.policy = *policy;
  clear_launch_error();
  launch_plan(a, (hipStream_t)stream);
  return launched();
}

int hardkv_pack(const hardkv_desc* d, const int32_t* count, const hardkv_tiers* tiers,
                hardkv_stream_t stream) {
  const int rc = validate(d);
  if (rc) return rc;
  if (d->packed_rows == 0 || !count || !tiers || !tiers->mode || !tiers->offset)
    return HARDKV_ERR_INVALID_ARG;
  clear_launch_error();
  launch_pack(d->batch * d->num_kv_heads, count, max_aged(d), tiers->mode, tiers->offset,
              d->packed_rows, (hipStream_t)stream);
  return launched();
}

int hardkv_tier_init(const hardkv_desc* d, const hardkv_tiers* tiers, hardkv_stream_t stream) {
  const int rc = validate(d);
  if (rc) return rc;
  if (d->tier_block == 0 || !tiers || !tiers->table || !tiers->held || !tiers->free_ids ||
      !tiers->free_top)
    return HARDKV_ERR_INVALID_ARG;
  clear_launch_error();
  launch_tier_init(tier_blocks(d, tiers), d->batch * d->num_kv_heads, (hipStream_t)stream);
  return launched();
}

int hardkv_tier_alloc(const hardkv_desc* d, const int32_t* count, const hardkv_tiers* tiers,
                      hardkv_stream_t stream) {
  const int rc = validate(d);
  if (rc) return rc;
  if (d->tier_block == 0 || !count || !tiers || !tiers->mode || !tiers->table || !tiers->held ||
      !tiers->free_ids || !tiers->free_top)
    return HARDKV_ERR_INVALID_ARG;
  clear_launch_error();
  launch_tier_alloc(tier_blocks(d, tiers), d->batch * d->num_kv_heads, count, max_aged(d),
                    tiers->mode, (hipStream_t)stream);
  return launched();
}

int hardkv_step(const hardkv_desc* d, const void* q, const hardkv_cache* cache,
                const int8_t* metric, const hardkv_tiers* tiers, float* out, void* ws,
                size_t ws_bytes, hardkv_stream_t stream) {
  int rc = common_checks(d, ws, ws_bytes);
  if (rc) return rc;
  if (!q || !scored_cache_ok(d, cache) || !tiers_ok(d, tiers) || !out)
    return HARDKV_ERR_INVALID_ARG;
  const hardkv_policy rewrite_all{HARDKV_POLICY_REWRITE, 1, 0, 0};
  run_step(d, &rewrite_all, q, cache, metric, tiers, out, ws, (hipStream_t)stream);
  return launched();
}

int hardkv_step_noalloc(const hardkv_desc* d, const void* q, const hardkv_cache* cache,
                        const int8_t* metric, const hardkv_tiers* tiers, float* out,
                        hardkv_stream_t stream) {
  const int rc = validate(d);
  if (rc) return rc;
  if (!q || !scored_cache_ok(d, cache) || !tiers_ok(d, tiers) || !out)
    return HARDKV_ERR_INVALID_ARG;
  if (layout(d).total > HARDKV_SCRATCH_BYTES) return HARDKV_ERR_WORKSPACE;
  void* ws = nullptr;
  const int src = scratch_of_current_device(&ws);
  if (src) return src;
  return hardkv_step(d, q, cache, metric, tiers, out, ws, HARDKV_SCRATCH_BYTES, stream);
}

int hardkv_step_policy(const hardkv_desc* d, const hardkv_policy* policy, const void* q,
                       const hardkv_cache* cache, const int8_t* metric,
                       const hardkv_tiers* tiers, float* out, void* ws, size_t ws_bytes,
                       hardkv_stream_t stream) {
  int rc = common_checks(d, ws, ws_bytes);
  if (rc) return rc;
  if (!policy_ok(policy) || !q || !scored_cache_ok(d, cache) || !tiers_ok(d, tiers) || !tiers->mode ||
      !out)
    return HARDKV_ERR_INVALID_ARG;
  run_step(d, policy, q, cache, metric, tiers, out, ws, (hipStream_t)stream);
  return launched();
}

int hardkv_step_inplace(const hardkv_desc* d, const void* q, const void* k_new,
                        const void* v_new, const int8_t* metric, const hardkv_state* s,
                        float* out, void* ws, size_t ws_bytes, hardkv_stream_t stream) {
  int rc = common_checks(d, ws, ws_bytes);
  if (rc) return rc;
  if (d->block_size != 0 || d->dense_window < 1 || d->sinks != 0 ||
      d->merge != HARDKV_MERGE_MEAN || d->packed_rows != 0 || window_of(d) != 1 ||
      d->pool_radius != 0 || d->calibration != HARDKV_CALIB_SPREAD || d->select_block != 0 ||
      d->tier_block != 0)
    return HARDKV_ERR_INVALID_ARG;
  if (!q || !k_new || !v_new || !s || !s->ring_k || !s->ring_v || !s->seq_len ||
      !tiers_ok(&s->tiers) || s->tiers.mode || !out)
    return HARDKV_ERR_INVALID_ARG;
  // head-wise block manager of the pool
  PoolPaging pg{};
  if (s->pool_block != 0) {
    const int bs = s->pool_block;
    if (bs < 1 || bs > 4096 || (bs & (bs - 1)) || s->pool_blocks < 1 || !s->pool_table ||
        !s->free_ids || !s->free_top)
      return HARDKV_ERR_INVALID_ARG;
    pg.lbs = log2i(bs);
    pg.maxb = ceil_div(d->sparse_cap, bs);
    pg.nblocks = s->pool_blocks;
    if ((int64_t)d->batch * d->num_kv_heads * pg.maxb >= ((int64_t)1 << 31) ||
        (int64_t)s->pool_blocks * bs >= ((int64_t)1 << 31))
      return HARDKV_ERR_INVALID_ARG;
    pg.table = s->pool_table;
    pg.free_ids = s->free_ids;
    pg.free_top = s->free_top;
  }
  const Layout L = layout(d);
  char* w = (char*)ws;
  hipStream_t st = (hipStream_t)stream;
  const hardkv_tiers* t = &s->tiers;
  clear_launch_error();

  AppendArgs ap{};
  ap.dtype = d->dtype;
  ap.D = d->head_dim;
  ap.B = d->batch;
  ap.hkv = d->num_kv_heads;
  ap.W = d->dense_window;
  ap.sparse_cap = d->sparse_cap;
  ap.ctx_cap = d->ctx_cap;
  ap.k_new = k_new;
  ap.v_new = v_new;
  ap.ring_k = (char*)s->ring_k;
  ap.ring_v = (char*)s->ring_v;
  ap.pool_k = (char*)t->k;
  ap.pool_v = (char*)t->v;
  ap.pool_pos = t->pos;
  ap.pool_count = t->count;
  ap.seq_len = s->seq_len;
  ap.pg = pg;
  ap.ksum = t->ksum;
  ap.vsum = t->vsum;
  ap.ccount = t->ccount;
  ap.C = d->chunk;
  ap.chunk_cap = d->chunk_cap;
  ap.q = q;  // the append also widens this step's queries for the score
  ap.q64 = (double*)(w + L.q64);
  ap.hq = d->num_q_heads;
  const Cand cand{nullptr, t->count, d->dense_window, d->ctx_cap, d->sparse_cap,
                  d->num_kv_heads};
  float* logit = (float*)(w + L.logit);
  float* l2 = (float*)(w + L.l2);
  double* stats = (double*)(w + L.stats);
  uint8_t* mask = (uint8_t*)(w + L.mask);
  int32_t* count = (int32_t*)(w + L.count);
  Rows pk = region_rows(d, t->k, d->sparse_cap);
  Rows pv = region_rows(d, t->v, d->sparse_cap);
  if (!metric && !pg.table) {
    // every head on the logit, per-head regions: append, score, select and
    // compaction of each head in one workgroup
    LifeArgs la{};
    la.ap = ap;
    la.ap.q64 = nullptr;
    la.ca = compact_args(d, L, w, pk, pv, cand, d->sparse_cap, mask, t);
    la.q = q;
    la.logit = logit;
    la.mask = mask;
    la.cap_stride = d->sparse_cap;
    la.stats = stats;
    la.top_p = d->top_p;
    la.wscale = mass_scale(d->sparse_cap);
    la.scale = 1.0 / sqrt((double)d->head_dim);
    launch_life(la, st);
  } else {
    if (pg.table) launch_pool_grow(ap, st);
    launch_append(ap, st);
    if (pg.table) {
      // pool rows through per-head block tables (one head per block)
      for (Rows* r : {&pk, &pv}) {
        r->table = pg.table;
        r->hkv = 1;
        r->lbs = pg.lbs;
        r->max_blocks = pg.maxb;
        r->headtab = d->num_kv_heads;
      }
    }
    do_score(d, L, w, q, nullptr, pk, cand, d->sparse_cap, metric, logit, l2, st, true);
    SelectArgs sa = select_args(d, cand, metric, logit, l2, stats, mask, count);
    sa.z_from_select = true;
    // separate launches: after the first steps the pools are a few hundred
    // tokens, where the fused kernel's one-workgroup-per-CU footprint (scores
    // in registers, weights in LDS) costs more than the two light kernels
    launch_calibrate(sa, st);
    launch_select(sa, st);
    CompactArgs ca = compact_args(d, L, w, pk, pv, cand, d->sparse_cap, mask, t);
    ca.pg = pg;
    launch_compact_inplace(ca, st);
    if (pg.table) launch_pool_shrink(pg, t->count, d->batch * d->num_kv_heads, st);
  }
  AttnArgs a = attn_args(d, L, w, q, t, out);
  if (pg.table) {
    a.sk = pk;
    a.sv = pv;
  }
  a.dk = region_rows(d, s->ring_k, d->dense_window);
  a.dv = region_rows(d, s->ring_v, d->dense_window);
  a.ctx_len = nullptr;  // the ring's tiers do not depend on the length
  a.ring = true;
  a.advance = s->seq_len;  // the merge, the step's last kernel, moves every sequence on
  launch_attn(a, st);
  return launched();
}

}  // extern "C"
