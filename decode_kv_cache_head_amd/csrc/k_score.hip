// Importance scores of aged tokens (HARD-KV, gist.science technical summary,
// section 2.B "Goal": max-pooled logits; key-norm metric alongside).
//
// Observation-window heads (section 2.B: SnapKV-style strategies) also take
// the max over the earlier queries of the window, then a max-pooling pass
// over neighbouring positions (k_pool).
//
// HBM-bound stream over the aged keys.  Each workgroup takes up to four
// consecutive 256-token tiles of one (b, h); a tile is staged into LDS with
// coalesced 16-byte loads, and the next tile's loads are issued before the
// current one is scored, so HBM traffic overlaps the arithmetic.  Every lane
// scores one token: the G query rows of the head's GQA group are read as
// float64 from wave-uniform addresses (scalar loads, SGPR operands), the
// token's key is widened exactly to float64 and the G dot products are
// accumulated in float64, so the only rounding the ranking key sees is the
// final fl32().
#include "internal.h"

namespace hk {

// q64[b][i][:] = this step's query (i = 0) or the i-th previous one (q_hist)
template <typename T>
__global__ __launch_bounds__(256) void k_q_to_f64(const T* __restrict__ q,
                                                   const T* __restrict__ q_hist, int window,
                                                   int64_t per_q, double* __restrict__ q64,
                                                   int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int64_t b = i / (window * per_q), rest = i % (window * per_q);
  const int64_t wi = rest / per_q, e = rest % per_q;
  const T* src = wi == 0 ? q + b * per_q + e : q_hist + (b * (window - 1) + wi - 1) * per_q + e;
  q64[i] = (double)Elt<T>::load1(src);
}

constexpr int kScoreTile = 256;
constexpr int kScoreTiles = 4;  // tiles per workgroup

// RELOAD: read the row again from LDS (volatile) rather than keep its
// float64 widening live across calls -- the window loop scores one row
// against several queries.
template <typename T, int D, int G, bool L2, bool RELOAD = false>
__device__ inline void score_row(const unsigned char* row, const double* __restrict__ qg,
                                 double (&acc)[G], double& ss) {
  constexpr int RB = D * (int)sizeof(T);
  constexpr int CPR = RB / 16;
  constexpr int EPC = Elt<T>::kPer16;
#pragma unroll
  for (int c = 0; c < CPR; ++c) {
    v4u raw;
    if constexpr (RELOAD)
      raw = *(const volatile v4u*)(row + c * 16);
    else
      raw = *(const v4u*)(row + c * 16);
    float f[EPC];
    Elt<T>::unpack(raw, f);
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      const double kd = (double)f[e];
#pragma unroll
      for (int g = 0; g < G; ++g) acc[g] = fma(qg[g * D + c * EPC + e], kd, acc[g]);
      if (L2) ss = fma(kd, kd, ss);
    }
  }
}

// Coalesced 16-byte loads of a 256-token tile; rows past the end re-read the
// last valid row (always in bounds, their scores are never written).
template <int CPR, bool P>
__device__ __forceinline__ void load_tile(v4u (&buf)[CPR], const Rows& rows, int b, int h,
                                          int t0, int n, int tid) {
#pragma unroll
  for (int j = 0; j < CPR; ++j) {
    const int idx = j * kScoreTile + tid;
    const int r = idx / CPR, c = idx % CPR;
    buf[j] = *(const v4u*)(rows.template row<P>(b, h, min(t0 + r, n - 1)) + c * 16);
  }
}

template <int CPR, int PAD>
__device__ __forceinline__ void store_tile(const v4u (&buf)[CPR], unsigned char* lds, int tid) {
#pragma unroll
  for (int j = 0; j < CPR; ++j) {
    const int idx = j * kScoreTile + tid;
    const int r = idx / CPR, c = idx % CPR;
    *(v4u*)(lds + r * PAD + c * 16) = buf[j];
  }
}

// One lane scores token t from its LDS row.  Window heads (WIN: more than
// one query in the window) also take the max over the earlier queries,
// whose float64 rows follow at a stride of qstride.
struct WinOut {
  bool on;           // this head uses the window metric
  float* dst;        // window metric (before pooling) or the pooled array itself
  int window;
  int64_t qstride;   // elements between consecutive window queries in q64
};

template <typename T, int D, int G, bool WIN>
__device__ __forceinline__ void score_lane(const unsigned char* row, const double* __restrict__ qg,
                                           bool is_l2, const WinOut& wo, int t, int n,
                                           float* __restrict__ logit, float* __restrict__ l2,
                                           int64_t obase, double scale) {
  double acc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = 0.0;
  double ss = 0.0;
  if (is_l2)
    score_row<T, D, G, true>(row, qg, acc, ss);
  else
    score_row<T, D, G, false>(row, qg, acc, ss);
  double mx = acc[0];
#pragma unroll
  for (int g = 1; g < G; ++g) mx = fmax(mx, acc[g]);
  double mw = mx;
  if constexpr (WIN) {
    if (wo.on) {
#pragma unroll 1
      for (int i = 1; i < wo.window; ++i) {
#pragma unroll
        for (int g = 0; g < G; ++g) acc[g] = 0.0;
        score_row<T, D, G, false, true>(row, qg + i * wo.qstride, acc, ss);
#pragma unroll
        for (int g = 0; g < G; ++g) mw = fmax(mw, acc[g]);
      }
    }
  }
  if (t < n) {
    logit[obase + t] = (float)(mx * scale);
    if (is_l2) l2[obase + t] = (float)sqrt(ss);
    if (wo.on) wo.dst[obase + t] = (float)(mw * scale);
  }
}

template <typename T, int D, int G, bool P, bool WIN>
__global__ __launch_bounds__(256) void k_score(const double* __restrict__ q64, int hq, Rows rows,
                                               Cand cand, const int8_t* __restrict__ metric,
                                               float* __restrict__ logit, float* __restrict__ l2,
                                               float* __restrict__ wdst, int window,
                                               int64_t cap_stride, double scale) {
  constexpr int RB = D * (int)sizeof(T);
  constexpr int CPR = RB / 16;
  constexpr int PAD = RB + 16;  // keeps per-lane row reads conflict free
  __shared__ __attribute__((aligned(16))) unsigned char lds[kScoreTile * PAD];
  const int b = blockIdx.z, h = blockIdx.y, hkv = gridDim.y;
  const int n = cand.n(b, h);
  const int tid = threadIdx.x;
  // this workgroup's tiles: kScoreTiles consecutive 256-token tiles
  const int tfirst = blockIdx.x * kScoreTiles;
  const int ntiles = min(kScoreTiles, (n + kScoreTile - 1) / kScoreTile - tfirst);
  if (ntiles <= 0) return;
  const double* __restrict__ qg = q64 + ((int64_t)b * window * hq + (int64_t)h * G) * D;
  const bool is_l2 = metric != nullptr && metric[h] == HARDKV_METRIC_L2;
  const WinOut wo{metric != nullptr && metric[h] == HARDKV_METRIC_WINDOW, wdst, window,
                  (int64_t)hq * D};
  const int64_t obase = ((int64_t)b * hkv + h) * cap_stride;

  v4u buf[CPR];
  load_tile<CPR, P>(buf, rows, b, h, tfirst * kScoreTile, n, tid);
  // steady state: the next tile's loads are in flight while this one is scored
  for (int tile = 0; tile + 1 < ntiles; ++tile) {
    store_tile<CPR, PAD>(buf, lds, tid);
    __syncthreads();
    load_tile<CPR, P>(buf, rows, b, h, (tfirst + tile + 1) * kScoreTile, n, tid);
    score_lane<T, D, G, WIN>(lds + tid * PAD, qg, is_l2, wo, (tfirst + tile) * kScoreTile + tid,
                             n, logit, l2, obase, scale);
    __syncthreads();
  }
  store_tile<CPR, PAD>(buf, lds, tid);
  __syncthreads();
  score_lane<T, D, G, WIN>(lds + tid * PAD, qg, is_l2, wo, (tfirst + ntiles - 1) * kScoreTile + tid,
                           n, logit, l2, obase, scale);
}

// Max-pooling of the window metric over positions [t - r, t + r] inside the
// candidates, for window heads: a 1024-token tile plus r on each side in
// LDS, then doubling passes (M_{2p}[i] = max(M_p[i], M_p[i + p])) and one
// query of two overlapping power-of-two windows per token.  Exact (max).
constexpr int kPoolTile = 1024;
constexpr int kPoolMaxR = 512;

__global__ __launch_bounds__(256) void k_pool(Cand cand, const int8_t* __restrict__ metric,
                                              const float* __restrict__ src,
                                              float* __restrict__ dst, int64_t cap_stride,
                                              int r) {
  __shared__ float s_a[kPoolTile + 2 * kPoolMaxR], s_b[kPoolTile + 2 * kPoolMaxR];
  const int b = blockIdx.z, h = blockIdx.y, hkv = gridDim.y, tid = threadIdx.x;
  if (metric == nullptr || metric[h] != HARDKV_METRIC_WINDOW) return;
  const int n = cand.n(b, h);
  const int t0 = blockIdx.x * kPoolTile;
  if (t0 >= n) return;
  const int64_t base = ((int64_t)b * hkv + h) * cap_stride;
  const int L = kPoolTile + 2 * r;  // s_a[i] holds position t0 - r + i
  for (int i = tid; i < L; i += 256) {
    const int t = t0 - r + i;
    s_a[i] = (t >= 0 && t < n) ? src[base + t] : -INFINITY;
  }
  __syncthreads();
  int K = 1;
  float* cur = s_a;
  float* nxt = s_b;
  while (2 * K <= 2 * r + 1) {
    for (int i = tid; i < L; i += 256) nxt[i] = i + K < L ? fmaxf(cur[i], cur[i + K]) : cur[i];
    __syncthreads();
    float* tmp = cur;
    cur = nxt;
    nxt = tmp;
    K *= 2;
  }
  // cur[i] = max over positions [t0 - r + i, t0 - r + i + K); token j needs
  // [j - r, j + r] = windows starting at j - r and j + r + 1 - K
  for (int j = tid; j < kPoolTile; j += 256) {
    const int t = t0 + j;
    if (t < n) dst[base + t] = fmaxf(cur[j], cur[j + 2 * r + 1 - K]);
  }
}

template <typename T, int D, int G, bool P>
static void launch_score_t(const ScoreArgs& a, hipStream_t st) {
  const int64_t per_q = (int64_t)a.hq * D;
  const int64_t nq = (int64_t)a.B * a.window * per_q;
  observe("k_q_to_f64", st);
  hipLaunchKernelGGL(k_q_to_f64<T>, dim3(ceil_div(nq, 256)), dim3(256), 0, st, (const T*)a.q,
                     (const T*)a.q_hist, a.window, per_q, a.q64, nq);
  dim3 grid(ceil_div(a.max_cand, kScoreTile * kScoreTiles), a.rows.hkv, a.B);
  if (grid.x == 0) return;
  // window heads: the metric goes straight to l2 unless it is pooled
  float* wdst = a.radius > 0 ? a.wx : a.l2;
  observe("k_score", st);
  if (a.window > 1)
    hipLaunchKernelGGL((k_score<T, D, G, P, true>), grid, dim3(256), 0, st, a.q64, a.hq, a.rows,
                       a.cand, a.metric, a.logit, a.l2, wdst, a.window, a.cap_stride, a.scale);
  else
    hipLaunchKernelGGL((k_score<T, D, G, P, false>), grid, dim3(256), 0, st, a.q64, a.hq, a.rows,
                       a.cand, a.metric, a.logit, a.l2, wdst, a.window, a.cap_stride, a.scale);
  if (a.radius > 0 && a.metric != nullptr) {
    observe("k_pool", st);
    hipLaunchKernelGGL(k_pool, dim3(ceil_div(a.max_cand, kPoolTile), a.rows.hkv, a.B), dim3(256),
                       0, st, a.cand, a.metric, (const float*)a.wx, a.l2, a.cap_stride, a.radius);
  }
}

void launch_score(const ScoreArgs& a, hipStream_t st) {
  HK_DISPATCH_P(a.dtype, a.D, a.G, a.rows.table != nullptr, launch_score_t, a, st);
}

}  // namespace hk
