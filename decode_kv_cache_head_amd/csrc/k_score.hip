// Importance scores of aged tokens (HARD-KV, gist.science technical summary,
// section 2.B "Goal": max-pooled logits; key-norm metric alongside).
//
// Observation-window heads (section 2.B: SnapKV-style strategies) also take
// the max over the earlier queries of the window, then a max-pooling pass
// over neighbouring positions (k_pool).
//
// Key-dissimilarity heads (section 2.B: similarity scores) score
// s_t = -(k_t . mu) / (||k_t|| ||mu||) with mu the sum of the head's candidate
// keys, which k_prep forms in float64 first.
//
// HBM-bound stream over the aged keys.  Each workgroup stages one 128-token
// tile of one (b, h) in LDS; two lanes score each token, one per half of the
// head dimension, with the G query rows of the head's GQA group read as
// float64 from wave-uniform addresses (scalar loads, SGPR operands).  The
// token's key is widened exactly to float64 and the dot products are
// accumulated in float64, so the only rounding the ranking key sees is the
// final fl32().  At G >= 8 (bf16, d = 128, no metric array) k_score_mx
// first picks each token's candidate heads on the matrix cores and takes the
// float64 dot of those only; the logit is the same.
#include "internal.h"

namespace hk {

// Before the score, one launch of 1024-thread blocks:
//   blocks [0, nqb): q64[b][i][:] = this step's query (i = 0) or the i-th
//     previous one (q_hist), widened to float64;
//   blocks [nqb, nqb + B Hkv): one per (b, h); key-dissimilarity heads sum
//     their candidate keys in float64 into kmu[b][h][0..D) and ||mu|| into
//     kmu[b][h][D]; R-KV heads sum their unit keys k / ||k|| instead (each
//     row's norm from its pieces, reduced over the lanes that hold them);
//     other heads return.  Each thread adds a fixed 16-byte
//     piece of a fixed set of rows, the next batch of rows in flight while
//     the current one is added; the row groups are then combined in a fixed
//     order (lane pairs inside each wave, then the waves in LDS).
constexpr int kPrepThreads = 1024;

template <typename T, int D, bool P>
__global__ __launch_bounds__(kPrepThreads) void k_prep(
    const T* __restrict__ q, const T* __restrict__ q_hist, int window, int64_t per_q,
    double* __restrict__ q64, int64_t nq, int nqb, int hkv, Rows rows, Cand cand,
    const int8_t* __restrict__ metric, double* __restrict__ kmu) {
  constexpr int EPC = Elt<T>::kPer16;
  constexpr int CPR = D * (int)sizeof(T) / 16;  // pieces per row (<= 64)
  constexpr int RG = kPrepThreads / CPR;         // row groups
  constexpr int U = 8;                           // rows per batch per thread
  constexpr int NW = kPrepThreads / 64;
  __shared__ double red[NW][CPR][EPC];
  __shared__ double sq[D];
  const int tid = threadIdx.x;
  if ((int)blockIdx.x < nqb) {
    const int64_t i = (int64_t)blockIdx.x * kPrepThreads + tid;
    if (i >= nq) return;
    const int64_t b = i / (window * per_q), rest = i % (window * per_q);
    const int64_t wi = rest / per_q, e = rest % per_q;
    const T* src = wi == 0 ? q + b * per_q + e : q_hist + (b * (window - 1) + wi - 1) * per_q + e;
    q64[i] = (double)Elt<T>::load1(src);
    return;
  }
  const int hb = blockIdx.x - nqb;
  const int b = hb / hkv, h = hb % hkv;
  const bool unit = metric[h] == HARDKV_METRIC_RKV;
  if (metric[h] != HARDKV_METRIC_KEYDIFF && !unit) return;
  const int n = cand.n(b, h);
  const int c = tid % CPR, r0 = tid / CPR;
  const int rb = rows.tb(b, h), rh = rows.th(h);
  auto fetch = [&](v4u (&raw)[U], int r) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int rr = r + u * RG;
      raw[u] = rr < n ? *(const v4u*)(rows.template row<P>(rb, rh, rr) + c * 16)
                      : v4u{0u, 0u, 0u, 0u};
    }
  };
  double acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.0;
  v4u cur[U], nxt[U];
  fetch(cur, r0);
  for (int r = r0; r < n; r += U * RG) {
    if (r + U * RG < n) fetch(nxt, r + U * RG);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float f[EPC];
      Elt<T>::unpack(cur[u], f);
      if (unit) {
        // the row's squared norm: this piece's part, then the CPR lanes of
        // the row (aligned groups of CPR consecutive lanes) in a fixed order
        double ss = 0.0;
#pragma unroll
        for (int e = 0; e < EPC; ++e) ss = fma((double)f[e], (double)f[e], ss);
#pragma unroll
        for (int o = 1; o < CPR; o <<= 1) ss += __shfl_xor(ss, o, 64);
        const double inv = ss > 0.0 ? 1.0 / sqrt(ss) : 0.0;
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[e] += (double)f[e] * inv;
      } else {
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[e] += (double)f[e];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = nxt[u];
  }
  // lanes l and l + CPR of a wave hold the same piece: pair them up to one
  // value per piece per wave (fixed pairing), then add the waves in order
  const int lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int o = CPR; o < 64; o <<= 1)
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] += __shfl_xor(acc[e], o, 64);
  if (lane < CPR) {
#pragma unroll
    for (int e = 0; e < EPC; ++e) red[w][lane][e] = acc[e];
  }
  __syncthreads();
  double* mu = kmu + ((int64_t)b * hkv + h) * (D + 1);
  if (tid < D) {
    const int pc = tid / EPC, e = tid % EPC;
    double sum = 0.0;
    for (int v = 0; v < NW; ++v) sum += red[v][pc][e];
    mu[tid] = sum;
    sq[tid] = sum * sum;
  }
  __syncthreads();
  if (tid == 0) {
    double ss = 0.0;
    for (int i = 0; i < D; ++i) ss += sq[i];
    mu[D] = sqrt(ss);
  }
}

constexpr int kScoreTile = 128;  // tokens per tile
// consecutive tiles per workgroup, the next one loaded while the current one
// is scored; at G = 8 the float64 work dominates and single tiles in more
// workgroups are faster
template <int G>
constexpr int score_group() { return G >= 8 ? 1 : 4; }

// Partial q.k over one split of the row: `row` points at the split's first
// byte, `qg` at the split's first query element; float64 from exact inputs.
// KD: also the partial dot with the key sum mu (same split, float64).
template <typename T, int D, int G, int PCS, bool L2, bool KD = false>
__device__ __forceinline__ void split_dot(const unsigned char* row, const double* __restrict__ qg,
                                          double (&acc)[G], double& ss,
                                          const double* __restrict__ mu = nullptr,
                                          double* mdot = nullptr) {
  constexpr int EPC = Elt<T>::kPer16;
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = 0.0;
  ss = 0.0;
  if (KD) *mdot = 0.0;
#pragma unroll
  for (int c = 0; c < PCS; ++c) {
    const v4u raw = *(const v4u*)(row + c * 16);
    float f[EPC];
    Elt<T>::unpack(raw, f);
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      const double kd = (double)f[e];
#pragma unroll
      for (int g = 0; g < G; ++g) acc[g] = fma(qg[g * D + c * EPC + e], kd, acc[g]);
      if (L2) ss = fma(kd, kd, ss);
      if (KD) *mdot = fma(mu[c * EPC + e], kd, *mdot);
    }
  }
}

// Consecutive 128-token tiles of one (b, h) per 256-thread workgroup (four,
// or one at G = 8).  A tile is staged into LDS with coalesced 16-byte loads,
// and the next tile's loads are issued into registers before the current one
// is scored, so each workgroup keeps its loads in flight while its float64
// arithmetic runs.  Every token is scored by two lanes in different waves,
// one per half of the head dimension: waves 0-1 take the first half of
// tokens 0-63 / 64-127, waves 2-3 the second half.  The half index is
// wave-uniform, so the float64 query elements stay scalar loads (SGPR
// operands of v_fma_f64); the second half's partial sums reach the first
// through LDS.
template <typename T, int D, int G, bool P, bool WIN>
__global__ __launch_bounds__(256) void k_score(const double* __restrict__ q64, int hq, Rows rows,
                                               Cand cand, const int8_t* __restrict__ metric,
                                               float* __restrict__ logit, float* __restrict__ l2,
                                               float* __restrict__ wdst, int window,
                                               int64_t cap_stride, double scale,
                                               const double* __restrict__ kmu) {
  constexpr int RB = D * (int)sizeof(T);
  constexpr int CPR = RB / 16;             // 16-byte pieces per row
  constexpr int PCS = CPR / 2;             // pieces per half row
  constexpr int PAD = RB + 16;             // conflict-free per-lane row reads
  constexpr int LOADS = kScoreTile * CPR / 256;
  __shared__ __attribute__((aligned(16))) unsigned char lds[kScoreTile * PAD];
  __shared__ double s_part[G + 2][kScoreTile];  // second half's dots, squared norm, key-sum dot
  // logical (tile group, h, b), tile group fastest; each head on one XCD
  const int hkv = gridDim.y, tid = threadIdx.x;
  const int L = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int id = xcd_by_head(L, gridDim.x, gridDim.y * gridDim.z);
  const int grp = id % gridDim.x, h = (id / gridDim.x) % hkv, b = id / (gridDim.x * hkv);
  const int n = cand.n(b, h);
  constexpr int kScoreGroup = score_group<G>();
  const int g0 = grp * kScoreGroup * kScoreTile;
  if (g0 >= n) return;
  const int w = tid >> 6, lane = tid & 63;
  const int half = __builtin_amdgcn_readfirstlane(w >> 1);
  const int tok = (w & 1) * 64 + lane;
  const bool is_l2 = metric != nullptr && metric[h] == HARDKV_METRIC_L2;
  const bool is_win = metric != nullptr && metric[h] == HARDKV_METRIC_WINDOW;
  const bool is_rkv = metric != nullptr && metric[h] == HARDKV_METRIC_RKV;
  const bool is_kd = is_rkv || (metric != nullptr && metric[h] == HARDKV_METRIC_KEYDIFF);
  // key-dissimilarity heads: the candidates' key sum (this half) and its norm
  const double* kmu_h = kmu + ((int64_t)b * hkv + h) * (D + 1);
  const int64_t qoff = ((int64_t)b * window * hq + (int64_t)h * G) * D + half * (D / 2);
  const unsigned char* row = lds + tok * PAD + half * (RB / 2);
  const int64_t obase = ((int64_t)b * hkv + h) * cap_stride;
  v4u buf[LOADS];
  const int rb = rows.tb(b, h), rh = rows.th(h);  // (b, h) as the row tables index them
  auto fetch = [&](int t0) {
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int idx = j * 256 + tid, r = idx / CPR, c = idx % CPR;
      // non-temporal: the keys are read once here and once more by the
      // compaction, far apart in time; streaming them keeps the caches for
      // the score arrays the selection reads next
      buf[j] = __builtin_nontemporal_load(
          (const v4u*)(rows.template row<P>(rb, rh, min(t0 + r, n - 1)) + c * 16));
    }
  };
  // scores of the staged tile starting at t0 (uniform over the workgroup)
  auto score_staged = [&](int t0) {
    const int t = t0 + tok;
    const double* __restrict__ qg = q64 + qoff;
    double acc[G], ss, md = 0.0;
    if (is_kd)
      split_dot<T, D, G, PCS, true, true>(row, qg, acc, ss, kmu_h + half * (D / 2), &md);
    else if (is_l2)
      split_dot<T, D, G, PCS, true>(row, qg, acc, ss);
    else
      split_dot<T, D, G, PCS, false>(row, qg, acc, ss);
    if (half) {
#pragma unroll
      for (int g = 0; g < G; ++g) s_part[g][tok] = acc[g];
      s_part[G][tok] = ss;
      s_part[G + 1][tok] = md;
    }
    __syncthreads();
    double mx = -INFINITY;
    if (!half) {
#pragma unroll
      for (int g = 0; g < G; ++g) mx = fmax(mx, acc[g] + s_part[g][tok]);
      if (t < n) {
        logit[obase + t] = (float)(mx * scale);
        if (is_l2) l2[obase + t] = (float)sqrt(ss + s_part[G][tok]);
        if (is_rkv) {
          // minus the mean cosine to the other candidates: (u_t . nu - 1) / (n - 1)
          const double nk = sqrt(ss + s_part[G][tok]);
          const double v = nk > 0.0 && n > 1 ? -((md + s_part[G + 1][tok]) / nk - 1.0) / (n - 1)
                                             : 0.0;
          l2[obase + t] = (float)v;
        } else if (is_kd) {
          const double nk = sqrt(ss + s_part[G][tok]), nm = kmu_h[D];
          const double v = nk > 0.0 && nm > 0.0 ? -(md + s_part[G + 1][tok]) / (nk * nm) : 0.0;
          l2[obase + t] = (float)v;
        }
      }
    }
    if (is_win) {
      // observation window: the earlier queries of the window, one partial
      // exchange each (a wave-uniform branch: the whole workgroup takes it)
      double mw = mx;
      if constexpr (WIN) {
#pragma unroll 1
        for (int i = 1; i < window; ++i) {
          split_dot<T, D, G, PCS, false>(row, qg + (int64_t)i * hq * D, acc, ss);
          __syncthreads();  // the previous exchange has been read
          if (half) {
#pragma unroll
            for (int g = 0; g < G; ++g) s_part[g][tok] = acc[g];
          }
          __syncthreads();
          if (!half) {
#pragma unroll
            for (int g = 0; g < G; ++g) mw = fmax(mw, acc[g] + s_part[g][tok]);
          }
        }
      }
      if (!half && t < n) wdst[obase + t] = (float)(mw * scale);
    }
  };
  fetch(g0);
  if constexpr (kScoreGroup == 1) {
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int idx = j * 256 + tid, r = idx / CPR, c = idx % CPR;
      *(v4u*)(lds + r * PAD + c * 16) = buf[j];
    }
    __syncthreads();
    score_staged(g0);
  } else {
#pragma unroll 1
    for (int k = 0; k < kScoreGroup; ++k) {
      const int t0 = g0 + k * kScoreTile;  // uniform over the workgroup
      if (t0 >= n) break;
      if (k) __syncthreads();  // the previous tile's LDS and exchange reads are done
#pragma unroll
      for (int j = 0; j < LOADS; ++j) {
        const int idx = j * 256 + tid, r = idx / CPR, c = idx % CPR;
        *(v4u*)(lds + r * PAD + c * 16) = buf[j];
      }
      __syncthreads();
      // the next tile's rows are in flight while this one is scored
      if (k + 1 < kScoreGroup && t0 + kScoreTile < n) fetch(t0 + kScoreTile);
      score_staged(t0);
    }
  }
}

// Logit-only launches with bf16 keys, d = 128 and G >= 8: the matrix cores
// find each token's winning query heads, float64 decides among them.
//   1. S = K Q^T and A = |K| |Q|^T as 16x16x32 bf16 MFMA products; the
//      products are exact in float32 (inside its range), so each float32
//      dot is within 127 * 2^-24 * A of the true one (recursive summation
//      of 128 terms; the kernel allows four times that, 2^-15 A).
//   2. Per token, head i with float32 dot v_i and bound e_i = 2^-15 A_i +
//      2^-117 (the second term covers subnormal products flushed to zero) is
//      a candidate when v_i + e_i reaches max_j (v_j - e_j): the head with
//      the true maximum always does (usually it is the only one).  A head
//      whose A_i overflows float32 has no bound and is always a candidate.
//   3. Two lanes per token (one per half of d, as in k_score) take the
//      float64 dot of each candidate from the exact inputs (the queries
//      widened exactly to float64 in LDS, the bf16 keys widened in
//      registers), in k_score's order, and keep the maximum.
// The logit fl32(max_g q_g . k_t / sqrt(d)) is the one k_score computes: the
// true maximum is always a candidate.  Float64 work falls from G to about one
// dot per token.
constexpr int kScoreMxQS = 128 + 2;  // float64 query row stride in LDS (rows on different banks)
// Workgroups per (b, h): each takes one contiguous run of the head's tiles,
// split by the head's actual candidate count (read on the device), with the
// next tile in flight.  A pool far below its capacity then dispatches few
// idle workgroups (fixed groups of the capacity would leave most of the
// grid idle).
constexpr int kScoreMxSplit = 8;

template <int G, bool P>
__global__ __launch_bounds__(256) void k_score_mx(const bf16_t* __restrict__ q, int hq,
                                                  Rows rows, Cand cand,
                                                  float* __restrict__ logit, int64_t cap_stride,
                                                  double scale) {
  constexpr int D = 128, RB = 256, CPR = 16, PAD = RB + 16;
  constexpr int LOADS = kScoreTile * CPR / 256;
  constexpr float kErr = 1.0f / 32768.0f;  // 2^-15: four times the float32 summation bound
  __shared__ __attribute__((aligned(16))) unsigned char lds[kScoreTile * PAD];
  __shared__ __attribute__((aligned(16))) double s_q[G][kScoreMxQS];  // bf16 widened exactly
  __shared__ uint32_t s_cand[kScoreTile];
  const int hkv = gridDim.y, tid = threadIdx.x;
  const int L = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int id = xcd_by_head(L, gridDim.x, gridDim.y * gridDim.z);
  const int grp = id % gridDim.x, h = (id / gridDim.x) % hkv, b = id / (gridDim.x * hkv);
  const int n = cand.n(b, h);
  const int ntiles = (n + kScoreTile - 1) / kScoreTile;
  const int per = (ntiles + (int)gridDim.x - 1) / (int)gridDim.x;
  const int tbeg = grp * per, tcnt = min(per, ntiles - tbeg);
  if (tcnt <= 0) return;
  const int g0 = tbeg * kScoreTile;
  const int rb = rows.tb(b, h), rh = rows.th(h);
  v4u buf[LOADS];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int idx = j * 256 + tid, r = idx / CPR, c = idx % CPR;
      buf[j] = __builtin_nontemporal_load(
          (const v4u*)(rows.template row<P>(rb, rh, min(t0 + r, n - 1)) + c * 16));
    }
  };
  fetch(g0);
  const int64_t qrow = (int64_t)b * hq + (int64_t)h * G;
  for (int i = tid; i < G * D / 8; i += 256) {  // 16-byte pieces, 8 values each
    float f[8];
    Elt<bf16_t>::unpack(*(const v4u*)(q + qrow * D + i * 8), f);
    double* dst = &s_q[i / (D / 8)][(i % (D / 8)) * 8];
#pragma unroll
    for (int e = 0; e < 8; e += 2) *(double2*)(dst + e) = double2{(double)f[e], (double)f[e + 1]};
  }
  const int w = tid >> 6, lane = tid & 63;
  const int qi = lane & 15, g4 = lane >> 4;
  v4u qb[4], qa[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    qb[s] = qi < G ? *(const v4u*)(q + (qrow + qi) * D + 32 * s + 8 * g4) : v4u{0u, 0u, 0u, 0u};
    qa[s] = qb[s] & 0x7fff7fffu;
  }
  const int tok = 32 * w + (lane & 31), half = lane >> 5;
  float* out = logit + ((int64_t)b * hkv + h) * cap_stride;
#pragma unroll 1
  for (int k = 0; k < tcnt; ++k) {
    const int t0 = g0 + k * kScoreTile;  // uniform over the workgroup
    if (t0 >= n) break;
    if (k) __syncthreads();  // the previous tile's LDS reads are done
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int idx = j * 256 + tid, r = idx / CPR, c = idx % CPR;
      *(v4u*)(lds + r * PAD + c * 16) = buf[j];
    }
    __syncthreads();
    // the next tile's rows are in flight while this one is scored
    if (k + 1 < tcnt) fetch(t0 + kScoreTile);
    // 1-2: wave w filters tokens [32 w, 32 w + 32), two 16-row products
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int r = 32 * w + 16 * c + qi;
      f32x4_t sd = {0.f, 0.f, 0.f, 0.f}, sa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const v4u ka = *(const v4u*)(lds + r * PAD + (32 * s + 8 * g4) * 2);
        sd = mfma16(ka, qb[s], sd);
        sa = mfma16(ka & 0x7fff7fffu, qa[s], sa);
      }
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        // token 32 w + 16 c + 4 g4 + cc, query head qi: its float32 dot v
        // lies within e of the true one (the summation bound 2^-15 A plus
        // 2^-117 for subnormal products, at most 2^-126 off each when
        // flushed), so the head may hold the maximum only if v + e reaches
        // the largest lower bound v' - e' of the token's heads.  A head whose
        // sum of |q k| overflows float32 has no bound: it is a candidate and
        // sets no lower bound.
        const float v = qi < G ? sd[cc] : -INFINITY;
        const float e = qi < G ? fmaf(kErr, sa[cc], 0x1p-117f) : 0.f;
        const bool bounded = e < INFINITY;
        // (at G <= 8 the heads sit in lanes 0-7 of the row: their own maximum)
        const float lb = bounded ? v - e : -INFINITY;
        const float lo = G <= 8 ? row_max8(lb) : row_max16(lb);
        const unsigned long long bal = __ballot(qi < G && (!bounded || v + e >= lo));
        if (qi == 0) s_cand[32 * w + 16 * c + 4 * g4 + cc] = (uint32_t)(bal >> (16 * g4)) & 0xffffu;
      }
    }
    // 3: float64 dots of the candidates, lanes l and l + 32 on the two halves
    // (s_cand of these tokens was written by this wave)
    uint32_t mask = s_cand[tok];
    const unsigned char* row = lds + tok * PAD + half * (RB / 2);
    double best = -INFINITY;
    while (mask) {
      const int i = __builtin_ctz(mask);
      mask &= mask - 1u;
      const double* qh = &s_q[i][half * (D / 2)];
      double acc = 0.0;
#pragma unroll 4
      for (int c = 0; c < 8; ++c) {
        const v4u raw = *(const v4u*)(row + c * 16);
        double g[8];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const double2 gg = *(const double2*)(qh + c * 8 + e);
          g[e] = gg.x;
          g[e + 1] = gg.y;
        }
        float f[8];
        Elt<bf16_t>::unpack(raw, f);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fma(g[e], (double)f[e], acc);
      }
      const double other = __shfl_xor(acc, 32, 64);
      best = fmax(best, half ? other + acc : acc + other);
    }
    const int t = t0 + tok;
    if (half == 0 && t < n) out[t] = (float)(best * scale);
  }
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
  // the filter (G >= 8, bf16, d = 128, no metric array) reads the bf16 queries
  constexpr bool kMx = sizeof(T) == 2 && D == 128 && G >= 8;
  const bool mx = kMx && a.metric == nullptr && a.window == 1;
  const int nqb = a.q_ready || mx ? 0 : ceil_div(nq, kPrepThreads);
  // with a metric array, one more block per (b, h) for the key sums
  const int nkb = a.metric != nullptr ? a.B * a.hkv : 0;
  if (nqb + nkb > 0) {
    observe("k_prep", st);
    hipLaunchKernelGGL((k_prep<T, D, P>), dim3(nqb + nkb), dim3(kPrepThreads), 0, st,
                       (const T*)a.q, (const T*)a.q_hist, a.window, per_q, a.q64, nq, nqb,
                       a.hkv, a.rows, a.cand, a.metric, a.kmu);
  }
  dim3 grid(ceil_div(a.max_cand, kScoreTile * score_group<G>()), a.hkv, a.B);
  if (grid.x == 0) return;
  // window heads: the metric goes straight to l2 unless it is pooled
  float* wdst = a.radius > 0 ? a.wx : a.l2;
  // the filter pays at G >= 8; at G = 4 the float64 dots of k_score already
  // hide behind its loads (0.195 vs 0.236 ms on the 16k headline shape)
  if constexpr (kMx) {
    if (mx) {
      observe("k_score", st);
      hipLaunchKernelGGL((k_score_mx<G, P>),
                         dim3(min(kScoreMxSplit, ceil_div(a.max_cand, kScoreTile)), a.hkv, a.B),
                         dim3(256), 0, st, (const bf16_t*)a.q, a.hq, a.rows, a.cand,
                         a.logit, a.cap_stride, a.scale);
      return;
    }
  }
  observe("k_score", st);
  if (a.window > 1)
    hipLaunchKernelGGL((k_score<T, D, G, P, true>), grid, dim3(256), 0, st, a.q64, a.hq, a.rows,
                       a.cand, a.metric, a.logit, a.l2, wdst, a.window, a.cap_stride, a.scale,
                       a.kmu);
  else
    hipLaunchKernelGGL((k_score<T, D, G, P, false>), grid, dim3(256), 0, st, a.q64, a.hq, a.rows,
                       a.cand, a.metric, a.logit, a.l2, wdst, a.window, a.cap_stride, a.scale,
                       a.kmu);
  if (a.radius > 0 && a.metric != nullptr) {
    observe("k_pool", st);
    hipLaunchKernelGGL(k_pool, dim3(ceil_div(a.max_cand, kPoolTile), a.hkv, a.B), dim3(256),
                       0, st, a.cand, a.metric, (const float*)a.wx, a.l2, a.cap_stride, a.radius);
  }
}

void launch_score(const ScoreArgs& a, hipStream_t st) {
  HK_DISPATCH_P(a.dtype, a.D, a.G, a.rows.table != nullptr, launch_score_t, a, st);
}

}  // namespace hk
