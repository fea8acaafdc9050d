// Selection machinery shared by the selection kernels and the fused
// lifecycle step: block reductions, the radix select by mass and its bin
// search (HARD-KV, gist.science technical summary, section 2.A Tier 2 and
// section 2.B "Outcome": the smallest top-p token set of each head).
#pragma once

#include "internal.h"

namespace hk {

template <int NW>
__device__ inline double block_sum_f64(double v, double* sh) {
  v = wave_sum_f64(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) sh[w] = v;
  __syncthreads();
  double r = sh[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r += sh[i];
  return r;
}

template <int NW>
__device__ inline float block_max_f32(float v, float* sh) {
  v = wave_max_f32(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) sh[w] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = fmaxf(r, sh[i]);
  return r;
}

template <int NW>
__device__ inline void block_sum2_f64(double& a, double& b, double* sh) {
  a = wave_sum_f64(a);
  b = wave_sum_f64(b);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) {
    sh[2 * w] = a;
    sh[2 * w + 1] = b;
  }
  __syncthreads();
  a = sh[0];
  b = sh[1];
#pragma unroll
  for (int i = 1; i < NW; ++i) {
    a += sh[2 * i];
    b += sh[2 * i + 1];
  }
}

// --------------------------------------------------------------- select ---
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

// ceil(p * Z) exactly, p a float in (0, 1), Z <= 2^63.
__device__ inline uint64_t ceil_mul(float p, uint64_t Z) {
  int ex;
  const float f = frexpf(p, &ex);                      // p = f * 2^ex, f in [0.5, 1)
  const uint64_t mant = (uint64_t)(f * 16777216.0f);   // exact 24-bit significand
  const int sh = 24 - ex;                              // p = mant * 2^-sh, sh >= 24
  const unsigned __int128 prod = (unsigned __int128)mant * Z;
  if (sh >= 120) return prod ? 1 : 0;
  const unsigned __int128 one = 1;
  return (uint64_t)((prod + ((one << sh) - 1)) >> sh);
}

// Histogram slot of bin b when NB bins are searched: one pad slot after
// every NB / 64 bins, so the 64 lanes of find_bin, each summing its own run
// of consecutive bins, read different LDS banks.
template <int NB>
__device__ __forceinline__ int hslot(uint32_t b) {
  return (int)(b + b / (NB / 64));
}
constexpr int kHistSlots = 2048 + 64;

struct SelShared {
  unsigned long long hist[kHistSlots];
  unsigned long long target;
  unsigned long long above;
  unsigned long long total;   // fixed-point mass of the head (pass 1)
  unsigned long long tally;   // k_calsel: selected count << 32 | waves done
  uint32_t bin;
  int wc[kSelWaves];
  int red[kSelWaves];
  int tpre[16 * kSelWaves];  // k_calsel: ties before (slot, wave), position order
  int blkcnt[kKeptMaxBlks];  // kept tokens per kKeptBlk block
};

// Lane l's value moved from lane l - K of its 16-lane row (0 for the first
// K lanes of the row), both 32-bit halves through DPP row shifts.
template <int K>
__device__ __forceinline__ uint64_t row_shr_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, 0x110 + K, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), 0x110 + K, 0xF, 0xF, true);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}
// Inclusive prefix sum over the 64 lanes of the wave: Hillis-Steele steps
// inside each 16-lane row, then the totals of the rows below added from
// lanes 15, 31 and 47.
__device__ __forceinline__ uint64_t wave_prefix_u64(uint64_t v) {
  v += row_shr_u64<1>(v);
  v += row_shr_u64<2>(v);
  v += row_shr_u64<4>(v);
  v += row_shr_u64<8>(v);
  const uint64_t r0 = readlane_u64(v, 15), r1 = readlane_u64(v, 31), r2 = readlane_u64(v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return v + (row >= 1 ? r0 : 0ull) + (row >= 2 ? r1 : 0ull) + (row >= 3 ? r2 : 0ull);
}

// Run by wave 0: the largest bin whose suffix mass (bins at or above it)
// reaches `target`; records the bin and the mass strictly above it.  With
// from_total, the target is first set to max(ceil(p * total), 1) and the
// total is recorded.
template <int NB>
__device__ inline void find_bin(SelShared& S, bool from_total, float p) {
  const int lane = threadIdx.x;
  constexpr int PER = NB / 64;
  unsigned long long s = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) s += S.hist[lane * (PER + 1) + i];
  // suffix sums over the lanes: total minus the exclusive prefix
  const unsigned long long pre = wave_prefix_u64(s);
  const unsigned long long total = readlane_u64(pre, 63);
  const unsigned long long suf = total - pre + s;
  unsigned long long target;
  if (from_total) {
    target = ceil_mul(p, total);
    if (target < 1) target = 1;
  } else {
    target = S.target;
  }
  const unsigned long long ok = __ballot(suf >= target);
  int L = __popcll(ok) - 1;  // suf falls with the lane: lanes 0..L reach the target
  L = L < 0 ? 0 : L;
  // inside lane L's PER bins: suffix sums over PER lanes, the same rule
  const unsigned long long base = readlane_u64(suf - s, L);  // mass above the chunk
  const unsigned long long hv = lane < PER ? S.hist[L * (PER + 1) + lane] : 0ull;
  const unsigned long long pre2 = wave_prefix_u64(hv);
  const unsigned long long suf2 = readlane_u64(pre2, 63) - pre2 + hv;
  const unsigned long long ok2 = __ballot(lane < PER && base + suf2 >= target);
  int J = __popcll(ok2) - 1;
  J = J < 0 ? 0 : J;
  if (lane == J) {
    S.bin = L * PER + J;
    S.above = base + suf2 - hv;
  }
  if (from_total && lane == 0) {
    S.target = target;
    S.total = total;
  }
}

// Where a selection's size goes: count[bh] = k and, when a mode array is
// given, the head's rewrite / sparse-loading choice for (A = n, k).
struct CountOut {
  int32_t* count;
  uint8_t* mode;
  hardkv_policy pol;
  int W;
  __device__ inline void put(int64_t bh, int n, int k) const {
    count[bh] = k;
    if (mode) mode[bh] = plan_mode(pol, n, k, W);
  }
};

// f(t, x[t]) for t = tid, tid + NT, tid + 2 NT, ... below n, in that order,
// with the loads issued U at a time (each thread's sequence of values is the
// same as one load per step; only the latency is hidden).
template <int NT, int U, typename F>
__device__ __forceinline__ void each_value(const float* x, int n, F f) {
  for (int t0 = (int)threadIdx.x; t0 < n; t0 += NT * U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + u * NT;
      v[u] = t < n ? x[t] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + u * NT;
      if (t < n) f(t, v[u]);
    }
  }
}

// Calibrated top-p selection of one head by a workgroup of NT threads
// (shared by the standalone select and the fused lifecycle step).  Radix
// select by MASS on the order-preserving key of the calibrated value
// c_t = cv(x[t]), t in [0, n): 11/11/10-bit passes over the tokens, each
// weight wfix(c, m, wscale) recomputed where a pass needs it; the tokens tied
// at the cutoff key are taken lowest position first.  Writes mk[0, n) and
// returns this thread's count of selected tokens (the caller adds them up).
// Requires 0 < n and top_p < 1; tab: the exp_nonpos table.
// count: also add each wave's kept tokens of every block of kKeptBlk
// positions into S.blkcnt (cleared here; complete after the caller's next
// barrier; requires ceil(n / kKeptBlk) <= kKeptMaxBlks).
template <int NT, typename CV>
__device__ inline int select_head(SelShared& S, int n, const float* x, CV cv, double m,
                                  float top_p, double wscale, const double* tab,
                                  uint8_t* __restrict__ mk, bool count = false) {
  constexpr int U = 8;
  static_assert(NT % kKeptBlk == 0 || kKeptBlk % NT == 0, "waves map to blocks");
  const int tid = threadIdx.x;
  if (count)
    for (int i = tid; i < kKeptMaxBlks; i += NT) S.blkcnt[i] = 0;
  // pass 1: top 11 bits of the key
  for (int i = tid; i < kHistSlots; i += NT) S.hist[i] = 0;
  __syncthreads();
  each_value<NT, U>(x, n, [&](int, float raw) {
    const float c = cv(raw);
    const uint64_t w = wfix(c, m, wscale, tab);
    if (w) atomicAdd(&S.hist[hslot<2048>(okey(c) >> 21)], (unsigned long long)w);
  });
  __syncthreads();
  if (tid < 64) find_bin<2048>(S, true, top_p);
  __syncthreads();
  const unsigned long long target = S.target;
  const uint32_t b1 = S.bin;
  unsigned long long above = S.above;
  __syncthreads();

  // pass 2: next 11 bits inside bin b1
  for (int i = tid; i < kHistSlots; i += NT) S.hist[i] = 0;
  if (tid == 0) S.target = target - above;
  __syncthreads();
  each_value<NT, U>(x, n, [&](int, float raw) {
    const float c = cv(raw);
    const uint32_t k = okey(c);
    if ((k >> 21) == b1)
      atomicAdd(&S.hist[hslot<2048>((k >> 10) & 2047u)],
                (unsigned long long)wfix(c, m, wscale, tab));
  });
  __syncthreads();
  if (tid < 64) find_bin<2048>(S, false, top_p);
  __syncthreads();
  const uint32_t b2 = S.bin;
  above += S.above;
  const unsigned long long t2 = S.target;
  __syncthreads();

  // pass 3: last 10 bits inside (b1, b2)
  for (int i = tid; i < kHistSlots; i += NT) S.hist[i] = 0;
  if (tid == 0) S.target = t2 - S.above;
  __syncthreads();
  const uint32_t pre = (b1 << 11) | b2;
  each_value<NT, U>(x, n, [&](int, float raw) {
    const float c = cv(raw);
    const uint32_t k = okey(c);
    if ((k >> 10) == pre)
      atomicAdd(&S.hist[hslot<1024>(k & 1023u)], (unsigned long long)wfix(c, m, wscale, tab));
  });
  __syncthreads();
  if (tid < 64) find_bin<1024>(S, false, top_p);
  __syncthreads();
  const uint32_t kstar = (pre << 10) | S.bin;
  above += S.above;
  // all tokens tied at K* carry the same weight; take r of them
  const unsigned long long wstar = wfix(okey_inv(kstar), m, wscale, tab);
  const unsigned long long need = target - above;
  const unsigned long long r = (need + wstar - 1) / wstar;
  // every token tied at K* carries wstar, so its bin holds mass / wstar of
  // them; when r reaches that count every tie is taken and the mask needs no
  // ranking (no barrier per block of tokens)
  const unsigned long long ntie_all = S.hist[hslot<1024>(S.bin)] / wstar;
  const int wv = tid >> 6, ln = tid & 63;
  if (r >= ntie_all) {
    int nsel = 0;
    for (int t0 = 0; t0 < n; t0 += NT * U) {
      float v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = t0 + u * NT + tid;
        v[u] = t < n ? x[t] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = t0 + u * NT + tid;
        const bool sel = t < n && okey(cv(v[u])) >= kstar;
        if (t < n) mk[t] = sel ? 1 : 0;
        nsel += sel;
        if (count) {
          const unsigned long long bal = __ballot(sel);
          if (ln == 0 && bal)
            atomicAdd(&S.blkcnt[(t0 + u * NT + 64 * wv) / kKeptBlk], (int)__popcll(bal));
        }
      }
    }
    return nsel;
  }

  // pass 4: mask, ties by ascending position; the next block's value is
  // loaded while the current one is ranked
  unsigned long long carried = 0;
  int nsel = 0;
  float nxt = tid < n ? x[tid] : 0.f;
  for (int t0 = 0; t0 < n; t0 += NT) {
    const int t = t0 + tid;
    const bool valid = t < n;
    const float raw = nxt;
    nxt = t + NT < n ? x[t + NT] : 0.f;
    const uint32_t k = valid ? okey(cv(raw)) : 0u;
    const bool tie = valid && k == kstar;
    const int ntie = __syncthreads_count(tie);
    unsigned long long rank = 0;
    if (ntie) {
      const unsigned long long bal = __ballot(tie);
      if (ln == 0) S.wc[wv] = __popcll(bal);
      __syncthreads();
      int off = 0;
      for (int i = 0; i < wv; ++i) off += S.wc[i];
      __syncthreads();
      rank = carried + off + __popcll(bal & ((1ull << ln) - 1ull));
      carried += ntie;
    }
    const bool sel = valid && (k > kstar || (tie && rank < r));
    if (valid) mk[t] = sel ? 1 : 0;
    nsel += sel;
    if (count) {
      const unsigned long long bal = __ballot(sel);
      if (ln == 0 && bal) atomicAdd(&S.blkcnt[(t0 + 64 * wv) / kKeptBlk], (int)__popcll(bal));
    }
  }
  return nsel;
}

// ------------------------------------------------------- small selection --
constexpr int kSmallSel = 128;  // tokens select_small takes (two waves)

struct SelSmall {
  uint32_t key[kSmallSel];
  unsigned long long w[kSmallSel];  // fixed-point weights in rank order
  unsigned long long wtot[2];       // the two waves' totals
};

// The same selection as select_head for n <= kSmallSel tokens whose
// calibrated values thread t < n holds in c: each token's rank in (key
// descending, position ascending) order is counted against every key, the
// weights wfix(c, m, wscale) are laid out in rank order and summed (integer
// prefix sums), and the shortest rank prefix reaching max(ceil(p * Z), 1) is
// kept.  No pass over memory: for the short pools of a steady lifecycle,
// where the radix passes' histogram clears, barriers and re-reads dominate.
// Requires 0 < n <= kSmallSel and top_p < 1; called by every thread of the
// workgroup.  Writes mk[0, n).
__device__ inline void select_small(SelSmall& S, int n, float c, double m, float top_p,
                                    double wscale, const double* tab, uint8_t* __restrict__ mk) {
  const int tid = threadIdx.x;
  const bool mine = tid < n;
  const uint32_t key = mine ? okey(c) : 0u;
  const unsigned long long w = mine ? (unsigned long long)wfix(c, m, wscale, tab) : 0ull;
  if (mine) S.key[tid] = key;
  __syncthreads();
  int rank = 0;
  if ((tid & ~63) < n) {  // waves holding tokens
    for (int j = 0; j < n; ++j) {
      const uint32_t kj = S.key[j];
      rank += (kj > key) | ((kj == key) & (j < tid));
    }
  }
  if (mine) S.w[rank] = w;
  __syncthreads();
  unsigned long long incl = 0;
  if (tid < kSmallSel) {  // waves 0 and 1, whole
    incl = wave_prefix_u64(tid < n ? S.w[tid] : 0ull);
    if ((tid & 63) == 63) S.wtot[tid >> 6] = incl;
  }
  __syncthreads();
  const unsigned long long total = S.wtot[0] + S.wtot[1];
  if (tid >= 64 && tid < kSmallSel) incl += S.wtot[0];
  unsigned long long target = ceil_mul(top_p, total);
  if (target < 1) target = 1;
  // k = 1 + the ranks whose inclusive prefix is still below the target
  const int below = __syncthreads_count(tid < n && incl < target);
  const int k = below + 1 < n ? below + 1 : n;
  if (mine) mk[tid] = rank < k ? 1 : 0;
}

// select_small for n <= 64 tokens held by the lanes of one wave (lane t:
// token t), run by that wave alone: ranks from the keys broadcast lane by
// lane, the weights moved to their rank's lane (forward permute), an integer
// prefix over the lanes and a ballot for the cutoff.  No LDS and no
// workgroup barrier; the caller's next barrier publishes the mask.
__device__ inline void select_wave(int n, float c, double m, float top_p, double wscale,
                                   const double* tab, uint8_t* __restrict__ mk) {
  const int lane = threadIdx.x & 63;
  const bool mine = lane < n;
  const uint32_t key = mine ? okey(c) : 0u;
  const unsigned long long w = mine ? (unsigned long long)wfix(c, m, wscale, tab) : 0ull;
  int rank = 0;
  for (int j = 0; j < n; ++j) {
    const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)key, j);
    rank += (kj > key) | ((kj == key) & (j < lane));
  }
  // lanes past the tokens keep their own index: the targets stay a permutation
  const int dst = mine ? rank : lane;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_permute(dst * 4, (int)(uint32_t)w);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_permute(dst * 4, (int)(uint32_t)(w >> 32));
  const unsigned long long incl = wave_prefix_u64(((unsigned long long)hi << 32) | lo);
  const unsigned long long total = readlane_u64(incl, 63);
  unsigned long long target = ceil_mul(top_p, total);
  if (target < 1) target = 1;
  const int below = __popcll(__ballot(lane < n && incl < target));
  const int k = below + 1 < n ? below + 1 : n;
  if (mine) mk[lane] = rank < k ? 1 : 0;
}

}  // namespace hk
