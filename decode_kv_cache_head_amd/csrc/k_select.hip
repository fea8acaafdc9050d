// Logits Calibration and Calibrated Top-p selection (HARD-KV, gist.science
// technical summary, section 2.B "Mechanism"/"Outcome" and section 2.A,
// Tier 2).
//
// calibrate: one workgroup per (b, h).  Deterministic float64 block
//   reductions (fixed lane/wave order, no atomics): moments for key-norm
//   heads, then m = max c and Z = sum exp(c - m).
// select: one 1024-thread workgroup per (b, h).  Radix select by MASS on the
//   order-preserving 32-bit key of the float32 calibrated value: 11/11/10-bit
//   passes, each accumulating per-bin mass in LDS in fixed point (2^-47
//   units up to 65536 candidates per head, coarser beyond: mass_scale)
//   (integer atomics, so the result does not depend on the order of the
//   additions).  The cutoff key K* is the bin where the mass accumulated from
//   the top first reaches ceil(p * Z); the tokens tied at K* are taken lowest
//   position first, as many as needed.  A final ordered pass writes the mask.
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

// Entropy-matched temperature (HARDKV_CALIB_ENTROPY) of one head, run by the
// whole workgroup.  each_logit(f) / each_metric(f) call f on every logit /
// metric value this thread holds.  Target: the entropy of softmax(logit),
// ln Z - sum(w d) / Z with d = x - max x, w = exp(d).  The inverse
// temperature beta in [0, 1024 / (max s - min s)] is bisected 32 times on the
// entropy of softmax(beta s) (a midpoint entropy above the target raises the
// lower end); c = (s - max s) * beta.  Every decision is taken on block sums
// that all threads read in the same order, so the branch is uniform.
constexpr int kEntropySteps = 32;
constexpr double kEntropySpan = 1024.0;

template <int NW, typename EachLogit, typename EachMetric>
__device__ inline void entropy_temperature(EachLogit each_logit, EachMetric each_metric,
                                           double* sh2, float* shf, double& shift,
                                           double& scale) {
  float lm = -INFINITY;
  each_logit([&](float x) { lm = fmaxf(lm, x); });
  const double lmax = (double)block_max_f32<NW>(lm, shf);
  double z = 0.0, zd = 0.0;
  each_logit([&](float x) {
    const double d = (double)x - lmax, w = exp(d);
    z += w;
    zd += w * d;
  });
  block_sum2_f64<NW>(z, zd, sh2);
  const double target = log(z) - zd / z;
  float smx = -INFINITY, smn = -INFINITY;
  each_metric([&](float x) {
    smx = fmaxf(smx, x);
    smn = fmaxf(smn, -x);
  });
  const double smax = (double)block_max_f32<NW>(smx, shf);
  const double smin = -(double)block_max_f32<NW>(smn, shf);
  if (smax == smin) {
    shift = 0.0;
    scale = 0.0;
    return;
  }
  double lo = 0.0, hi = kEntropySpan / (smax - smin);
  for (int it = 0; it < kEntropySteps; ++it) {
    const double mid = 0.5 * (lo + hi);
    double zb = 0.0, zbd = 0.0;
    each_metric([&](float x) {
      const double d = (double)x - smax, w = exp(mid * d);
      zb += w;
      zbd += w * d;
    });
    block_sum2_f64<NW>(zb, zbd, sh2);
    const double H = log(zb) - mid * zbd / zb;
    if (H > target)
      lo = mid;
    else
      hi = mid;
  }
  shift = smax;
  scale = 0.5 * (lo + hi);
}

// ------------------------------------------------------------ calibrate ---
__global__ __launch_bounds__(256) void k_calibrate(Cand cand, const int8_t* __restrict__ metric,
                                                   const float* __restrict__ logit,
                                                   const float* __restrict__ l2,
                                                   int64_t cap_stride, double* __restrict__ stats,
                                                   int calib) {
  __shared__ double shd[8];
  __shared__ float shf[4];
  const int h = blockIdx.x, b = blockIdx.y, hkv = gridDim.x, tid = threadIdx.x;
  const int n = cand.n(b, h);
  const int64_t bh = (int64_t)b * hkv + h;
  const float* x = logit + bh * cap_stride;
  const bool is_l2 = aux_metric(metric, h);  // second score array
  double shift = 0.0, scale = 1.0;
  if (is_l2 && calib == HARDKV_CALIB_ENTROPY) {
    const float* s = l2 + bh * cap_stride;
    shift = 0.0;
    scale = 0.0;
    if (n > 0)  // uniform over the workgroup
      entropy_temperature<4>(
          [&](auto f) {
            for (int t = tid; t < n; t += 256) f(x[t]);
          },
          [&](auto f) {
            for (int t = tid; t < n; t += 256) f(s[t]);
          },
          shd, shf, shift, scale);
    x = s;
  } else if (is_l2) {
    const float* s = l2 + bh * cap_stride;
    double sx = 0.0, sy = 0.0;
    for (int t = tid; t < n; t += 256) {
      sx += (double)x[t];
      sy += (double)s[t];
    }
    sx = block_sum_f64<4>(sx, shd);
    sy = block_sum_f64<4>(sy, shd);
    const double mux = n ? sx / n : 0.0, mus = n ? sy / n : 0.0;
    double vx = 0.0, vy = 0.0;
    for (int t = tid; t < n; t += 256) {
      const double dx = (double)x[t] - mux, dy = (double)s[t] - mus;
      vx += dx * dx;
      vy += dy * dy;
    }
    vx = block_sum_f64<4>(vx, shd);
    vy = block_sum_f64<4>(vy, shd);
    const double sdx = n ? sqrt(vx / n) : 0.0, sds = n ? sqrt(vy / n) : 0.0;
    if (sdx == 0.0 || sds == 0.0) {
      shift = 0.0;
      scale = 0.0;
    } else {
      shift = mus;
      scale = sdx / sds;
    }
    x = s;
  }
  float m = -INFINITY;
  for (int t = tid; t < n; t += 256) m = fmaxf(m, is_l2 ? cval(x[t], shift, scale) : x[t]);
  m = block_max_f32<4>(m, shf);
  double Z = 0.0;
  for (int t = tid; t < n; t += 256) {
    const float c = is_l2 ? cval(x[t], shift, scale) : x[t];
    Z += exp((double)c - (double)m);
  }
  Z = block_sum_f64<4>(Z, shd);
  if (tid == 0) {
    double* o = stats + bh * 4;
    o[0] = shift;
    o[1] = scale;
    o[2] = n ? (double)m : 0.0;
    o[3] = n ? Z : 0.0;
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
  uint32_t bin;
  int wc[kSelWaves];
  int red[kSelWaves];
  int tpre[16 * kSelWaves];  // k_calsel: ties before (slot, wave), position order
};

// Run by wave 0: the largest bin whose suffix mass (bins at or above it)
// reaches `target`; records the bin and the mass strictly above it.  With
// from_total, the target is first set to max(ceil(p * total), 1).
template <int NB>
__device__ inline void find_bin(SelShared& S, bool from_total, float p) {
  const int lane = threadIdx.x;
  constexpr int PER = NB / 64;
  unsigned long long s = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) s += S.hist[lane * (PER + 1) + i];
  unsigned long long suf = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned long long v = __shfl_down(suf, o, 64);
    if (lane + o < 64) suf += v;
  }
  unsigned long long target;
  if (from_total) {
    const unsigned long long total = __shfl(suf, 0, 64);
    target = ceil_mul(p, total);
    if (target < 1) target = 1;
  } else {
    target = S.target;
  }
  const unsigned long long ok = __ballot(suf >= target);
  int L = __popcll(ok) - 1;  // suf falls with the lane: lanes 0..L reach the target
  L = L < 0 ? 0 : L;
  // inside lane L's PER bins: suffix sums over PER lanes, the same rule
  const unsigned long long base = __shfl(suf - s, L, 64);  // mass above the chunk
  const unsigned long long hv = lane < PER ? S.hist[L * (PER + 1) + lane] : 0ull;
  unsigned long long suf2 = hv;
#pragma unroll
  for (int o = 1; o < PER; o <<= 1) {
    const unsigned long long v = __shfl_down(suf2, o, 64);
    if (lane + o < PER) suf2 += v;
  }
  const unsigned long long ok2 = __ballot(lane < PER && base + suf2 >= target);
  int J = __popcll(ok2) - 1;
  J = J < 0 ? 0 : J;
  if (lane == J) {
    S.bin = L * PER + J;
    S.above = base + suf2 - hv;
  }
  if (from_total && lane == 0) S.target = target;
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

__global__ __launch_bounds__(kSelThreads) void k_select(Cand cand, const int8_t* __restrict__ metric,
                                                        const float* __restrict__ logit,
                                                        const float* __restrict__ l2,
                                                        int64_t cap_stride,
                                                        const double* __restrict__ stats,
                                                        float top_p, double wscale,
                                                        uint8_t* __restrict__ mask, CountOut co) {
  __shared__ SelShared S;
  const int h = blockIdx.x, b = blockIdx.y, hkv = gridDim.x, tid = threadIdx.x;
  const int n = cand.n(b, h);
  const int64_t bh = (int64_t)b * hkv + h;
  uint8_t* mk = mask + bh * cap_stride;
  if (n == 0) {
    if (tid == 0) co.put(bh, n, 0);
    return;
  }
  if (!(top_p < 1.0f)) {
    for (int t = tid; t < n; t += kSelThreads) mk[t] = 1;
    if (tid == 0) co.put(bh, n, n);
    return;
  }
  const bool is_l2 = aux_metric(metric, h);  // second score array
  const float* x = (is_l2 ? l2 : logit) + bh * cap_stride;
  const double shift = stats[bh * 4 + 0], scale = stats[bh * 4 + 1], m = stats[bh * 4 + 2];
  auto cv = [&](int t) -> float { return is_l2 ? cval(x[t], shift, scale) : x[t]; };

  // pass 1: top 11 bits of the key
  for (int i = tid; i < kHistSlots; i += kSelThreads) S.hist[i] = 0;
  __syncthreads();
  for (int t = tid; t < n; t += kSelThreads) {
    const float c = cv(t);
    const uint64_t w = wfix(c, m, wscale);
    if (w) atomicAdd(&S.hist[hslot<2048>(okey(c) >> 21)], (unsigned long long)w);
  }
  __syncthreads();
  if (tid < 64) find_bin<2048>(S, true, top_p);
  __syncthreads();
  const unsigned long long target = S.target;
  const uint32_t b1 = S.bin;
  unsigned long long above = S.above;
  __syncthreads();

  // pass 2: next 11 bits inside bin b1
  for (int i = tid; i < kHistSlots; i += kSelThreads) S.hist[i] = 0;
  if (tid == 0) S.target = target - above;
  __syncthreads();
  for (int t = tid; t < n; t += kSelThreads) {
    const float c = cv(t);
    const uint32_t k = okey(c);
    if ((k >> 21) == b1)
      atomicAdd(&S.hist[hslot<2048>((k >> 10) & 2047u)],
                (unsigned long long)wfix(c, m, wscale));
  }
  __syncthreads();
  if (tid < 64) find_bin<2048>(S, false, top_p);
  __syncthreads();
  const uint32_t b2 = S.bin;
  above += S.above;
  const unsigned long long t2 = S.target;
  __syncthreads();

  // pass 3: last 10 bits inside (b1, b2)
  for (int i = tid; i < kHistSlots; i += kSelThreads) S.hist[i] = 0;
  if (tid == 0) S.target = t2 - S.above;
  __syncthreads();
  const uint32_t pre = (b1 << 11) | b2;
  for (int t = tid; t < n; t += kSelThreads) {
    const float c = cv(t);
    const uint32_t k = okey(c);
    if ((k >> 10) == pre)
      atomicAdd(&S.hist[hslot<1024>(k & 1023u)], (unsigned long long)wfix(c, m, wscale));
  }
  __syncthreads();
  if (tid < 64) find_bin<1024>(S, false, top_p);
  __syncthreads();
  const uint32_t kstar = (pre << 10) | S.bin;
  above += S.above;
  // all tokens tied at K* carry the same weight; take r of them
  const unsigned long long wstar = wfix(okey_inv(kstar), m, wscale);
  const unsigned long long need = target - above;
  const unsigned long long r = (need + wstar - 1) / wstar;

  // pass 4: mask, ties by ascending position
  const int wv = tid >> 6, ln = tid & 63;
  unsigned long long carried = 0;
  int nsel = 0;
  for (int t0 = 0; t0 < n; t0 += kSelThreads) {
    const int t = t0 + tid;
    const bool valid = t < n;
    const uint32_t k = valid ? okey(cv(t)) : 0u;
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
  }
  // block sum of nsel
  int v = nsel;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if (ln == 0) S.red[wv] = v;
  __syncthreads();
  if (tid == 0) {
    int tot = 0;
    for (int i = 0; i < kSelWaves; ++i) tot += S.red[i];
    co.put(bh, n, tot);
  }
}

// ------------------------------------------------ calibrate + select -----
// Both steps for one (b, h) in one 1024-thread workgroup, with the head's
// scores held in registers (NPT per thread, token t = tid + 1024 i), so every
// pass after the first load runs from registers.  Same rules as k_calibrate
// and k_select; the float64 reductions run over 1024 threads instead of 256,
// so the diagnostic statistics may differ in their last bits.
template <int NPT>
__global__ __launch_bounds__(kSelThreads) void k_calsel(Cand cand, const int8_t* __restrict__ metric,
                                                        const float* __restrict__ logit,
                                                        const float* __restrict__ l2,
                                                        int64_t cap_stride,
                                                        double* __restrict__ stats, float top_p,
                                                        double wscale, uint8_t* __restrict__ mask,
                                                        CountOut co, int calib) {
  __shared__ SelShared S;
  // fixed-point weight of token tid + 1024 i at [i][tid], from pass 1 on
  __shared__ unsigned long long s_w[NPT * kSelThreads];
  __shared__ double shd[2 * kSelWaves];
  __shared__ float shf[kSelWaves];
  const int h = blockIdx.x, b = blockIdx.y, hkv = gridDim.x, tid = threadIdx.x;
  const int n = cand.n(b, h);
  const int64_t bh = (int64_t)b * hkv + h;
  uint8_t* mk = mask + bh * cap_stride;
  const bool is_l2 = aux_metric(metric, h);  // second score array
  if (n == 0) {
    if (tid == 0) {
      double* o = stats + bh * 4;
      o[0] = 0.0;
      o[1] = is_l2 ? 0.0 : 1.0;
      o[2] = 0.0;
      o[3] = 0.0;
      co.put(bh, n, 0);
    }
    return;
  }
  const float* xs = logit + bh * cap_stride;
  float c[NPT];
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int t = tid + kSelThreads * i;
    c[i] = t < n ? xs[t] : 0.f;
  }
  double shift = 0.0, scale = 1.0;
  if (is_l2 && calib == HARDKV_CALIB_ENTROPY) {
    const float* ss = l2 + bh * cap_stride;
    float sv[NPT];
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int t = tid + kSelThreads * i;
      sv[i] = t < n ? ss[t] : 0.f;
    }
    entropy_temperature<kSelWaves>(
        [&](auto f) {
#pragma unroll
          for (int i = 0; i < NPT; ++i)
            if (tid + kSelThreads * i < n) f(c[i]);
        },
        [&](auto f) {
#pragma unroll
          for (int i = 0; i < NPT; ++i)
            if (tid + kSelThreads * i < n) f(sv[i]);
        },
        shd, shf, shift, scale);
#pragma unroll
    for (int i = 0; i < NPT; ++i) c[i] = cval(sv[i], shift, scale);
  } else if (is_l2) {
    const float* ss = l2 + bh * cap_stride;
    float sv[NPT];
    double sx = 0.0, sy = 0.0;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int t = tid + kSelThreads * i;
      sv[i] = t < n ? ss[t] : 0.f;
      sx += (double)c[i];
      sy += (double)sv[i];
    }
    sx = block_sum_f64<kSelWaves>(sx, shd);
    sy = block_sum_f64<kSelWaves>(sy, shd);
    const double mux = sx / n, mus = sy / n;
    double vx = 0.0, vy = 0.0;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      if (tid + kSelThreads * i < n) {
        const double dx = (double)c[i] - mux, dy = (double)sv[i] - mus;
        vx += dx * dx;
        vy += dy * dy;
      }
    }
    vx = block_sum_f64<kSelWaves>(vx, shd);
    vy = block_sum_f64<kSelWaves>(vy, shd);
    const double sdx = sqrt(vx / n), sds = sqrt(vy / n);
    if (sdx == 0.0 || sds == 0.0) {
      shift = 0.0;
      scale = 0.0;
    } else {
      shift = mus;
      scale = sdx / sds;
    }
#pragma unroll
    for (int i = 0; i < NPT; ++i) c[i] = cval(sv[i], shift, scale);
  }
  float mloc = -INFINITY;
#pragma unroll
  for (int i = 0; i < NPT; ++i)
    if (tid + kSelThreads * i < n) mloc = fmaxf(mloc, c[i]);
  const double m = (double)block_max_f32<kSelWaves>(mloc, shf);

  // pass 1: weights, Z, and the histogram of the top 11 key bits
  for (int i = tid; i < kHistSlots; i += kSelThreads) S.hist[i] = 0;
  __syncthreads();
  double Z = 0.0;
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    uint64_t w = 0;
    if (tid + kSelThreads * i < n) {
      const double wd = exp((double)c[i] - m);
      Z += wd;
      w = (uint64_t)__double2ull_rn(wd * wscale);  // = wfix(c, m, wscale)
      if (w) atomicAdd(&S.hist[hslot<2048>(okey(c[i]) >> 21)], (unsigned long long)w);
    }
    s_w[i * kSelThreads + tid] = w;
  }
  Z = block_sum_f64<kSelWaves>(Z, shd);  // contains the barrier before find_bin
  if (tid == 0) {
    double* o = stats + bh * 4;
    o[0] = shift;
    o[1] = scale;
    o[2] = m;
    o[3] = Z;
  }
  if (!(top_p < 1.0f)) {
#pragma unroll
    for (int i = 0; i < NPT; ++i)
      if (tid + kSelThreads * i < n) mk[tid + kSelThreads * i] = 1;
    if (tid == 0) co.put(bh, n, n);
    return;
  }
  if (tid < 64) find_bin<2048>(S, true, top_p);
  __syncthreads();
  const unsigned long long target = S.target;
  const uint32_t b1 = S.bin;
  unsigned long long above = S.above;
  __syncthreads();

  for (int i = tid; i < kHistSlots; i += kSelThreads) S.hist[i] = 0;
  if (tid == 0) S.target = target - above;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const uint32_t k = okey(c[i]);
    if (tid + kSelThreads * i < n && (k >> 21) == b1)
      atomicAdd(&S.hist[hslot<2048>((k >> 10) & 2047u)], s_w[i * kSelThreads + tid]);
  }
  __syncthreads();
  if (tid < 64) find_bin<2048>(S, false, top_p);
  __syncthreads();
  const uint32_t b2 = S.bin;
  above += S.above;
  const unsigned long long t2 = S.target;
  __syncthreads();

  for (int i = tid; i < kHistSlots; i += kSelThreads) S.hist[i] = 0;
  if (tid == 0) S.target = t2 - S.above;
  __syncthreads();
  const uint32_t pre = (b1 << 11) | b2;
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const uint32_t k = okey(c[i]);
    if (tid + kSelThreads * i < n && (k >> 10) == pre)
      atomicAdd(&S.hist[hslot<1024>(k & 1023u)], s_w[i * kSelThreads + tid]);
  }
  __syncthreads();
  if (tid < 64) find_bin<1024>(S, false, top_p);
  __syncthreads();
  const uint32_t kstar = (pre << 10) | S.bin;
  above += S.above;
  const unsigned long long wstar = wfix(okey_inv(kstar), m, wscale);
  const unsigned long long need = target - above;
  const unsigned long long r = (need + wstar - 1) / wstar;
  // every token tied at K* has weight wstar, so the bin holds mass / wstar of
  // them; when r reaches that count all are taken and no ranking is needed
  const unsigned long long ntie = S.hist[hslot<1024>(S.bin)] / wstar;

  // Tokens tied at K* are taken in position order t = tid + 1024 i, i.e.
  // ordered by (slot i, wave, lane): count the ties of every (slot, wave),
  // scan them once (wave 0), then each tie's rank is its entry plus the tied
  // lanes below it in its wave's ballot.
  const int wv = tid >> 6, ln = tid & 63;
  const bool rank_ties = r < ntie;  // uniform
  uint32_t tmask = 0;
#pragma unroll
  for (int i = 0; i < NPT; ++i)
    if (tid + kSelThreads * i < n && okey(c[i]) == kstar) tmask |= 1u << i;
  if (rank_ties) {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const unsigned long long bal = __ballot((tmask >> i) & 1u);
      if (ln == 0) S.tpre[i * kSelWaves + wv] = __popcll(bal);
    }
    __syncthreads();
    if (tid < 64) {
      constexpr int PER = NPT * kSelWaves / 64;  // entries per lane, in order
      int e[PER], sum = 0;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        e[j] = S.tpre[tid * PER + j];
        sum += e[j];
      }
      int incl = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o, 64);
        if (tid >= o) incl += u;
      }
      int run = incl - sum;
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        S.tpre[tid * PER + j] = run;
        run += e[j];
      }
    }
    __syncthreads();
  }
  int nsel = 0;
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    if (kSelThreads * i >= n) break;  // uniform
    const int t = tid + kSelThreads * i;
    const bool valid = t < n;
    const bool tie = (tmask >> i) & 1u;
    bool take_tie = tie;
    if (rank_ties) {
      const unsigned long long bal = __ballot(tie);
      const unsigned long long rank = (unsigned long long)S.tpre[i * kSelWaves + wv] +
                                      __popcll(bal & ((1ull << ln) - 1ull));
      take_tie = tie && rank < r;
    }
    const bool sel = valid && (okey(c[i]) > kstar || take_tie);
    if (valid) mk[t] = sel ? 1 : 0;
    nsel += sel;
  }
  int v = nsel;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if (ln == 0) S.red[wv] = v;
  __syncthreads();
  if (tid == 0) {
    int tot = 0;
    for (int j = 0; j < kSelWaves; ++j) tot += S.red[j];
    co.put(bh, n, tot);
  }
}

static CountOut count_out(const SelectArgs& a) { return CountOut{a.count, a.mode, a.policy, a.cand.W}; }

__global__ __launch_bounds__(256) void k_plan(Cand cand, int B, const int32_t* __restrict__ count,
                                              uint8_t* __restrict__ mode, hardkv_policy pol) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= B * cand.hkv) return;
  const int n = cand.n(i / cand.hkv, i % cand.hkv);
  int k = count[i];
  k = k < 0 ? 0 : (k > n ? n : k);
  mode[i] = plan_mode(pol, n, k, cand.W);
}

void launch_plan(const SelectArgs& a, hipStream_t st) {
  observe("k_plan", st);
  hipLaunchKernelGGL(k_plan, dim3(ceil_div((int64_t)a.B * a.hkv, 256)), dim3(256), 0, st, a.cand,
                     a.B, a.count, a.mode, a.policy);
}

// Exclusive scan of the rewritten heads' row needs in (b, h) order, one
// workgroup, 1024 heads per round with the running total carried.
__global__ __launch_bounds__(kSelThreads) void k_pack(int n_heads, const int32_t* __restrict__ count,
                                                      int cap, uint8_t* __restrict__ mode,
                                                      int32_t* __restrict__ offset,
                                                      int packed_rows) {
  __shared__ long long s_w[kSelWaves];
  const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63;
  long long run = 0;
  for (int base = 0; base < n_heads; base += kSelThreads) {
    const int i = base + tid;
    const bool rw = i < n_heads && mode[i] == HARDKV_MODE_REWRITE;
    int need = 0;
    if (rw) {
      const int k = count[i];
      need = k < 0 ? 0 : (k > cap ? cap : k);
    }
    long long incl = need;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const long long u = __shfl_up(incl, o, 64);
      if (ln >= o) incl += u;
    }
    if (ln == 63) s_w[wv] = incl;
    __syncthreads();
    long long before = run, total = run;
    for (int j = 0; j < kSelWaves; ++j) {
      if (j < wv) before += s_w[j];
      total += s_w[j];
    }
    const long long off = before + incl - need;
    if (i < n_heads) {
      offset[i] = (int32_t)off;
      if (rw && off + need > packed_rows) mode[i] = HARDKV_MODE_SPARSE;
    }
    run = total;
    __syncthreads();
  }
}

void launch_pack(int n_heads, const int32_t* count, int cap, uint8_t* mode, int32_t* offset,
                 int packed_rows, hipStream_t st) {
  observe("k_pack", st);
  hipLaunchKernelGGL(k_pack, dim3(1), dim3(kSelThreads), 0, st, n_heads, count, cap, mode, offset,
                     packed_rows);
}

bool calsel_fits(int max_cand) { return max_cand <= 16 * kSelThreads; }

void launch_calsel(const SelectArgs& a, int max_cand, hipStream_t st) {
  observe("k_calsel", st);
  const dim3 grid(a.hkv, a.B), blk(kSelThreads);
  if (max_cand <= 4 * kSelThreads)
    hipLaunchKernelGGL(k_calsel<4>, grid, blk, 0, st, a.cand, a.metric, a.logit, a.l2,
                       a.cap_stride, a.stats, a.top_p, mass_scale(a.cand.cap), a.mask,
                       count_out(a), a.calib);
  else
    hipLaunchKernelGGL(k_calsel<16>, grid, blk, 0, st, a.cand, a.metric, a.logit, a.l2,
                       a.cap_stride, a.stats, a.top_p, mass_scale(a.cand.cap), a.mask,
                       count_out(a), a.calib);
}

void launch_calibrate(const SelectArgs& a, hipStream_t st) {
  observe("k_calibrate", st);
  hipLaunchKernelGGL(k_calibrate, dim3(a.hkv, a.B), dim3(256), 0, st, a.cand, a.metric, a.logit,
                     a.l2, a.cap_stride, a.stats, a.calib);
}

void launch_select(const SelectArgs& a, hipStream_t st) {
  observe("k_select", st);
  hipLaunchKernelGGL(k_select, dim3(a.hkv, a.B), dim3(kSelThreads), 0, st, a.cand, a.metric,
                     a.logit, a.l2, a.cap_stride, (const double*)a.stats, a.top_p,
                     mass_scale(a.cand.cap), a.mask, count_out(a));
}

}  // namespace hk
