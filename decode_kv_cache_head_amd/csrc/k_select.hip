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
#include <algorithm>
#include <type_traits>

#include "select_core.h"

namespace hk {

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
// One 1024-thread workgroup per (b, h); every pass reads the head's scores
// with sixteen loads in flight per thread (each thread adds its values in
// position order, so the float64 sums do not depend on the batching).
//   logit heads:   m = max x; Z = sum exp(x - m)
//   spread rule:   sums of x and s and max s; then the two squared
//                  deviations; shift = mean s, scale = sd(x) / sd(s); the
//                  calibration is non-decreasing in s, so m = cval(max s)
//   entropy rule:  the bisection of entropy_temperature, then m and Z
// exp of non-positive arguments through exp_nonpos.
constexpr int kCalThreads = 1024;
constexpr int kCalWaves = kCalThreads / 64;

__global__ __launch_bounds__(kCalThreads) void k_calibrate(Cand cand, const int8_t* __restrict__ metric,
                                                           const float* __restrict__ logit,
                                                           const float* __restrict__ l2,
                                                           int64_t cap_stride,
                                                           double* __restrict__ stats, int calib,
                                                           bool with_z) {
  constexpr int U = 16;
  __shared__ double shd[2 * kCalWaves];
  __shared__ float shf[kCalWaves];
  __shared__ double s_et[64];
  const int hkv = gridDim.x, tid = threadIdx.x;
  int b, h;
  head_of_block(b, h);
  const int n = cand.n(b, h);
  const int64_t bh = (int64_t)b * hkv + h;
  const float* x = logit + bh * cap_stride;
  const float* sv = l2 + bh * cap_stride;
  const bool is_l2 = aux_metric(metric, h);  // second score array
  exp_table_init(s_et);
  double shift = 0.0, scale = 1.0;
  float m = -INFINITY;
  if (is_l2 && calib == HARDKV_CALIB_ENTROPY) {
    shift = 0.0;
    scale = 0.0;
    if (n > 0)  // uniform over the workgroup
      entropy_temperature<kCalWaves>(
          [&](auto f) { each_value<kCalThreads, U>(x, n, [&](int, float v) { f(v); }); },
          [&](auto f) { each_value<kCalThreads, U>(sv, n, [&](int, float v) { f(v); }); },
          shd, shf, shift, scale);
    float ml = -INFINITY;
    each_value<kCalThreads, U>(sv, n, [&](int, float v) { ml = fmaxf(ml, cval(v, shift, scale)); });
    m = block_max_f32<kCalWaves>(ml, shf);
  } else if (is_l2) {
    double sx = 0.0, sy = 0.0;
    float smax = -INFINITY;
    for (int t0 = tid; t0 < n; t0 += kCalThreads * U) {
      float a[U], c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = t0 + u * kCalThreads;
        a[u] = t < n ? x[t] : 0.f;
        c[u] = t < n ? sv[t] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (t0 + u * kCalThreads < n) {
          sx += (double)a[u];
          sy += (double)c[u];
          smax = fmaxf(smax, c[u]);
        }
      }
    }
    block_sum2_f64<kCalWaves>(sx, sy, shd);
    smax = block_max_f32<kCalWaves>(smax, shf);
    const double mux = n ? sx / n : 0.0, mus = n ? sy / n : 0.0;
    double vx = 0.0, vy = 0.0;
    for (int t0 = tid; t0 < n; t0 += kCalThreads * U) {
      float a[U], c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = t0 + u * kCalThreads;
        a[u] = t < n ? x[t] : 0.f;
        c[u] = t < n ? sv[t] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (t0 + u * kCalThreads < n) {
          const double dx = (double)a[u] - mux, dy = (double)c[u] - mus;
          vx += dx * dx;
          vy += dy * dy;
        }
      }
    }
    block_sum2_f64<kCalWaves>(vx, vy, shd);
    const double sdx = n ? sqrt(vx / n) : 0.0, sds = n ? sqrt(vy / n) : 0.0;
    if (sdx == 0.0 || sds == 0.0) {
      shift = 0.0;
      scale = 0.0;
    } else {
      shift = mus;
      scale = sdx / sds;
    }
    m = n ? cval(smax, shift, scale) : -INFINITY;
  } else {
    float ml = -INFINITY;
    each_value<kCalThreads, U>(x, n, [&](int, float v) { ml = fmaxf(ml, v); });
    m = block_max_f32<kCalWaves>(ml, shf);
  }
  const float* src = is_l2 ? sv : x;
  double Z = 0.0;
  if (with_z) {  // uniform
    each_value<kCalThreads, U>(src, n, [&](int, float v) {
      const float c = is_l2 ? cval(v, shift, scale) : v;
      Z += exp_nonpos((double)c - (double)m, s_et);
    });
    Z = block_sum_f64<kCalWaves>(Z, shd);
  }
  if (tid == 0) {
    double* o = stats + bh * 4;
    o[0] = shift;
    o[1] = scale;
    o[2] = n ? (double)m : 0.0;
    if (with_z) o[3] = n ? Z : 0.0;
  }
}

// --------------------------------------------------------------- select ---
__global__ __launch_bounds__(kSelThreads) void k_select(Cand cand, const int8_t* __restrict__ metric,
                                                        const float* __restrict__ logit,
                                                        const float* __restrict__ l2,
                                                        int64_t cap_stride,
                                                        double* __restrict__ stats,
                                                        float top_p, double wscale,
                                                        uint8_t* __restrict__ mask, CountOut co,
                                                        bool write_z, int32_t* __restrict__ kept,
                                                        int kept_stride) {
  __shared__ SelShared S;
  __shared__ double s_et[64];
  const int hkv = gridDim.x, tid = threadIdx.x;
  int b, h;
  head_of_block(b, h);
  const int n = cand.n(b, h);
  const int64_t bh = (int64_t)b * hkv + h;
  uint8_t* mk = mask + bh * cap_stride;
  if (n == 0) {
    if (tid == 0) co.put(bh, n, 0);
    return;
  }
  exp_table_init(s_et);
  const int nblk = (n + kKeptBlk - 1) / kKeptBlk;
  const bool count = kept != nullptr && nblk <= kKeptMaxBlks;
  if (!(top_p < 1.0f)) {
    for (int t = tid; t < n; t += kSelThreads) mk[t] = 1;
    if (tid == 0) co.put(bh, n, n);
    if (count)
      for (int i = tid; i < nblk; i += kSelThreads) kept[bh * kept_stride + i] = min(kKeptBlk, n - i * kKeptBlk);
    return;
  }
  const bool is_l2 = aux_metric(metric, h);  // second score array
  const float* x = (is_l2 ? l2 : logit) + bh * cap_stride;
  const double shift = stats[bh * 4 + 0], scale = stats[bh * 4 + 1], m = stats[bh * 4 + 2];
  auto cv = [&](float raw) -> float { return is_l2 ? cval(raw, shift, scale) : raw; };

  const int nsel = select_head<kSelThreads>(S, n, x, cv, m, top_p, wscale, s_et, mk, count);
  // Z as the fixed-point total of pass 1 (within n 2^-48 of the float64 sum)
  if (write_z && tid == 0) stats[bh * 4 + 3] = (double)S.total / wscale;
  // block sum of nsel
  const int wv = tid >> 6, ln = tid & 63;
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
  if (count)
    for (int i = tid; i < nblk; i += kSelThreads) kept[bh * kept_stride + i] = S.blkcnt[i];
}

// ------------------------------------------------ calibrate + select -----
// Both steps for one (b, h) in one 1024-thread workgroup, with the head's
// scores held in registers (NPT per thread, token t = tid + 1024 i), so every
// pass after the first load runs from registers.  Same rules as k_calibrate
// and k_select; the float64 reductions run over 1024 threads instead of 256,
// so the diagnostic statistics may differ in their last bits.  AUX false:
// launched without a metric array, every head ranks by its logit, and the
// second-metric paths (moments, entropy bisection) are compiled out, which
// keeps the 16-slot form inside the 128 registers a 1024-thread workgroup
// allows (with them it spilled to scratch).
template <int NPT, bool AUX>
__global__ __launch_bounds__(kSelThreads) void k_calsel(Cand cand, const int8_t* __restrict__ metric,
                                                        const float* __restrict__ logit,
                                                        const float* __restrict__ l2,
                                                        int64_t cap_stride,
                                                        double* __restrict__ stats, float top_p,
                                                        double wscale, uint8_t* __restrict__ mask,
                                                        CountOut co, int calib,
                                                        int32_t* __restrict__ kept,
                                                        int kept_stride) {
  __shared__ SelShared S;
  // fixed-point weight of token tid + 1024 i at [i][tid], from pass 1 on
  __shared__ unsigned long long s_w[NPT * kSelThreads];
  __shared__ double shd[2 * kSelWaves];
  __shared__ float shf[kSelWaves];
  __shared__ double s_et[64];
  const int hkv = gridDim.x, tid = threadIdx.x;
  int b, h;
  head_of_block(b, h);
  const int n = cand.n(b, h);
  const int64_t bh = (int64_t)b * hkv + h;
  uint8_t* mk = mask + bh * cap_stride;
  const bool is_l2 = AUX && aux_metric(metric, h);  // second score array
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
  double shift = 0.0, scale = 1.0;
  if (!is_l2) {
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int t = tid + kSelThreads * i;
      c[i] = t < n ? xs[t] : 0.f;
    }
  } else {
    // a second-metric head: its logits and metric values wait in this
    // thread's own weight slots (free until pass 1 writes the weights there;
    // slot i holds the logit in its low and the metric in its high half),
    // not in registers, while the temperature is worked out
    float* sl = reinterpret_cast<float*>(s_w) + 2 * tid;
    constexpr int SV = 2 * kSelThreads;  // floats per row of weight slots
    const float* ss = l2 + bh * cap_stride;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int t = tid + kSelThreads * i;
      sl[i * SV] = t < n ? xs[t] : 0.f;
      sl[i * SV + 1] = t < n ? ss[t] : 0.f;
    }
    if (calib == HARDKV_CALIB_ENTROPY) {
      entropy_temperature<kSelWaves>(
          [&](auto f) {
#pragma unroll
            for (int i = 0; i < NPT; ++i)
              if (tid + kSelThreads * i < n) f(sl[i * SV]);
          },
          [&](auto f) {
#pragma unroll
            for (int i = 0; i < NPT; ++i)
              if (tid + kSelThreads * i < n) f(sl[i * SV + 1]);
          },
          shd, shf, shift, scale);
    } else {
      double sx = 0.0, sy = 0.0;
#pragma unroll
      for (int i = 0; i < NPT; ++i) {
        sx += (double)sl[i * SV];
        sy += (double)sl[i * SV + 1];
      }
      sx = block_sum_f64<kSelWaves>(sx, shd);
      sy = block_sum_f64<kSelWaves>(sy, shd);
      const double mux = sx / n, mus = sy / n;
      double vx = 0.0, vy = 0.0;
#pragma unroll
      for (int i = 0; i < NPT; ++i) {
        if (tid + kSelThreads * i < n) {
          const double dx = (double)sl[i * SV] - mux, dy = (double)sl[i * SV + 1] - mus;
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
    }
#pragma unroll
    for (int i = 0; i < NPT; ++i) c[i] = cval(sl[i * SV + 1], shift, scale);
  }
  float mloc = -INFINITY;
#pragma unroll
  for (int i = 0; i < NPT; ++i)
    if (tid + kSelThreads * i < n) mloc = fmaxf(mloc, c[i]);
  exp_table_init(s_et);  // read after the barriers of the block maximum
  const double m = (double)block_max_f32<kSelWaves>(mloc, shf);

  // pass 1: weights, Z, and the histogram of the top 11 key bits; from here
  // on the tokens are known by their order-preserving keys
  for (int i = tid; i < kHistSlots; i += kSelThreads) S.hist[i] = 0;
  for (int i = tid; i < 2 * NPT; i += kSelThreads) S.blkcnt[i] = 0;
  if (tid == 0) S.tally = 0ull;
  __syncthreads();
  uint32_t key[NPT];
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    key[i] = okey(c[i]);
    uint64_t w = 0;
    if (tid + kSelThreads * i < n) {
      w = fix_round(exp_nonpos((double)c[i] - m, s_et) * wscale);  // = wfix(c, m, wscale, s_et)
      if (w) atomicAdd(&S.hist[hslot<2048>(key[i] >> 21)], (unsigned long long)w);
    }
    s_w[i * kSelThreads + tid] = w;
  }
  __syncthreads();
  if (!(top_p < 1.0f)) {
#pragma unroll
    for (int i = 0; i < NPT; ++i)
      if (tid + kSelThreads * i < n) mk[tid + kSelThreads * i] = 1;
    if (tid == 0) co.put(bh, n, n);
    if (kept)
      for (int i = tid; i < (n + kKeptBlk - 1) / kKeptBlk; i += kSelThreads)
        kept[bh * kept_stride + i] = min(kKeptBlk, n - i * kKeptBlk);
  }
  if (tid < 64) find_bin<2048>(S, true, top_p);
  __syncthreads();
  if (tid == 0) {
    // Z as the fixed-point total (within n 2^-48 of the float64 sum; the
    // step reads only shift, scale and m downstream)
    double* o = stats + bh * 4;
    o[0] = shift;
    o[1] = scale;
    o[2] = m;
    o[3] = (double)S.total / wscale;
  }
  if (!(top_p < 1.0f)) return;  // uniform
  const unsigned long long target = S.target;
  const uint32_t b1 = S.bin;
  unsigned long long above = S.above;
  __syncthreads();

  for (int i = tid; i < kHistSlots; i += kSelThreads) S.hist[i] = 0;
  if (tid == 0) S.target = target - above;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    if (tid + kSelThreads * i < n && (key[i] >> 21) == b1)
      atomicAdd(&S.hist[hslot<2048>((key[i] >> 10) & 2047u)], s_w[i * kSelThreads + tid]);
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
    if (tid + kSelThreads * i < n && (key[i] >> 10) == pre)
      atomicAdd(&S.hist[hslot<1024>(key[i] & 1023u)], s_w[i * kSelThreads + tid]);
  }
  __syncthreads();
  if (tid < 64) find_bin<1024>(S, false, top_p);
  __syncthreads();
  const uint32_t kstar = (pre << 10) | S.bin;
  above += S.above;
  const unsigned long long wstar = wfix(okey_inv(kstar), m, wscale, s_et);
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
    if (tid + kSelThreads * i < n && key[i] == kstar) tmask |= 1u << i;
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
  // mask: for each slot the wave's 64 decisions (tokens 1024 i + 64 wv ..)
  // come from one ballot; lanes 0..3 each put 16 of them as bytes into LDS
  // (the histogram's space, free now), then every thread stores 16
  // consecutive bytes: whole-line stores instead of 64-byte pieces
  static_assert(NPT * kSelThreads <= (int)sizeof(S.hist), "mask staging");
  uint8_t* sm = reinterpret_cast<uint8_t*>(S.hist);
  __syncthreads();  // every read of the histogram is done
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
    const bool sel = valid && (key[i] > kstar || take_tie);
    const unsigned long long bal = __ballot(sel);
    nsel += __popcll(bal);
    // slot i is tokens [1024 i, 1024 i + 1024): waves 0-7 the first 512
    if (kept && ln == 0 && bal) atomicAdd(&S.blkcnt[2 * i + (wv >= 8)], (int)__popcll(bal));
    if (ln < 4) {
      const uint32_t bits = (uint32_t)(bal >> (16 * ln)) & 0xffffu;
      // each nibble of bits becomes four 0/1 bytes
      uint4 v;
      v.x = ((bits & 15u) * 0x00204081u) & 0x01010101u;
      v.y = (((bits >> 4) & 15u) * 0x00204081u) & 0x01010101u;
      v.z = (((bits >> 8) & 15u) * 0x00204081u) & 0x01010101u;
      v.w = (((bits >> 12) & 15u) * 0x00204081u) & 0x01010101u;
      *(uint4*)(sm + kSelThreads * i + 64 * wv + 16 * ln) = v;
    }
  }
  __syncthreads();
  if (kept)
    for (int i = tid; i < (n + kKeptBlk - 1) / kKeptBlk; i += kSelThreads)
      kept[bh * kept_stride + i] = S.blkcnt[i];
  for (int t0 = 16 * tid; t0 < n; t0 += 16 * kSelThreads) {
    if (t0 + 16 <= n && ((uintptr_t)(mk + t0) & 15) == 0) {
      *(uint4*)(mk + t0) = *(const uint4*)(sm + t0);
    } else {
      for (int q = 0; q < 16 && t0 + q < n; ++q) mk[t0 + q] = sm[t0 + q];
    }
  }
  // count: the waves add (selected << 32 | 1) to one LDS word; the wave that
  // finds the other fifteen already there writes the total
  if (ln == 0) {
    const unsigned long long old =
        atomicAdd(&S.tally, ((unsigned long long)nsel << 32) | 1ull);
    if ((old & 0xffffffffull) == kSelWaves - 1) co.put(bh, n, (int)(old >> 32) + nsel);
  }
}

// ------------------------------------------------------ block selection ---
// Top-p over whole blocks (section 2.C: selected blocks are moved into
// contiguous ranges).  One 1024-thread workgroup per (b, h), after
// calibrate: block j holds the candidates at positions [j bs, (j + 1) bs);
// its mass is the integer sum of its candidates' fixed-point weights
// wfix(c, m) (LDS atomics: deterministic).  The blocks are sorted by (mass
// desc, block id asc) with a bitonic network in LDS, a block-wide scan of the
// sorted masses finds the shortest prefix reaching ceil(p * total), and every
// candidate of a kept block is kept.
__global__ __launch_bounds__(kSelThreads) void k_blocksel(Cand cand, const int8_t* __restrict__ metric,
                                                          const float* __restrict__ logit,
                                                          const float* __restrict__ l2,
                                                          int64_t cap_stride,
                                                          const double* __restrict__ stats,
                                                          float top_p, double wscale,
                                                          uint8_t* __restrict__ mask, CountOut co,
                                                          int bs) {
  constexpr int NT = kSelThreads;
  __shared__ unsigned long long s_mass[kBlockSelMax];
  __shared__ uint16_t s_idx[kBlockSelMax];
  __shared__ uint8_t s_kept[kBlockSelMax];
  __shared__ unsigned long long s_wsum[kSelWaves];
  __shared__ double s_et[64];
  __shared__ int s_k;
  __shared__ int s_red[kSelWaves];
  const int hkv = gridDim.x, tid = threadIdx.x;
  int b, h;
  head_of_block(b, h);
  const int wv = tid >> 6, ln = tid & 63;
  const int n = cand.n(b, h);
  const int64_t bh = (int64_t)b * hkv + h;
  uint8_t* mk = mask + bh * cap_stride;
  if (n == 0) {
    if (tid == 0) co.put(bh, n, 0);
    return;
  }
  if (!(top_p < 1.0f)) {
    for (int t = tid; t < n; t += NT) mk[t] = 1;
    if (tid == 0) co.put(bh, n, n);
    return;
  }
  exp_table_init(s_et);
  const int S = cand.sinks;                 // position of candidate 0
  const int jb0 = S / bs;
  const int nb = (S + n - 1) / bs - jb0 + 1;  // <= kBlockSelMax (validated)
  int np = 64;
  while (np < nb) np <<= 1;
  for (int i = tid; i < np; i += NT) {
    s_mass[i] = 0ull;
    s_idx[i] = (uint16_t)i;  // entries past nb: mass 0, ids above every block's
    s_kept[i] = 0;
  }
  if (tid == 0) s_k = np;
  __syncthreads();
  const bool is_l2 = aux_metric(metric, h);
  const float* x = (is_l2 ? l2 : logit) + bh * cap_stride;
  const double shift = stats[bh * 4 + 0], scale = stats[bh * 4 + 1], m = stats[bh * 4 + 2];
  each_value<NT, 8>(x, n, [&](int t, float raw) {
    const float c = is_l2 ? cval(raw, shift, scale) : raw;
    const uint64_t w = wfix(c, m, wscale, s_et);
    if (w) atomicAdd(&s_mass[(S + t) / bs - jb0], (unsigned long long)w);
  });
  __syncthreads();
  // bitonic sort: entry i precedes entry j when its mass is larger, or equal
  // with a lower block id
  for (int k = 2; k <= np; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < np; i += NT) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const unsigned long long ma = s_mass[i], mb = s_mass[ixj];
          const uint16_t ia = s_idx[i], ib = s_idx[ixj];
          const bool a_first = ma > mb || (ma == mb && ia < ib);
          const bool forward = (i & k) == 0;
          if (forward != a_first) {
            s_mass[i] = mb;
            s_mass[ixj] = ma;
            s_idx[i] = ib;
            s_idx[ixj] = ia;
          }
        }
      }
      __syncthreads();
    }
  }
  // inclusive prefix of the sorted masses: thread tid takes entries
  // [tid E, tid E + E), a wave scan, then the waves below in order
  const int E = np > NT ? np / NT : 1;
  unsigned long long run = 0;
  if (tid * E < np)
    for (int e = 0; e < E; ++e) run += s_mass[tid * E + e];
  const unsigned long long incl = wave_prefix_u64(run);
  if (ln == 63) s_wsum[wv] = incl;
  __syncthreads();
  unsigned long long before = 0, total = 0;
  for (int i = 0; i < kSelWaves; ++i) {
    if (i < wv) before += s_wsum[i];
    total += s_wsum[i];
  }
  unsigned long long target = ceil_mul(top_p, total);
  if (target < 1) target = 1;
  unsigned long long acc = before + incl - run;
  if (tid * E < np) {
    for (int e = 0; e < E; ++e) {
      acc += s_mass[tid * E + e];
      if (acc >= target) {
        atomicMin(&s_k, tid * E + e + 1);
        break;
      }
    }
  }
  __syncthreads();
  const int kb = min(s_k, nb);
  for (int r = tid; r < kb; r += NT) s_kept[s_idx[r]] = 1;
  __syncthreads();
  int nsel = 0;
  for (int t = tid; t < n; t += NT) {
    const uint8_t kept = s_kept[(S + t) / bs - jb0];
    mk[t] = kept;
    nsel += kept;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) nsel += __shfl_xor(nsel, o, 64);
  if (ln == 0) s_red[wv] = nsel;
  __syncthreads();
  if (tid == 0) {
    int tot = 0;
    for (int i = 0; i < kSelWaves; ++i) tot += s_red[i];
    co.put(bh, n, tot);
  }
}

static CountOut count_out(const SelectArgs& a) { return CountOut{a.count, a.mode, a.policy, a.cand.W}; }

void launch_blocksel(const SelectArgs& a, hipStream_t st) {
  observe("k_blocksel", st);
  hipLaunchKernelGGL(k_blocksel, dim3(a.hkv, a.B), dim3(kSelThreads), 0, st, a.cand, a.metric,
                     a.logit, a.l2, a.cap_stride, (const double*)a.stats, a.top_p,
                     mass_scale(a.cand.cap), a.mask, count_out(a), a.block);
}

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

// ------------------------------------------- rewritten tier's block manager --
// (section 2.C "Metadata": a head-wise block manager for head-adaptive
// budgets under static shapes.)
__global__ __launch_bounds__(256) void k_tier_init(TierBlocks tb, int n_heads) {
  const int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x, stride = (int64_t)gridDim.x * 256;
  for (int64_t i = i0; i < tb.nblocks; i += stride) tb.free_ids[i] = (int32_t)i;
  for (int64_t i = i0; i < n_heads; i += stride) tb.held[i] = 0;
  for (int64_t i = i0; i < (int64_t)n_heads * tb.maxb; i += stride) tb.table[i] = -1;
  if (i0 == 0) tb.free_top[0] = tb.nblocks;
}

void launch_tier_init(const TierBlocks& tb, int n_heads, hipStream_t st) {
  observe("k_tier_init", st);
  const int64_t work = std::max<int64_t>((int64_t)n_heads * tb.maxb, tb.nblocks);
  const int grid = (int)std::min<int64_t>(std::max<int64_t>(ceil_div(work, 256), 1), 1024);
  hipLaunchKernelGGL(k_tier_init, dim3(grid), dim3(256), 0, st, tb, n_heads);
}

// Exclusive scan of v over the heads in (b, h) order into s[0 .. n] (s[n] =
// total), 1024 heads per round with the running total carried; returns the
// total.  Every thread returns with the scan visible in LDS.
template <typename F>
__device__ inline int tier_scan(int n, F val, int* s, int* s_w) {
  const int tid = threadIdx.x, wv = tid >> 6, ln = tid & 63;
  int run = 0;
  for (int base = 0; base < n; base += kSelThreads) {
    const int i = base + tid;
    const int v = i < n ? val(i) : 0;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o, 64);
      if (ln >= o) incl += u;
    }
    if (ln == 63) s_w[wv] = incl;
    __syncthreads();
    int before = run, total = run;
    for (int j = 0; j < kSelWaves; ++j) {
      if (j < wv) before += s_w[j];
      total += s_w[j];
    }
    if (i < n) s[i] = before + incl - v;
    run = total;
    __syncthreads();
  }
  if (tid == 0) s[n] = run;
  __syncthreads();
  return run;
}

// The head whose scan range [s[i], s[i + 1]) holds entry e (s ascending,
// e < s[n]): the last i with s[i] <= e.
__device__ inline int tier_head_of(const int* s, int n, int e) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s[mid] <= e) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// One workgroup: every head returns its blocks to the free stack, then the
// rewritten heads take ceil(k / tb) blocks each from the top, in (b, h)
// order; a head that does not fit (nor any after it) is sparse-loaded.
__global__ __launch_bounds__(kSelThreads) void k_tier_alloc(TierBlocks tb, int n_heads,
                                                            const int32_t* __restrict__ count,
                                                            int cap, uint8_t* __restrict__ mode) {
  __shared__ int s_scan[kTierMaxHeads + 1];
  __shared__ int s_w[kSelWaves];
  const int tid = threadIdx.x;
  // device-resident sizes are clamped to the pool, so a state that was never
  // set up cannot send a store past it
  int top0 = tb.free_top[0];
  top0 = top0 < 0 ? 0 : (top0 > tb.nblocks ? tb.nblocks : top0);
  // 1. push the held blocks: head i's go to stack entries top0 + s[i] + j
  const int held_all = tier_scan(
      n_heads,
      [&](int i) -> int {
        const int h = tb.held[i];
        return h < 0 ? 0 : (h > tb.maxb ? tb.maxb : h);
      },
      s_scan, s_w);
  const int pushed = min(held_all, tb.nblocks - top0);
  for (int e = tid; e < pushed; e += kSelThreads) {
    const int i = tier_head_of(s_scan, n_heads, e);
    tb.free_ids[top0 + e] = tb.table[(int64_t)i * tb.maxb + (e - s_scan[i])];
  }
  __syncthreads();  // the pushes are done before any head's table changes
  const int top1 = top0 + pushed;
  // 2. pop the needs of the rewritten heads
  const int needed = tier_scan(
      n_heads,
      [&](int i) -> int {
        if (mode[i] != HARDKV_MODE_REWRITE) return 0;
        int k = count[i];
        k = k < 0 ? 0 : (k > cap ? cap : k);
        return (k + (1 << tb.lbs) - 1) >> tb.lbs;
      },
      s_scan, s_w);
  // heads whose range ends at or below top1 fit; they form a prefix
  for (int i = tid; i < n_heads; i += kSelThreads) {
    const int need = s_scan[i + 1] - s_scan[i];
    const bool fits = s_scan[i + 1] <= top1;
    tb.held[i] = fits ? need : 0;
    if (mode[i] == HARDKV_MODE_REWRITE && !fits) mode[i] = HARDKV_MODE_SPARSE;
  }
  // the fitting prefix's total: all of it, or the start of the last head
  // that starts at or below top1 (that head ends past it)
  const int fit_total = needed <= top1 ? needed : s_scan[tier_head_of(s_scan, n_heads, top1)];
  for (int e = tid; e < fit_total; e += kSelThreads) {
    const int i = tier_head_of(s_scan, n_heads, e);
    tb.table[(int64_t)i * tb.maxb + (e - s_scan[i])] = tb.free_ids[top1 - 1 - e];
  }
  if (tid == 0) tb.free_top[0] = top1 - fit_total;
}

void launch_tier_alloc(const TierBlocks& tb, int n_heads, const int32_t* count, int cap,
                       uint8_t* mode, hipStream_t st) {
  observe("k_tier_alloc", st);
  hipLaunchKernelGGL(k_tier_alloc, dim3(1), dim3(kSelThreads), 0, st, tb, n_heads, count, cap,
                     mode);
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
  const bool aux = a.metric != nullptr;
  const bool small = max_cand <= 4 * kSelThreads;
  auto kern = small ? (aux ? k_calsel<4, true> : k_calsel<4, false>)
                    : (aux ? k_calsel<16, true> : k_calsel<16, false>);
  hipLaunchKernelGGL(kern, grid, blk, 0, st, a.cand, a.metric, a.logit, a.l2, a.cap_stride,
                     a.stats, a.top_p, mass_scale(a.cand.cap), a.mask, count_out(a), a.calib,
                     a.kept_blk, a.kept_stride);
}

void launch_calibrate(const SelectArgs& a, hipStream_t st) {
  observe("k_calibrate", st);
  hipLaunchKernelGGL(k_calibrate, dim3(a.hkv, a.B), dim3(kCalThreads), 0, st, a.cand, a.metric,
                     a.logit, a.l2, a.cap_stride, a.stats, a.calib, !a.z_from_select);
}

void launch_select(const SelectArgs& a, hipStream_t st) {
  observe("k_select", st);
  hipLaunchKernelGGL(k_select, dim3(a.hkv, a.B), dim3(kSelThreads), 0, st, a.cand, a.metric,
                     a.logit, a.l2, a.cap_stride, a.stats, a.top_p, mass_scale(a.cand.cap),
                     a.mask, count_out(a), a.z_from_select, a.kept_blk, a.kept_stride);
}

}  // namespace hk
