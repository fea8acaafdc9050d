// Importance scores of aged tokens (HARD-KV, gist.science technical summary,
// section 2.B "Goal": max-pooled logits; key-norm metric alongside).
//
// HBM-bound stream over the aged keys.  Each workgroup stages a 256-token
// tile of one (b, h) into LDS with coalesced 16-byte loads, then every lane
// scores one token: the G query rows of the head's GQA group are read as
// float64 from wave-uniform addresses (scalar loads, SGPR operands), the
// token's key is widened exactly to float64 and the G dot products are
// accumulated in float64, so the only rounding the ranking key sees is the
// final fl32().
#include "internal.h"

namespace hk {

template <typename T>
__global__ __launch_bounds__(256) void k_q_to_f64(const T* __restrict__ q, double* __restrict__ q64,
                                                   int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) q64[i] = (double)Elt<T>::load1(q + i);
}

constexpr int kScoreTile = 256;

template <typename T, int D, int G, bool L2>
__device__ inline void score_row(const unsigned char* row, const double* __restrict__ qg,
                                 double (&acc)[G], double& ss) {
  constexpr int RB = D * (int)sizeof(T);
  constexpr int CPR = RB / 16;
  constexpr int EPC = Elt<T>::kPer16;
#pragma unroll
  for (int c = 0; c < CPR; ++c) {
    const uint4 raw = *(const uint4*)(row + c * 16);
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

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void k_score(const double* __restrict__ q64, int hq, Rows rows,
                                               Cand cand, const int8_t* __restrict__ metric,
                                               float* __restrict__ logit, float* __restrict__ l2,
                                               int64_t cap_stride, double scale) {
  constexpr int RB = D * (int)sizeof(T);
  constexpr int CPR = RB / 16;
  constexpr int PAD = RB + 16;  // keeps per-lane row reads conflict free
  __shared__ __attribute__((aligned(16))) unsigned char lds[kScoreTile * PAD];
  const int b = blockIdx.z, h = blockIdx.y, hkv = gridDim.y;
  const int n = cand.n(b, h);
  const int t0 = blockIdx.x * kScoreTile;
  if (t0 >= n) return;
  const int tid = threadIdx.x;

  // Rows past the end re-read the last valid row (always in bounds); their
  // scores are never written.
  uint4 buf[CPR];
#pragma unroll
  for (int j = 0; j < CPR; ++j) {
    const int idx = j * kScoreTile + tid;
    const int r = idx / CPR, c = idx % CPR;
    const int t = min(t0 + r, n - 1);
    buf[j] = *(const uint4*)(rows.row(b, h, t) + c * 16);
  }
#pragma unroll
  for (int j = 0; j < CPR; ++j) {
    const int idx = j * kScoreTile + tid;
    const int r = idx / CPR, c = idx % CPR;
    *(uint4*)(lds + r * PAD + c * 16) = buf[j];
  }
  __syncthreads();

  const int t = t0 + tid;
  if (t >= n) return;
  const double* __restrict__ qg = q64 + ((int64_t)b * hq + (int64_t)h * G) * D;
  const bool is_l2 = metric != nullptr && metric[h] == HARDKV_METRIC_L2;
  double acc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = 0.0;
  double ss = 0.0;
  const unsigned char* row = lds + tid * PAD;
  if (is_l2)
    score_row<T, D, G, true>(row, qg, acc, ss);
  else
    score_row<T, D, G, false>(row, qg, acc, ss);
  double mx = acc[0];
#pragma unroll
  for (int g = 1; g < G; ++g) mx = fmax(mx, acc[g]);
  const int64_t o = ((int64_t)b * hkv + h) * cap_stride + t;
  logit[o] = (float)(mx * scale);
  if (is_l2) l2[o] = (float)sqrt(ss);
}

template <typename T, int D, int G>
static void launch_score_t(const ScoreArgs& a, hipStream_t st) {
  const int64_t nq = (int64_t)a.B * a.hq * D;
  hipLaunchKernelGGL(k_q_to_f64<T>, dim3(ceil_div(nq, 256)), dim3(256), 0, st, (const T*)a.q,
                     a.q64, nq);
  dim3 grid(ceil_div(a.max_cand, kScoreTile), a.rows.hkv, a.B);
  if (grid.x == 0) return;
  hipLaunchKernelGGL((k_score<T, D, G>), grid, dim3(256), 0, st, a.q64, a.hq, a.rows, a.cand,
                     a.metric, a.logit, a.l2, a.cap_stride, a.scale);
}

void launch_score(const ScoreArgs& a, hipStream_t st) {
  HK_DISPATCH(a.dtype, a.D, a.G, launch_score_t, a, st);
}

}  // namespace hk
