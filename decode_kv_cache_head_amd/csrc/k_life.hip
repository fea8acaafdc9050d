// One decode step of the token lifecycle for one (b, h) in one workgroup
// (HARD-KV, gist.science technical summary, section 2.A: the four-step
// pipeline; dense -> sparse -> condensed as tokens age), for launches whose
// heads all rank by the raw logit and whose pools are per-head regions:
//
//   1. append: the token in ring slot P % W (position P - W) moves to the end
//      of the pool, the new key / value take its slot (as k_append);
//   2. score: fl32(max_g q_g . k_t / sqrt(d)) for every pool row, float64
//      dots of the exact inputs in k_score's order (each dot is the sum of
//      its two half-row partial sums), written to the logit workspace;
//   3. calibrate + select: m = max logit, the radix select by mass of
//      select_core.h (temperature 1: c = logit), mask to the workspace;
//   4. compaction in place with the evicted rows merged into the running
//      chunk sums (inplace_core.h), which also writes the new count.
//
// The separate kernels run the same arithmetic with a launch per stage;
// here the four stages follow each other inside the workgroup, so a step
// over small pools pays one launch instead of five.  The attention launches
// follow as usual.
#include "inplace_core.h"
#include "select_core.h"

namespace hk {

constexpr int kLifeThreads = 512;
constexpr int kLifeTile = 128;  // pool rows scored per round

template <typename T, int D, int G>
struct LifeScoreLds {
  static constexpr int RB = D * (int)sizeof(T);
  static constexpr int PAD = RB + 16;  // conflict-free per-lane row reads
  __attribute__((aligned(16))) unsigned char rows[kLifeTile * PAD];
  double part[G][kLifeTile];  // second half-row partial dots
  double gmax[kLifeTile];     // head group 1's maximum
  float fmx[kLifeThreads / 64];
};

template <typename T, int D, int G>
union LifeLds {
  LifeScoreLds<T, D, G> sc;
  SelShared sel;
  SelSmall small;
  InplaceLds<T, D, false> cp;
};

template <typename T, int D, int G>
__global__ __launch_bounds__(kLifeThreads) void k_life(LifeArgs A) {
  constexpr int NT = kLifeThreads;
  constexpr int RB = D * (int)sizeof(T);
  constexpr int CPR = RB / 16;           // 16-byte pieces per row
  constexpr int PCS = CPR / 2;           // pieces per half row
  constexpr int EPC = Elt<T>::kPer16;    // elements per piece
  constexpr int PAD = LifeScoreLds<T, D, G>::PAD;
  constexpr int HG = G >= 2 ? 2 : 1;     // query-head groups scoring a token
  constexpr int GH = G / HG;             // heads per group
  constexpr int LOADS = kLifeTile * CPR / NT;
  static_assert(LOADS >= 1 && kLifeTile * CPR % NT == 0, "tile shape");
  __shared__ __attribute__((aligned(16))) double s_q[G * D];
  __shared__ double s_et[64];
  __shared__ LifeLds<T, D, G> U;
  const AppendArgs& ap = A.ap;
  const CompactArgs& ca = A.ca;
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int64_t bh = (int64_t)b * ap.hkv + h;

  // ---- 1. append, and this head's queries widened to float64
  {
    const T* qg = (const T*)A.q + ((int64_t)b * ap.hq + (int64_t)h * G) * D;
    for (int i = tid; i < G * D; i += NT) s_q[i] = (double)Elt<T>::load1(qg + i);
  }
  exp_table_init(s_et);
  const int P = ap.seq_len[b];
  const int cnt0 = ap.pool_count[bh];
  const bool append = P >= ap.W && ap.W > 0;
  const bool room = append && cnt0 >= 0 && cnt0 < ap.sparse_cap && P < ap.ctx_cap;
  int n = cnt0 + (room ? 1 : 0);
  n = n < 0 ? 0 : (n > ap.sparse_cap ? ap.sparse_cap : n);
  const char* pool_k = (const char*)ap.pool_k + bh * ap.sparse_cap * RB;
  v4u buf[LOADS];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int idx = j * NT + tid, r = idx / CPR, c = idx % CPR;
      buf[j] = __builtin_nontemporal_load((const v4u*)(pool_k + (int64_t)min(t0 + r, n - 1) * RB + c * 16));
    }
  };
  // the first tile's rows are read while the append is under way: rows below
  // cnt0 are not written by it, and the appended row (pool row cnt0, whose
  // load here returns an unused value) enters the tile from the registers
  // that carry it from the ring
  if (n > 0) fetch(0);
  const int tsr = tid / CPR, cpc = tid % CPR;
  const bool mine = append && tid < 2 * CPR;
  v4u old{};
  {
    const int slot = append ? P % ap.W : 0;
    char* rk = ap.ring_k + (bh * ap.W + slot) * RB;
    char* rv = ap.ring_v + (bh * ap.W + slot) * RB;
    if (mine) old = *(const v4u*)((tsr ? rv : rk) + cpc * 16);
    __syncthreads();  // every read of the old ring row is done
    if (mine) {
      if (room) *(v4u*)((tsr ? ap.pool_v : ap.pool_k) + ((bh * ap.sparse_cap + cnt0) * RB) + cpc * 16) = old;
      *(v4u*)((tsr ? rv : rk) + cpc * 16) =
          *(const v4u*)((const char*)(tsr ? ap.v_new : ap.k_new) + bh * RB + cpc * 16);
    }
    if (tid == 0 && room) ap.pool_pos[bh * ap.sparse_cap + cnt0] = P - ap.W;
  }
  __syncthreads();  // the appended row is visible to the whole workgroup

  // ---- 2. score: thread (token, half, head group)
  const int tok = tid % kLifeTile;
  const int half = __builtin_amdgcn_readfirstlane((tid / kLifeTile) & 1);
  const int hg = __builtin_amdgcn_readfirstlane(tid / (2 * kLifeTile));
  const bool scorer = hg < HG;
  float* logit = A.logit + bh * A.cap_stride;
  float lmax = -INFINITY;
  float my_lg = 0.f;  // this thread's logit of the last tile (token tid when n <= one tile)
  const bool app_in_tile0 = room && cnt0 < kLifeTile;
  for (int t0 = 0; t0 < n; t0 += kLifeTile) {
    if (t0) __syncthreads();  // the previous round's LDS reads are done
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int idx = j * NT + tid, r = idx / CPR, c = idx % CPR;
      if (!(t0 == 0 && app_in_tile0 && r == cnt0)) *(v4u*)(U.sc.rows + r * PAD + c * 16) = buf[j];
    }
    if (t0 == 0 && app_in_tile0 && mine && tsr == 0)
      *(v4u*)(U.sc.rows + cnt0 * PAD + cpc * 16) = old;
    __syncthreads();
    if (t0 + kLifeTile < n) fetch(t0 + kLifeTile);  // in flight while this tile is scored
    double acc[GH];
#pragma unroll
    for (int g = 0; g < GH; ++g) acc[g] = 0.0;
    // waves whose 64 tokens all lie past the pool skip the dot products
    if (scorer && t0 + (tok & ~63) < n) {
      const unsigned char* row = U.sc.rows + tok * PAD + half * (RB / 2);
      const double* qh = s_q + (hg * GH) * D + half * (D / 2);
#pragma unroll
      for (int c = 0; c < PCS; ++c) {
        float f[EPC];
        Elt<T>::unpack(*(const v4u*)(row + c * 16), f);
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          const double kd = (double)f[e];
#pragma unroll
          for (int g = 0; g < GH; ++g) acc[g] = fma(qh[g * D + c * EPC + e], kd, acc[g]);
        }
      }
      if (half) {
#pragma unroll
        for (int g = 0; g < GH; ++g) U.sc.part[hg * GH + g][tok] = acc[g];
      }
    }
    __syncthreads();
    double mx = -INFINITY;
    if (scorer && !half) {
#pragma unroll
      for (int g = 0; g < GH; ++g) mx = fmax(mx, acc[g] + U.sc.part[hg * GH + g][tok]);
      if (hg == 1) U.sc.gmax[tok] = mx;
    }
    __syncthreads();
    if (hg == 0 && !half && t0 + tok < n) {
      if (HG == 2) mx = fmax(mx, U.sc.gmax[tok]);
      const float lg = (float)(mx * A.scale);
      logit[t0 + tok] = lg;
      lmax = fmaxf(lmax, lg);
      my_lg = lg;
    }
  }
  // head maximum m (the calibrated values are the logits)
  lmax = wave_max_f32(lmax);
  __syncthreads();
  if ((tid & 63) == 0) U.sc.fmx[tid >> 6] = lmax;
  __syncthreads();
  float m = U.sc.fmx[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) m = fmaxf(m, U.sc.fmx[i]);
  __syncthreads();  // the score's LDS is free for the selection

  // ---- 3. select (the logit writes above are visible after the barrier)
  uint8_t* mk = A.mask + bh * A.cap_stride;
  if (n > 0) {
    if (!(A.top_p < 1.0f)) {
      for (int t = tid; t < n; t += NT) mk[t] = 1;
    } else if (n <= 64) {
      // one wave: lane t holds token t's logit
      if (tid < 64) select_wave(n, my_lg, (double)m, A.top_p, A.wscale, s_et, mk);
    } else if (n <= kSmallSel) {
      // one tile: thread t < n holds token t's logit
      static_assert(kSmallSel <= kLifeTile, "small pools fit one score tile");
      select_small(U.small, n, my_lg, (double)m, A.top_p, A.wscale, s_et, mk);
    } else {
      select_head<NT>(U.sel, n, logit, [](float raw) -> float { return raw; }, (double)m,
                      A.top_p, A.wscale, s_et, mk);
    }
  }
  if (tid == 0) {
    double* o = A.stats + bh * 4;
    o[0] = 0.0;
    o[1] = 1.0;
    o[2] = n ? (double)m : 0.0;
    o[3] = 0.0;  // Z is not formed here (nothing downstream reads it)
  }
  __syncthreads();  // the mask is written; the selection's LDS is free

  // ---- 4. compaction in place, chunk sums, count
  compact_inplace_head<T, D, false>(ca, b, h, n, U.cp);
}

template <typename T, int D, int G>
static void launch_life_t(const LifeArgs& a, hipStream_t st) {
  observe("k_life", st);
  hipLaunchKernelGGL((k_life<T, D, G>), dim3(a.ap.hkv, a.ap.B), dim3(kLifeThreads), 0, st, a);
}

void launch_life(const LifeArgs& a, hipStream_t st) {
  HK_DISPATCH(a.ap.dtype, a.ap.D, a.ap.hq / a.ap.hkv, launch_life_t, a, st);
}

}  // namespace hk
