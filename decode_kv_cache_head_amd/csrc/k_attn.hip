// Decode attention over the three tiers of the Cascade Cache (HARD-KV,
// arXiv abstract; gist.science technical summary, sections 2.A and 3).
//
// Split-K: the entries of one (b, h) -- dense rows, sparse (rewritten) rows
// and non-empty condensed chunks -- are cut into 256-entry tiles; one
// workgroup handles one tile for all G query heads of the KV head, so each
// K/V row is read from HBM once per step (GQA packing).  Every wave takes 64
// entries: a row is spread over LPR lanes that each load one 16-byte piece
// (coalesced), the G dot products are reduced across those lanes with DPP,
// scores go to LDS, then the V rows are streamed and accumulated with the
// wave's max subtracted.  The four waves combine in LDS and write one
// partial (max, sum, numerator) per query head; k_attn_merge joins the
// partials of every tile.
//
// Condensed entries hold float32 sums and a count n: their logit is
// q.(ksum / n) / sqrt(d) + ln n and their value vsum / n.
#include "internal.h"

namespace hk {

constexpr int kAttnTile = 256;

template <typename E, int D>
struct Lay {
  static constexpr int RB = D * (int)sizeof(E);
  static constexpr int LPR = RB / 16;          // lanes per row
  static constexpr int EPL = 16 / (int)sizeof(E);  // elements per lane
  static constexpr int RPI = 64 / LPR;          // rows per wave iteration
  static constexpr int IT = 64 / RPI;           // iterations per 64 rows
};

struct TileCounts {
  int nd, ns, nc, ntd, nts, ntc;
};

__device__ inline TileCounts tile_counts(const AttnArgs& a, int b, int h) {
  TileCounts t;
  int T = a.ctx_len ? a.ctx_len[b] : 0;
  T = T < 0 ? 0 : (T > a.ctx_cap ? a.ctx_cap : T);
  const int A = T > a.W ? T - a.W : 0;
  if (a.ring) {
    t.nd = a.W;
    t.nc = a.chunk_cap;
  } else {
    t.nd = T - A;
    t.nc = (A + a.C - 1) / a.C;
    if (t.nc > a.chunk_cap) t.nc = a.chunk_cap;
  }
  int ns = a.count[b * a.hkv + h];
  t.ns = ns < 0 ? 0 : (ns > a.sparse_cap ? a.sparse_cap : ns);
  t.ntd = (t.nd + kAttnTile - 1) / kAttnTile;
  t.nts = (t.ns + kAttnTile - 1) / kAttnTile;
  t.ntc = (t.nc + kAttnTile - 1) / kAttnTile;
  return t;
}

// One wave, up to 64 entries starting at row r0 of `kr`/`vr` (rows r0 + i
// map to row index r0 + i + roff of the source).  CHUNK: float32 sums with
// counts.  Writes the wave's max m, sum l and numerator o (lanes 0..LPR-1
// hold the full numerator, EPL elements each).
template <typename E, int D, int G, typename QT, bool CHUNK>
__device__ inline void wave_attn(const QT* __restrict__ qg, const Rows& kr, const Rows& vr, int b,
                                 int h, int r0, int wn, const int32_t* __restrict__ cc, float scale,
                                 float* s_sc, float (&m)[G], float (&l)[G],
                                 float (&o)[G][Lay<E, D>::EPL]) {
  using L = Lay<E, D>;
  constexpr int LPR = L::LPR, EPL = L::EPL, RPI = L::RPI, IT = L::IT;
  const int lane = threadIdx.x & 63;
  const int grp = lane / LPR, piece = lane % LPR;
  float qf[G][EPL];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[g][e] = Elt<QT>::load1(qg + g * D + piece * EPL + e);

  uint4 kb[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int r = it * RPI + grp;
    kb[it] = make_uint4(0, 0, 0, 0);
    if (r < wn) kb[it] = *(const uint4*)(kr.row(b, h, r0 + r) + piece * 16);
  }
#pragma unroll
  for (int g = 0; g < G; ++g) m[g] = -INFINITY;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int r = it * RPI + grp;
    float f[EPL];
    Elt<E>::unpack(kb[it], f);
    float dot[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) s = fmaf(qf[g][e], f[e], s);
      dot[g] = group_sum<LPR>(s);
    }
    bool valid = r < wn;
    float bias = 0.f, inv = 1.f;
    if (CHUNK) {
      const int cnt = valid ? cc[r0 + r] : 0;
      valid = valid && cnt > 0;
      inv = valid ? 1.f / (float)cnt : 0.f;
      bias = valid ? __logf((float)cnt) : 0.f;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float sc = valid ? dot[g] * inv * scale + bias : -INFINITY;
      m[g] = fmaxf(m[g], sc);
      if (piece == 0) s_sc[r * G + g] = sc;
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) m[g] = across_groups_max<LPR>(m[g]);

  uint4 vb[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int r = it * RPI + grp;
    vb[it] = make_uint4(0, 0, 0, 0);
    if (r < wn) vb[it] = *(const uint4*)(vr.row(b, h, r0 + r) + piece * 16);
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[g][e] = 0.f;
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int r = it * RPI + grp;
    float f[EPL];
    Elt<E>::unpack(vb[it], f);
    float inv = 1.f;
    if (CHUNK) {
      const int cnt = r < wn ? cc[r0 + r] : 0;
      inv = cnt > 0 ? 1.f / (float)cnt : 0.f;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float sc = s_sc[r * G + g];
      const float p = (r < wn && sc != -INFINITY) ? __expf(sc - m[g]) : 0.f;
      l[g] += p;
      const float pv = CHUNK ? p * inv : p;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[g][e] = fmaf(pv, f[e], o[g][e]);
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    l[g] = across_groups_sum<LPR>(l[g]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[g][e] = across_groups_sum<LPR>(o[g][e]);
  }
}

template <typename E, int D, int G, typename QT, bool CHUNK>
__device__ inline void tile_attn(const AttnArgs& a, const QT* qg, const Rows& kr, const Rows& vr,
                                 int b, int h, int r0, int nrows, const int32_t* cc, float* s_sc,
                                 float* s_m, float* s_l, float* s_o, float* part_out) {
  using L = Lay<E, D>;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int wn = nrows - w * 64;
  wn = wn < 0 ? 0 : (wn > 64 ? 64 : wn);
  float m[G], l[G], o[G][L::EPL];
  wave_attn<E, D, G, QT, CHUNK>(qg, kr, vr, b, h, r0 + w * 64, wn, cc, (float)a.scale,
                                s_sc + w * 64 * G, m, l, o);
  if (lane < L::LPR) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < L::EPL; ++e) s_o[(w * G + g) * D + lane * L::EPL + e] = o[g][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      s_m[w * G + g] = m[g];
      s_l[w * G + g] = l[g];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * D; i += 256) {
    const int g = i / D, e = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) M = fmaxf(M, s_m[v * G + g]);
    float O = 0.f, S = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float mv = s_m[v * G + g];
        if (mv != -INFINITY) {
          const float f = __expf(mv - M);
          O = fmaf(f, s_o[(v * G + g) * D + e], O);
          S = fmaf(f, s_l[v * G + g], S);
        }
      }
    }
    float* p = part_out + g * (D + 2);
    p[2 + e] = O;
    if (e == 0) {
      p[0] = M;
      p[1] = S;
    }
  }
}

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void k_attn(AttnArgs a) {
  __shared__ float s_sc[kAttnTile * G];
  __shared__ float s_m[4 * G], s_l[4 * G];
  __shared__ float s_o[4 * G * D];
  const int x = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const TileCounts tc = tile_counts(a, b, h);
  if (x >= tc.ntd + tc.nts + tc.ntc) return;
  const int64_t bh = (int64_t)b * a.hkv + h;
  const T* qg = (const T*)a.q + ((int64_t)b * a.hq + (int64_t)h * G) * D;
  float* part_out = a.part + (bh * a.max_tiles + x) * G * (D + 2);
  if (x < tc.ntd) {
    int T_ = a.ctx_len ? a.ctx_len[b] : 0;
    T_ = T_ < 0 ? 0 : (T_ > a.ctx_cap ? a.ctx_cap : T_);
    const int roff = a.ring ? 0 : (T_ > a.W ? T_ - a.W : 0);
    const int r0 = x * kAttnTile;
    tile_attn<T, D, G, T, false>(a, qg, a.dk, a.dv, b, h, roff + r0,
                                 min(kAttnTile, tc.nd - r0), nullptr, s_sc, s_m, s_l, s_o,
                                 part_out);
  } else if (x < tc.ntd + tc.nts) {
    const int r0 = (x - tc.ntd) * kAttnTile;
    tile_attn<T, D, G, T, false>(a, qg, a.sk, a.sv, b, h, r0, min(kAttnTile, tc.ns - r0),
                                 nullptr, s_sc, s_m, s_l, s_o, part_out);
  } else {
    const int r0 = (x - tc.ntd - tc.nts) * kAttnTile;
    Rows ck{(const char*)a.ksum, nullptr, a.chunk_cap, a.hkv, 0, 0, D * 4};
    Rows cv{(const char*)a.vsum, nullptr, a.chunk_cap, a.hkv, 0, 0, D * 4};
    tile_attn<float, D, G, T, true>(a, qg, ck, cv, b, h, r0, min(kAttnTile, tc.nc - r0),
                                    a.ccount + bh * a.chunk_cap, s_sc, s_m, s_l, s_o, part_out);
  }
}

// One wave per (b, query head): joins the partials of every tile.
template <typename T, int D, int G>
__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wid >= a.B * a.hq) return;
  const int b = wid / a.hq, qh = wid % a.hq, h = qh / G, g = qh % G;
  const TileCounts tc = tile_counts(a, b, h);
  const int nt = tc.ntd + tc.nts + tc.ntc;
  const int64_t bh = (int64_t)b * a.hkv + h;
  constexpr int PE = D / 64;  // elements per lane
  float M = -INFINITY, S = 0.f, O[PE];
#pragma unroll
  for (int e = 0; e < PE; ++e) O[e] = 0.f;
  for (int x = 0; x < nt; ++x) {
    const float* p = a.part + ((bh * a.max_tiles + x) * G + g) * (D + 2);
    const float mx = p[0];
    if (mx == -INFINITY) continue;
    const float nm = fmaxf(M, mx);
    const float fa = M == -INFINITY ? 0.f : __expf(M - nm);
    const float fb = __expf(mx - nm);
    S = S * fa + p[1] * fb;
#pragma unroll
    for (int e = 0; e < PE; ++e) O[e] = O[e] * fa + p[2 + lane * PE + e] * fb;
    M = nm;
  }
  float* out = a.out + ((int64_t)b * a.hq + qh) * D;
#pragma unroll
  for (int e = 0; e < PE; ++e) out[lane * PE + e] = S > 0.f ? O[e] / S : 0.f;
}

int attn_max_tiles(int W, int sparse_cap, int chunk_cap) {
  return ceil_div(W, kAttnTile) + ceil_div(sparse_cap, kAttnTile) + ceil_div(chunk_cap, kAttnTile);
}

template <typename T, int D, int G>
static void launch_attn_t(const AttnArgs& a, hipStream_t st) {
  if (a.max_tiles > 0)
    hipLaunchKernelGGL((k_attn<T, D, G>), dim3(a.max_tiles, a.hkv, a.B), dim3(256), 0, st, a);
  hipLaunchKernelGGL((k_attn_merge<T, D, G>), dim3(ceil_div((int64_t)a.B * a.hq, 4)), dim3(256),
                     0, st, a);
}

void launch_attn(const AttnArgs& a, hipStream_t st) {
  HK_DISPATCH(a.dtype, a.D, a.G, launch_attn_t, a, st);
}

}  // namespace hk
