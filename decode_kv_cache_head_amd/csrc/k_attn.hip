// Decode attention over the three tiers of the Cascade Cache (HARD-KV,
// arXiv abstract; gist.science technical summary, sections 2.A and 3).
//
// Split-K: the entries of one (b, h) -- dense rows, sparse (rewritten) rows
// and non-empty condensed chunks -- are cut into 512-entry tiles; one
// workgroup handles one tile for all G query heads of the KV head, so each
// K/V row is read from HBM once per step (GQA packing).  The four waves
// share a tile evenly (up to 128 entries each).  On the vector path a row
// is spread over LPR lanes that each load one 16-byte piece
// (coalesced), the G dot products are reduced across those lanes with DPP,
// scores go to LDS, then the V rows are streamed and accumulated with the
// wave's max subtracted.  The four waves combine in LDS and write one
// partial (max, sum, numerator) per query head; k_attn_merge joins the
// partials of every tile.
//
// Heads served by sparse loading (mode byte HARDKV_MODE_SPARSE) read their
// sparse entries from the cache rows at the tier's positions instead of the
// rewritten slots (section 2.C, "Techniques").
//
// Condensed entries hold float32 sums and a count n: their logit is
// q.(ksum / n) / sqrt(d) + ln n and their value vsum / n.
//
// bf16 rows with d = 128 and G >= 4 take the matrix-core path (wave_attn_mx):
// scores and the weighted value sum are 16x16x32 bf16 MFMA products with
// float32 accumulation; the weights enter the second product as a bf16
// high part plus a bf16 remainder, so each weight carries 16 significant bits.
// With bf16 queries the condensed tiles do the same with their float32 sums
// split into two bf16 terms (wave_attn_mx_chunk).  At G >= 8 the condensed
// tiles run as a second launch so they do not set the row tiles' register
// budget.
#include "internal.h"

namespace hk {

// Entries per workgroup tile of any tier.  The four waves split a tile
// evenly, so on a long tier each wave runs four 32-entry steps per
// workgroup start-up.
constexpr int kAttnTile = 512;

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
  int first;     // partial slots taken by the fused compaction's tiles
  int gap_at;    // dense entry r is position r, or r + gap_len from gap_at on
  int gap_len;
};

__device__ inline TileCounts tile_counts(const AttnArgs& a, int b, int h) {
  TileCounts t;
  int T = a.ctx_len ? a.ctx_len[b] : 0;
  T = T < 0 ? 0 : (T > a.ctx_cap ? a.ctx_cap : T);
  const int A = T > a.W + a.sinks ? T - a.W - a.sinks : 0;  // candidates [S, S + A)
  t.gap_at = a.sinks;
  t.gap_len = a.ring ? 0 : A;
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
  t.first = 0;
  if (a.fused_tt > 0) {
    // the compaction's tiles attended the sparse and condensed tiers
    int n = A > a.sparse_cap ? a.sparse_cap : A;
    t.first = (n + a.fused_tt - 1) / a.fused_tt;
    t.nts = 0;
    t.ntc = 0;
  }
  return t;
}

// One wave, wn entries starting at row r0 of `kr`/`vr`, in rounds of
// 8 iterations x RPI rows.  Each round issues the K and the V loads of all
// its rows first, then scores, then rescales the running (m, l, o) to the
// new maximum and accumulates p * v.  CHUNK: float32 sums with counts.
// Lanes 0..LPR-1 end with the full numerator (EPL elements each).
// IDX: entry r is row idx[r0 + r] of kr / vr (clamped to [0, idx_max]) --
// sparse loading of kept rows from the cache.  Otherwise entry r is row
// r0 + r, moved up by gap_len from row gap_at on (the dense tier skips the
// candidate range).
template <typename E, int D, int G, typename QT, bool CHUNK, bool P, bool IDX>
__device__ inline void wave_attn(const QT* __restrict__ qg, const Rows& kr, const Rows& vr, int b,
                                 int h, int r0, int wn, const int32_t* __restrict__ cc,
                                 const int32_t* __restrict__ idx, int idx_max, int gap_at,
                                 int gap_len, float scale, float (&m)[G], float (&l)[G],
                                 float (&o)[G][Lay<E, D>::EPL]) {
  using L = Lay<E, D>;
  constexpr int LPR = L::LPR, EPL = L::EPL, RPI = L::RPI;
  constexpr int IT = G >= 8 ? 4 : 8;  // G = 8: smaller rounds keep two waves per SIMD
  constexpr int RR = IT * RPI;  // rows per round
  const int lane = threadIdx.x & 63;
  const int grp = lane / LPR, piece = lane % LPR;
  QPiece<E, QT, EPL> qp[G];
#pragma unroll
  for (int g = 0; g < G; ++g) qp[g].load(qg + g * D + piece * EPL);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[g][e] = 0.f;
  }
  for (int base = 0; base < wn; base += RR) {
    v4u kb[IT], vb[IT];
    int cnt[IT], row[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int r = min(base + it * RPI + grp, wn - 1);  // in bounds; masked below
      if (IDX) {
        const int t = idx[r0 + r];
        row[it] = t < 0 ? 0 : (t > idx_max ? idx_max : t);
      } else {
        row[it] = r0 + r;
        if (row[it] >= gap_at) row[it] += gap_len;
      }
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      kb[it] = *(const v4u*)(kr.template row<P>(b, h, row[it]) + piece * 16);
      vb[it] = *(const v4u*)(vr.template row<P>(b, h, row[it]) + piece * 16);
      if (CHUNK) cnt[it] = cc[row[it]];
    }
    float s[IT][G];
    float mr[G];
#pragma unroll
    for (int g = 0; g < G; ++g) mr[g] = -INFINITY;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const bool valid = base + it * RPI + grp < wn && (!CHUNK || cnt[it] > 0);
      float inv = 1.f, bias = 0.f;
      if (CHUNK) {
        inv = valid ? 1.f / (float)cnt[it] : 0.f;
        bias = valid ? __logf((float)cnt[it]) : 0.f;
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float dot = group_sum<LPR>(qp[g].dot(kb[it]));
        s[it][g] = valid ? dot * inv * scale + bias : -INFINITY;
        mr[g] = fmaxf(mr[g], s[it][g]);
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      mr[g] = across_groups_max<LPR>(mr[g]);
      const float mn = fmaxf(m[g], mr[g]);
      const float alpha = (m[g] == -INFINITY) ? 0.f : __expf(m[g] - mn);
      l[g] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[g][e] *= alpha;
      m[g] = mn;
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      float f[EPL];
      Elt<E>::unpack(vb[it], f);
      float inv = 1.f;
      if (CHUNK) inv = cnt[it] > 0 ? 1.f / (float)cnt[it] : 0.f;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p = s[it][g] == -INFINITY ? 0.f : __expf(s[it][g] - m[g]);
        l[g] += p;
        const float pv = CHUNK ? p * inv : p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[g][e] = fmaf(pv, f[e], o[g][e]);
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    l[g] = across_groups_sum<LPR>(l[g]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[g][e] = across_groups_sum<LPR>(o[g][e]);
  }
}

// ------------------------------------------------ matrix-core row tiles --
// Word j of the bf16 pairs (x.half, y.half): the same element of two rows.
template <int HI>
__device__ __forceinline__ uint32_t pair_of(uint32_t x, uint32_t y) {
  return HI ? __builtin_amdgcn_perm(y, x, 0x07060302u) : __builtin_amdgcn_perm(y, x, 0x05040100u);
}

template <int B>
__device__ __forceinline__ uint32_t word_of(const v4u& v) {
  return B == 0 ? v.x : (B == 1 ? v.y : (B == 2 ? v.z : v.w));
}

// Column blk of the 8x8 bf16 block held as 8 rows of 8: 8 values (rows 0..7)
// packed in pairs, the A operand of the value product.
template <int BLK>
__device__ __forceinline__ v4u column_of(const v4u (&r)[8]) {
  v4u c;
  c.x = pair_of<BLK & 1>(word_of<BLK / 2>(r[0]), word_of<BLK / 2>(r[1]));
  c.y = pair_of<BLK & 1>(word_of<BLK / 2>(r[2]), word_of<BLK / 2>(r[3]));
  c.z = pair_of<BLK & 1>(word_of<BLK / 2>(r[4]), word_of<BLK / 2>(r[5]));
  c.w = pair_of<BLK & 1>(word_of<BLK / 2>(r[6]), word_of<BLK / 2>(r[7]));
  return c;
}

template <int BLK>
__device__ __forceinline__ void pv_block(const v4u (&vb)[8], const v4u& ph, const v4u& pl,
                                         f32x4_t (&acc)[8]) {
  const v4u va = column_of<BLK>(vb);
  acc[BLK] = mfma16(va, ph, acc[BLK]);
  acc[BLK] = mfma16(va, pl, acc[BLK]);
}

// One wave, up to 64 bf16 rows (d = 128) starting at entry r0, G <= 16 query
// heads, in steps of 32 entries.  Lane l = 16 g + i (i = l % 16, g = l / 16).
//   scores  S^T = K Q^T: two 16-row products whose row r is entry
//           8 (r / 4) + r % 4 (+4 for the second), so lane l receives the
//           scores of entries 8 g .. 8 g + 7 for query head i; the d order of
//           the contraction is d = 32 s + 8 g + j in both operands;
//   values  O^T = V^T P^T with d permuted as d = 8 r + blk for row r of
//           product blk: lane l loads 16 bytes (d = 8 i .. 8 i + 7) of each
//           of its 8 entries and transposes them in registers.
// On return lane l holds, for query head i, the running max m (common to the
// 4 lanes of i), its own part of the sum l, and acc[blk][c] = the numerator
// at d = 8 (4 g + c) + blk.  Rows are addressed as in wave_attn.
template <int G, bool P, bool IDX>
__device__ inline void wave_attn_mx(const bf16_t* __restrict__ qg, const Rows& kr,
                                    const Rows& vr, int b, int h, int r0, int wn,
                                    const int32_t* __restrict__ idx, int idx_max, int gap_at,
                                    int gap_len, float scale, float& m_run, float& l_run,
                                    f32x4_t (&acc)[8]) {
  constexpr int D = 128;
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, g = lane >> 4;
  v4u qb[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    qb[s] = i < G ? *(const v4u*)(qg + i * D + 32 * s + 8 * g) : v4u{0u, 0u, 0u, 0u};
  m_run = -INFINITY;
  l_run = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto row_of = [&](int r) -> int {
    r = r < wn ? r : wn - 1;  // in bounds; weight 0 below
    if (IDX) {
      const int t = idx[r0 + r];
      return t < 0 ? 0 : (t > idx_max ? idx_max : t);
    }
    const int t = r0 + r;
    return t >= gap_at ? t + gap_len : t;
  };
  for (int base = 0; base < wn; base += 32) {
    const int ek = base + 8 * (i >> 2) + (i & 3);
    const char* k0 = kr.template row<P>(b, h, row_of(ek)) + 16 * g;
    const char* k1 = kr.template row<P>(b, h, row_of(ek + 4)) + 16 * g;
    v4u kb0[4], kb1[4], vb[8];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      kb0[s] = *(const v4u*)(k0 + 64 * s);
      kb1[s] = *(const v4u*)(k1 + 64 * s);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      vb[j] = *(const v4u*)(vr.template row<P>(b, h, row_of(base + 8 * g + j)) + 16 * i);
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      s0 = mfma16(kb0[s], qb[s], s0);
      s1 = mfma16(kb1[s], qb[s], s1);
    }
    float sc[8];
    float mx = -INFINITY;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      sc[c] = base + 8 * g + c < wn ? s0[c] * scale : -INFINITY;
      sc[4 + c] = base + 8 * g + 4 + c < wn ? s1[c] * scale : -INFINITY;
      mx = fmaxf(mx, fmaxf(sc[c], sc[4 + c]));
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m_run, mx);
    const float alpha = m_run == -INFINITY ? 0.f : __expf(m_run - mn);
    l_run *= alpha;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] *= alpha;
    m_run = mn;
    bf16x8_t hi, lo;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = sc[j] == -INFINITY ? 0.f : __expf(sc[j] - mn);
      l_run += p;
      hi[j] = (__bf16)p;
      lo[j] = (__bf16)(p - (float)hi[j]);
    }
    const v4u ph = __builtin_bit_cast(v4u, hi), pl = __builtin_bit_cast(v4u, lo);
    pv_block<0>(vb, ph, pl, acc);
    pv_block<1>(vb, ph, pl, acc);
    pv_block<2>(vb, ph, pl, acc);
    pv_block<3>(vb, ph, pl, acc);
    pv_block<4>(vb, ph, pl, acc);
    pv_block<5>(vb, ph, pl, acc);
    pv_block<6>(vb, ph, pl, acc);
    pv_block<7>(vb, ph, pl, acc);
  }
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
}

// x ~= hi + lo with hi = bf16(x) and lo = bf16(x - hi): 16 significant bits
// of each float32, packed as the pairs (x0, x1) an MFMA operand word holds.
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const __bf16 h0 = (__bf16)x0, h1 = (__bf16)x1;
  hi = __builtin_bit_cast(uint32_t, bf16x2_t{h0, h1});
  lo = __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)(x0 - (float)h0), (__bf16)(x1 - (float)h1)});
}

__device__ __forceinline__ float comp(const v4u& v, int c) {
  return __uint_as_float(c == 0 ? v.x : (c == 1 ? v.y : (c == 2 ? v.z : v.w)));
}

// Value product of one block for float32 rows held as vf[j][0..1] (8 floats
// of d = 8 i .. 8 i + 7 of entry j): A = V^T split into two bf16 terms,
// B = the weights' two terms; the lo x lo product (below 2^-18) is dropped.
template <int BLK>
__device__ __forceinline__ void pv_block_f32(const v4u (&vf)[8][2], const v4u& ph, const v4u& pl,
                                             f32x4_t (&acc)[8]) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj)
    split2(comp(vf[2 * jj][BLK / 4], BLK % 4), comp(vf[2 * jj + 1][BLK / 4], BLK % 4), h[jj],
           l[jj]);
  const v4u vh = {h[0], h[1], h[2], h[3]}, vl = {l[0], l[1], l[2], l[3]};
  acc[BLK] = mfma16(vh, ph, acc[BLK]);
  acc[BLK] = mfma16(vh, pl, acc[BLK]);
  acc[BLK] = mfma16(vl, ph, acc[BLK]);
}

// The condensed tier on the matrix cores: like wave_attn_mx, with float32
// sums (ksum, vsum) and counts n.  Entry e's logit is q.ksum_e / n_e *
// scale + ln n_e and its value vsum_e / n_e (the weight enters divided by
// n_e).  Key and value sums enter as two bf16 terms each (relative error
// below 2^-17 per element), the weights as two terms as well.
template <int G>
__device__ inline void wave_attn_mx_chunk(const bf16_t* __restrict__ qg, const Rows& kr,
                                          const Rows& vr, int b, int h, int r0, int wn,
                                          const int32_t* __restrict__ cc, float scale,
                                          float& m_run, float& l_run, f32x4_t (&acc)[8]) {
  constexpr int D = 128;
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, g = lane >> 4;
  v4u qb[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    qb[s] = i < G ? *(const v4u*)(qg + i * D + 32 * s + 8 * g) : v4u{0u, 0u, 0u, 0u};
  m_run = -INFINITY;
  l_run = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int base = 0; base < wn; base += 32) {
    const int ek = base + 8 * (i >> 2) + (i & 3);
    const char* k0 = kr.template row<false>(b, h, r0 + min(ek, wn - 1)) + 32 * g;
    const char* k1 = kr.template row<false>(b, h, r0 + min(ek + 4, wn - 1)) + 32 * g;
    v4u kf[2][4][2], vf[8][2];
    int cn[8];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      kf[0][s][0] = *(const v4u*)(k0 + 128 * s);
      kf[0][s][1] = *(const v4u*)(k0 + 128 * s + 16);
      kf[1][s][0] = *(const v4u*)(k1 + 128 * s);
      kf[1][s][1] = *(const v4u*)(k1 + 128 * s + 16);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = base + 8 * g + j;
      cn[j] = e < wn ? cc[r0 + e] : 0;
    }
    // scores: each k-step's 8 floats as two bf16 terms against the bf16 query
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const v4u& a0 = kf[c][s][0];
        const v4u& a1 = kf[c][s][1];
        uint32_t hh[4], ll[4];
        split2(__uint_as_float(a0.x), __uint_as_float(a0.y), hh[0], ll[0]);
        split2(__uint_as_float(a0.z), __uint_as_float(a0.w), hh[1], ll[1]);
        split2(__uint_as_float(a1.x), __uint_as_float(a1.y), hh[2], ll[2]);
        split2(__uint_as_float(a1.z), __uint_as_float(a1.w), hh[3], ll[3]);
        const v4u kh = {hh[0], hh[1], hh[2], hh[3]}, kl = {ll[0], ll[1], ll[2], ll[3]};
        f32x4_t& sc = c ? s1 : s0;
        sc = mfma16(kh, qb[s], sc);
        sc = mfma16(kl, qb[s], sc);
      }
    }
    // the value rows, loaded once the key sums have been consumed
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const char* vrow = vr.template row<false>(b, h, r0 + min(base + 8 * g + j, wn - 1)) + 32 * i;
      vf[j][0] = *(const v4u*)vrow;
      vf[j][1] = *(const v4u*)(vrow + 16);
    }
    float lg[8], inv[8];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float dot = j < 4 ? s0[j] : s1[j - 4];
      const bool valid = cn[j] > 0;
      inv[j] = valid ? 1.f / (float)cn[j] : 0.f;
      lg[j] = valid ? dot * inv[j] * scale + __logf((float)cn[j]) : -INFINITY;
      mx = fmaxf(mx, lg[j]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m_run, mx);
    const float alpha = m_run == -INFINITY ? 0.f : __expf(m_run - mn);
    l_run *= alpha;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] *= alpha;
    m_run = mn;
    float pw[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = lg[j] == -INFINITY ? 0.f : __expf(lg[j] - mn);
      l_run += p;
      pw[j] = p * inv[j];
    }
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) split2(pw[2 * jj], pw[2 * jj + 1], ph[jj], pl[jj]);
    const v4u phv = {ph[0], ph[1], ph[2], ph[3]}, plv = {pl[0], pl[1], pl[2], pl[3]};
    pv_block_f32<0>(vf, phv, plv, acc);
    pv_block_f32<1>(vf, phv, plv, acc);
    pv_block_f32<2>(vf, phv, plv, acc);
    pv_block_f32<3>(vf, phv, plv, acc);
    pv_block_f32<4>(vf, phv, plv, acc);
    pv_block_f32<5>(vf, phv, plv, acc);
    pv_block_f32<6>(vf, phv, plv, acc);
    pv_block_f32<7>(vf, phv, plv, acc);
  }
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
}

// LDS row stride of the per-wave numerators (padded against bank conflicts
// of the matrix-core path's stores, where lanes of one store hold different
// query heads).
template <int D>
constexpr int kSO = D + 4;

// The four waves' (m, l, o) in LDS -> one partial (max, sum, numerator) per
// query head of the tile.
template <int G, int D>
__device__ inline void combine_waves(const float* s_m, const float* s_l, const float* s_o,
                                     float* part_out) {
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
          O = fmaf(f, s_o[(v * G + g) * kSO<D> + e], O);
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

// bf16 rows, d = 128, G >= 4: the matrix-core path.
template <typename E, int D, int G, bool CHUNK>
constexpr bool kUseMx = !CHUNK && D == 128 && G >= 4 && sizeof(E) == 2;
// float32 chunk sums with bf16 queries, d = 128, G >= 4: the matrix-core
// condensed path.
template <int D, int G, bool CHUNK, typename QT>
constexpr bool kUseMxChunk = CHUNK && D == 128 && G >= 4 && sizeof(QT) == 2;

// One tile of up to kAttnTile entries: wave w takes entries [w RW, (w + 1) RW).
template <typename E, int D, int G, typename QT, bool CHUNK, bool P, bool IDX = false>
__device__ inline void tile_attn(const AttnArgs& a, const QT* qg, const Rows& kr, const Rows& vr,
                                 int b, int h, int r0, int nrows, const int32_t* cc, float* s_m,
                                 float* s_l, float* s_o, float* part_out,
                                 const int32_t* idx = nullptr, int idx_max = 0,
                                 int gap_at = 0, int gap_len = 0) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // entries per wave: the tile's rows spread evenly over the four waves in
  // whole 32-entry steps, so a short tier does not fall on one wave
  const int RW = min(kAttnTile / 4, ((nrows + 127) >> 7) << 5);
  int wn = nrows - w * RW;
  wn = wn < 0 ? 0 : (wn > RW ? RW : wn);
  if constexpr (kUseMx<E, D, G, CHUNK> || kUseMxChunk<D, G, CHUNK, QT>) {
    float m, l;
    f32x4_t acc[8];
    if constexpr (CHUNK)
      wave_attn_mx_chunk<G>((const bf16_t*)qg, kr, vr, b, h, r0 + w * RW, wn, cc,
                            (float)a.scale, m, l, acc);
    else
      wave_attn_mx<G, P, IDX>((const bf16_t*)qg, kr, vr, b, h, r0 + w * RW, wn, idx, idx_max,
                              gap_at, gap_len, (float)a.scale, m, l, acc);
    const int i = lane & 15, g = lane >> 4;
    if (i < G) {
      float* so = s_o + (w * G + i) * kSO<D>;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int d0 = 8 * (4 * g + c);
        *(float4*)(so + d0) = float4{acc[0][c], acc[1][c], acc[2][c], acc[3][c]};
        *(float4*)(so + d0 + 4) = float4{acc[4][c], acc[5][c], acc[6][c], acc[7][c]};
      }
      if (g == 0) {
        s_m[w * G + i] = wn > 0 ? m : -INFINITY;
        s_l[w * G + i] = l;
      }
    }
  } else {
    using L = Lay<E, D>;
    float m[G], l[G], o[G][L::EPL];
    wave_attn<E, D, G, QT, CHUNK, P, IDX>(qg, kr, vr, b, h, r0 + w * RW, wn, cc, idx, idx_max,
                                          gap_at, gap_len, (float)a.scale, m, l, o);
    if (lane < L::LPR) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < L::EPL; ++e) s_o[(w * G + g) * kSO<D> + lane * L::EPL + e] = o[g][e];
    }
    if (lane == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        s_m[w * G + g] = m[g];
        s_l[w * G + g] = l[g];
      }
    }
  }
  combine_waves<G, D>(s_m, s_l, s_o, part_out);
}

// PS: the sparse tier's rows go through per-head block tables (the lifecycle
// pool under its block manager, with the ring as the dense tier, or the
// rewritten tier under its block manager, beside a cache of either layout).
// PART 0: every tile of the head; 1: the dense and sparse tiles; 2: the
// condensed tiles (grid x counts from the first condensed tile).  Launches
// whose row tiles take the matrix-core path split the two kinds, so the
// float32 chunk tiles do not set the register budget of the row tiles.
template <typename T, int D, int G, bool P, bool PS, int PART>
__device__ inline void attn_tiles(const AttnArgs& a) {
  __shared__ float s_m[4 * G], s_l[4 * G];
  __shared__ __align__(16) float s_o[4 * G * kSO<D>];
  const int h = blockIdx.y, b = blockIdx.z;
  const TileCounts tc = tile_counts(a, b, h);
  const int x = PART == 2 ? tc.ntd + tc.nts + (int)blockIdx.x : (int)blockIdx.x;
  if (x >= tc.ntd + tc.nts + (PART == 1 ? 0 : tc.ntc)) return;
  const int64_t bh = (int64_t)b * a.hkv + h;
  const T* qg = (const T*)a.q + ((int64_t)b * a.hq + (int64_t)h * G) * D;
  float* part_out = a.part + (bh * a.max_tiles + tc.first + x) * G * (D + 2);
  if (PART != 2 && x < tc.ntd) {
    // dense entries: sinks [0, S), then the window from S + A (ring: slots)
    const int r0 = x * kAttnTile;
    tile_attn<T, D, G, T, false, P>(a, qg, a.dk, a.dv, b, h, r0, min(kAttnTile, tc.nd - r0),
                                    nullptr, s_m, s_l, s_o, part_out, nullptr, 0, tc.gap_at,
                                    tc.gap_len);
  } else if (PART != 2 && x < tc.ntd + tc.nts) {
    const int r0 = (x - tc.ntd) * kAttnTile;
    const int ns = min(kAttnTile, tc.ns - r0);
    if (a.mode && a.mode[bh] == HARDKV_MODE_SPARSE) {
      // sparse loading: the kept rows stay in the cache, found through pos
      tile_attn<T, D, G, T, false, P, true>(a, qg, a.dk, a.dv, b, h, r0, ns, nullptr, s_m, s_l,
                                            s_o, part_out, a.pos + bh * a.sparse_cap,
                                            a.ctx_cap - 1);
    } else if (a.offset) {
      // packed tier: this head's slots start at row offset[b][h]
      Rows sk = a.sk, sv = a.sv;
      sk.base += (int64_t)a.offset[bh] * sk.row_bytes;
      sv.base += (int64_t)a.offset[bh] * sv.row_bytes;
      sk.region = sv.region = 0;
      tile_attn<T, D, G, T, false, false>(a, qg, sk, sv, b, h, r0, ns, nullptr, s_m, s_l, s_o,
                                          part_out);
    } else if constexpr (PS) {
      tile_attn<T, D, G, T, false, true>(a, qg, a.sk, a.sv, a.sk.tb(b, h), a.sk.th(h), r0, ns,
                                         nullptr, s_m, s_l, s_o, part_out);
    } else {
      tile_attn<T, D, G, T, false, false>(a, qg, a.sk, a.sv, b, h, r0, ns, nullptr, s_m, s_l,
                                          s_o, part_out);
    }
  } else if constexpr (PART != 1) {
    const int r0 = (x - tc.ntd - tc.nts) * kAttnTile;
    Rows ck{(const char*)a.ksum, nullptr, a.chunk_cap, a.hkv, 0, 0, D * 4};
    Rows cv{(const char*)a.vsum, nullptr, a.chunk_cap, a.hkv, 0, 0, D * 4};
    tile_attn<float, D, G, T, true, false>(a, qg, ck, cv, b, h, r0, min(kAttnTile, tc.nc - r0),
                                           a.ccount + bh * a.chunk_cap, s_m, s_l, s_o, part_out);
  }
}

// Joins the partials of every tile of R query heads of sequence b, heads
// qh0, qh0 + 4, ... (those below qh_end), each into its output row; one wave
// (lane = this thread's lane), the loads of all R rows issued together.
template <int D, int G, int R = 1>
__device__ inline void merge_rows(const AttnArgs& a, int b, int qh0, int qh_end, int lane) {
  const int h = qh0 / G;
  const TileCounts tc = tile_counts(a, b, h);
  const int nt = tc.first + tc.ntd + tc.nts + tc.ntc;
  const int64_t bh = (int64_t)b * a.hkv + h;
  constexpr int PE = D / 64;  // elements per lane
  float M[R], S[R], O[R][PE];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    M[r] = -INFINITY;
    S[r] = 0.f;
#pragma unroll
    for (int e = 0; e < PE; ++e) O[r][e] = 0.f;
  }
  constexpr int U = 8;  // partials fetched per round and row, loads issued together
  for (int x0 = 0; x0 < nt; x0 += U) {
    float pm[R][U], pl[R][U], po[R][U][PE];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int g = min(qh0 + 4 * r, qh_end - 1) % G;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int x = min(x0 + u, nt - 1);
        const float* p = a.part + ((bh * a.max_tiles + x) * G + g) * (D + 2);
        pm[r][u] = x0 + u < nt ? p[0] : -INFINITY;
        pl[r][u] = p[1];
#pragma unroll
        for (int e = 0; e < PE; ++e) po[r][u][e] = p[2 + lane * PE + e];
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float mx = pm[r][u];
        if (mx == -INFINITY) continue;
        const float nm = fmaxf(M[r], mx);
        const float fa = M[r] == -INFINITY ? 0.f : __expf(M[r] - nm);
        const float fb = __expf(mx - nm);
        S[r] = S[r] * fa + pl[r][u] * fb;
#pragma unroll
        for (int e = 0; e < PE; ++e) O[r][e] = O[r][e] * fa + po[r][u][e] * fb;
        M[r] = nm;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int qh = qh0 + 4 * r;
    if (qh >= qh_end) break;
    float* out = a.out + ((int64_t)b * a.hq + qh) * D;
#pragma unroll
    for (int e = 0; e < PE; ++e) out[lane * PE + e] = S[r] > 0.f ? O[r][e] / S[r] : 0.f;
  }
}

// Minimum waves per SIMD the compiler must leave room for: the G = 8 dense
// and sparse row tiles fit three (about 140 registers, no spills) instead of
// the two their default allocation allows; the float32 chunk tiles and the
// G = 4 tiles would spill, so they keep the default.
template <int G, int PART>
constexpr int attn_min_waves() { return G == 8 && PART == 1 ? 3 : 1; }

template <typename T, int D, int G, bool P, bool PS, int PART>
__global__ __launch_bounds__(256, (attn_min_waves<G, PART>())) void k_attn(AttnArgs a) {
  attn_tiles<T, D, G, P, PS, PART>(a);
  if constexpr (PART == 2) {
    // the step's last launch: with merge_chunks (the ring's tiers, one chunk
    // tile per head) this workgroup holds the head's only chunk tile, and
    // the row tiles' partials came from the launch before, so it joins them
    // all itself and, for head 0, advances the sequence
    if (a.merge_chunks) {
      const int h = blockIdx.y, b = blockIdx.z;
      if (blockIdx.x != 0) return;
      __syncthreads();  // this tile's partial is written
      const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
      // wave w joins query heads w, w + 4, ... of this KV head
      if (w < G) merge_rows<D, G, (G + 3) / 4>(a, b, h * G + w, (h + 1) * G, lane);
      if (h == 0 && threadIdx.x == 0) a.advance[b] += 1;
    }
  }
}

// One wave per (b, query head): joins the partials of every tile.  With
// a.advance (the lifecycle), thread i < B also moves sequence i on by one
// token; nothing in this launch reads those lengths.
template <typename T, int D, int G>
__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
  if (a.advance) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < a.B) a.advance[i] += 1;
  }
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wid >= a.B * a.hq) return;
  merge_rows<D, G>(a, wid / a.hq, wid % a.hq, wid % a.hq + 1, lane);
}

// W: dense rows at most (window plus sinks)
// (the fused compaction's tiles hold at least 512 candidates, so they fit in
// the sparse tier's slots too)
int attn_max_tiles(int W, int sparse_cap, int chunk_cap) {
  return ceil_div(W, kAttnTile) + ceil_div(sparse_cap, kAttnTile) + ceil_div(chunk_cap, kAttnTile);
}

template <typename T, int D, int G, bool P>
static void launch_attn_t(const AttnArgs& a, hipStream_t st) {
  constexpr bool split = kUseMx<T, D, G, false> && G >= 8;
  const int gd = ceil_div(a.W + a.sinks, kAttnTile), gc = ceil_div(a.chunk_cap, kAttnTile);
  const int gx = a.fused_tt > 0 ? gd : a.max_tiles;
  int grows = split && a.fused_tt == 0 ? gx - gc : gx;
  // an odd row grid: workgroups go to the XCDs round-robin by linear id, so
  // with an even one the first (ring or dense) tile of every head would fall
  // on half the XCDs or fewer; the extra workgroup finds no tile and returns
  if (grows > 1 && (grows & 1) == 0) ++grows;
  // sparse tier through per-head block tables: the lifecycle's pool, or the
  // rewritten tier under its block manager
  const bool pool_paged = a.sk.table != nullptr;
  if (grows > 0) {
    observe("k_attn", st);
    const dim3 grid(grows, a.hkv, a.B);
    if (pool_paged)
      hipLaunchKernelGGL((k_attn<T, D, G, P, true, split ? 1 : 0>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((k_attn<T, D, G, P, false, split ? 1 : 0>), grid, dim3(256), 0, st, a);
  }
  if (split && gc > 0 && a.fused_tt == 0) {
    // the ring's tiers give every head exactly ceil(chunk_cap / tile) chunk
    // tiles; with one, that tile joins the head's partials (no merge launch)
    AttnArgs c = a;
    c.merge_chunks = a.ring && gc == 1;
    observe("k_attn_chunks", st);
    hipLaunchKernelGGL((k_attn<T, D, G, false, false, 2>), dim3(gc, a.hkv, a.B), dim3(256), 0, st,
                       c);
    if (c.merge_chunks) return;
  }
  observe("k_attn_merge", st);
  hipLaunchKernelGGL((k_attn_merge<T, D, G>), dim3(ceil_div((int64_t)a.B * a.hq, 4)), dim3(256),
                     0, st, a);
}

void launch_attn(const AttnArgs& a, hipStream_t st) {
  HK_DISPATCH_P(a.dtype, a.D, a.G, a.dk.table != nullptr, launch_attn_t, a, st);
}

}  // namespace hk
