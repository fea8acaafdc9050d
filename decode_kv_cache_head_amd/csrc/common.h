// Device helpers shared by the HARD-KV gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hardkv.h"

namespace hk {

// ---------------------------------------------------------------- elements --
// 16-byte piece as a native vector: loads and stores stay single
// instructions and register arrays of pieces are promoted to VGPRs.
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

struct bf16_t {
  uint16_t bits;
};

template <typename T>
struct Elt;
template <>
struct Elt<float> {
  static constexpr int kPer16 = 4;  // elements per 16-byte piece
  __device__ static inline void unpack(const v4u& v, float (&f)[4]) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
  __device__ static inline float load1(const float* p) { return *p; }
};
template <>
struct Elt<bf16_t> {
  static constexpr int kPer16 = 8;
  // bf16 -> f32 is exact: the 16 bits are the high half of the f32 pattern.
  __device__ static inline void unpack(const v4u& v, float (&f)[8]) {
    f[0] = __uint_as_float(v.x << 16);
    f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16);
    f[3] = __uint_as_float(v.y & 0xffff0000u);
    f[4] = __uint_as_float(v.z << 16);
    f[5] = __uint_as_float(v.z & 0xffff0000u);
    f[6] = __uint_as_float(v.w << 16);
    f[7] = __uint_as_float(v.w & 0xffff0000u);
  }
  __device__ static inline float load1(const bf16_t* p) {
    return __uint_as_float(((uint32_t)p->bits) << 16);
  }
};

// ------------------------------------------------------------ row sources --
// Where the rows of one tensor live for every (sequence b, KV head h).
//   contiguous: row(b, h, t) = base + ((b * Hkv + h) * region + t) * row_bytes
//   paged:      row(b, h, t) = base + ((table[b][t >> lbs] * Hkv + h) * bs + (t & (bs-1))) * row_bytes
struct Rows {
  const char* base;
  const int32_t* table;
  int64_t region;
  int32_t hkv;
  int32_t lbs;  // log2(block size) when paged
  int32_t max_blocks;
  int32_t row_bytes;
  int32_t off;  // added to every position (the first candidate position)
  // > 0: per-head block tables (the lifecycle pool's block manager): blocks
  // hold one head's rows and sequence b's head h uses table row b * headtab + h;
  // row() is then called with tb(b, h), th(h) (hkv = 1 in that case)
  int32_t headtab;
  __device__ inline int tb(int b, int h) const { return headtab ? b * headtab + h : b; }
  __device__ inline int th(int h) const { return headtab ? 0 : h; }
  // PAGED is a compile-time property of the launch, so the unrolled loads of
  // a tile stay in one basic block.
  template <bool PAGED>
  __device__ inline const char* row(int b, int h, int t) const {
    t += off;
    if constexpr (PAGED) {
      int blk = table[(int64_t)b * max_blocks + (t >> lbs)];
      blk = blk < 0 ? 0 : blk;  // an unset entry (-1) reads block 0, never before the pool
      return base + ((((int64_t)blk * hkv + h) << lbs) + (t & ((1 << lbs) - 1))) * row_bytes;
    } else {
      return base + (((int64_t)b * hkv + h) * region + t) * row_bytes;
    }
  }
};

// Number of candidate (aged / pool) tokens of (b, h).
//   single step: clamp(ctx_len[b], 0, ctx_cap) - W - sinks, clamped to [0, cap]
//   lifecycle:   count[b * Hkv + h], clamped to [0, cap]
struct Cand {
  const int32_t* ctx_len;
  const int32_t* count;
  int32_t W;
  int32_t ctx_cap;
  int32_t cap;
  int32_t hkv;
  int32_t sinks;
  __device__ inline int n(int b, int h) const {
    int v;
    if (count) {
      v = count[b * hkv + h];
    } else {
      int T = ctx_len[b];
      T = T < 0 ? 0 : (T > ctx_cap ? ctx_cap : T);
      v = T - W - sinks;
    }
    v = v < 0 ? 0 : v;
    return v > cap ? cap : v;
  }
};

// ------------------------------------------------------------- ordering ---
// Order-preserving key of a float: larger value -> larger key, -0 == +0.
__device__ inline uint32_t okey(float c) {
  c = c + 0.0f;  // -0 + +0 = +0
  const uint32_t u = __float_as_uint(c);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ inline float okey_inv(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// Heads whose ranking metric is the second score array (key norm or the
// pooled window metric) rather than the raw logit.
__device__ inline bool aux_metric(const int8_t* metric, int h) {
  return metric != nullptr && metric[h] != HARDKV_METRIC_QK;
}

// Calibrated value c = fl32((x - shift) * scale).  For shift 0 and scale 1
// (QK heads) this is x itself.
__device__ inline float cval(float x, double shift, double scale) {
  return (float)(((double)x - shift) * scale);
}

// exp(x) for x <= 0 in float64, table-driven (P. T. P. Tang, "Table-driven
// implementation of the exponential function in IEEE floating-point
// arithmetic", ACM TOMS 15(2), 1989): x = k ln2/64 + r with |r| <= ln2/128
// (ln2/64 split in a 39-bit high part, so k times it is exact for the k
// here, and a low part), k = 64 q + j, exp(x) = 2^q 2^(j/64) e^r, e^r - 1
// from its Taylor series to degree 5 (truncation below 4e-17 relative).
// tab[j] = 2^(j/64) (exp_table_init).  x below -100 is taken as -100: the
// result, < 4e-44, rounds to 0 in every fixed-point use here.
__device__ inline double exp_nonpos(double x, const double* tab) {
  x = fmax(x, -100.0);
  const double kd = rint(x * 0x1.71547652b82fep+6);  // x * 64 / ln 2
  double r = fma(-kd, 0x1.62e42fefa4000p-7, x);
  r = fma(-kd, -0x1.8432a1b0e2634p-49, r);
  const double p =
      r * (1.0 + r * (0.5 + r * (1.0 / 6.0 + r * (1.0 / 24.0 + r * (1.0 / 120.0)))));
  const int k = (int)kd;
  const double t = tab[k & 63];
  return ldexp(fma(t, p, t), k >> 6);
}
// Fills tab[0..63] with 2^(j/64); threads 0..63 of the calling workgroup
// each write one entry (a barrier must follow before exp_nonpos reads it).
__device__ inline void exp_table_init(double* tab) {
  if (threadIdx.x < 64) tab[threadIdx.x] = exp2((double)threadIdx.x * (1.0 / 64.0));
}

// round(v) for 0 <= v < 2^52, ties to even: adding 2^52 leaves the nearest
// integer in the low mantissa bits.
__device__ inline uint64_t fix_round(double v) {
  return (uint64_t)__double_as_longlong(v + 0x1p52) - 0x4330000000000000ull;
}

// Fixed-point weight round(exp(c - m) * scale); exp(c - m) <= 1 and scale a
// power of two <= 2^47, so the product is exact and below 2^52.
__device__ inline uint64_t wfix(float c, double m, double scale, const double* tab) {
  return fix_round(exp_nonpos((double)c - m, tab) * scale);
}

// Fixed-point scale of the selection masses for heads of up to n_max
// candidates: each weight exp(c - m) <= 1 becomes round(w * 2^s) with
// s = min(47, 63 - ceil(log2 n_max)), so a head's total stays within 2^63
// (2^-47 units up to 65536 candidates).
inline double mass_scale(int n_max) {
  int l = 0;
  while (l < 31 && (1 << l) < n_max) ++l;
  return ldexp(1.0, 63 - l < 47 ? 63 - l : 47);
}

// ------------------------------------------------------ XCD placement ----
// The chip's 8 XCDs (each with its own L2 and scalar caches) receive the
// workgroups of a launch round-robin by linear id.  xcd_contiguous renumbers
// linear id L of N so that each XCD works through one contiguous range of
// the logical order instead: consecutive tiles of a head then run on the
// same XCD and share its caches (a bijection on [0, N)).
__device__ inline int xcd_contiguous(int L, int N) {
  constexpr int X = 8;
  const int per = (N + X - 1) / X;
  const int tall = N % X == 0 ? X : N % X;  // XCDs that receive `per` workgroups
  const int xcd = L % X, local = L / X;
  return xcd < tall ? xcd * per + local : tall * per + (xcd - tall) * (per - 1) + local;
}

// Logical id grp + ngrp * hb of a launch that gives each of nh heads (hb =
// b * Hkv + h) ngrp workgroups, all on one XCD: each XCD takes its heads in
// order, one head's workgroups after the other.  The heads are dealt to the
// XCDs in rows of 8: row r (heads 8r .. 8r + 7) gives XCD x head
// 8r + (x + r) mod 8, a rotation that changes from row to row.  With 8 KV
// heads a row is one sequence, so every XCD holds one head of each sequence
// (a batch of unequal lengths still gives the XCDs equal work, which
// contiguous ranges of heads would not) and, over 8 sequences, each KV head
// once (heads that score with different metrics, and so write different
// amounts, are spread as well).  When nh is not a multiple of 8 the XCDs
// cannot take equal head counts: then contiguous ranges (a bijection on
// [0, ngrp * nh) either way).
__device__ inline int xcd_by_head(int L, int ngrp, int nh) {
  constexpr int X = 8;
  if (nh % X) return xcd_contiguous(L, ngrp * nh);
  const int xcd = L % X, local = L / X;
  const int r = local / ngrp;
  return (r * X + (xcd + r) % X) * ngrp + local % ngrp;
}

// (b, h) of a one-workgroup-per-head launch over grid (Hkv, B), numbered as
// the tiled score launch numbers its heads (ngrp = 1), so that each head is
// selected on the XCD whose L2 received its scores.
__device__ inline void head_of_block(int& b, int& h) {
  const int id = xcd_by_head(blockIdx.x + gridDim.x * blockIdx.y, 1, gridDim.x * gridDim.y);
  h = id % gridDim.x;
  b = id / gridDim.x;
}

// ------------------------------------------------------- wave reductions --
__device__ inline double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ inline float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Sum over aligned groups of LPR lanes (LPR in {4, 8, 16, 32, 64}); every
// lane of the group receives the group's sum.  Within 16-lane DPP rows the
// exchanges use DPP moves; larger groups finish with lane shuffles.
template <int LPR>
__device__ inline float group_sum(float v) {
  // quad butterfly: xor 1, xor 2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  if constexpr (LPR == 8) {
    // row_half_mirror: lane i <-> 7 - i within each half row; after the quad
    // step this adds the other quad of the 8-lane group.
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
  } else if constexpr (LPR >= 16) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));  // row_ror:4
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));  // row_ror:8
    if constexpr (LPR >= 32) v += __shfl_xor(v, 16, 64);
    if constexpr (LPR >= 64) v += __shfl_xor(v, 32, 64);
  }
  return v;
}

// Lanes l and l ^ o for o >= LPR hold different rows; reduce across them.
template <int LPR>
__device__ inline float across_groups_max(float v) {
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
template <int LPR>
__device__ inline float across_groups_sum(float v) {
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
  return v;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// 16x16x32 bf16 matrix product, float32 accumulation: D(16x16) += A(16x32)
// B(32x16), where lane l holds A[l % 16][8 (l / 16) + j] and
// B[8 (l / 16) + j][l % 16] (j = 0..7) and D[4 (l / 16) + i][l % 16]
// (i = 0..3).  Products of bf16 values are exact in float32.
__device__ __forceinline__ f32x4_t mfma16(const v4u& a, const v4u& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Max over the 16 lanes of a DPP row; every lane of the row receives it.
// Each step keeps the larger of two values by compare and select: for the
// finite or -inf values it serves this equals fmaxf, without the NaN
// canonicalisations fmaxf adds around every DPP move.
__device__ inline float row_max16(float v) {
  float o;
  o = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));
  v = o > v ? o : v;
  o = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));
  v = o > v ? o : v;
  o = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, true));
  v = o > v ? o : v;
  o = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, true));
  v = o > v ? o : v;
  return v;
}
// The same over each group of 8 lanes (lanes 0-7 and 8-15 of every row):
// the quad maxima, then each lane against its mirror in the half row.
__device__ inline float row_max8(float v) {
  float o;
  o = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));
  v = o > v ? o : v;
  o = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));
  v = o > v ? o : v;
  o = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, true));
  v = o > v ? o : v;
  return v;
}

// Takes the word by value: bit-casting an ext-vector element in place
// (__builtin_bit_cast(T, v.y)) is compiled as a cast of element 0.
__device__ __forceinline__ bf16x2_t as_bf2(uint32_t u) { return __builtin_bit_cast(bf16x2_t, u); }

// q.k partial over one lane's 16-byte piece.  bf16 rows with bf16 queries use
// the packed dot (v_dot2c_f32_bf16, products exact, float32 accumulation);
// float rows use float FMAs.
template <typename E, typename QT, int EPL>
struct QPiece {
  float f[EPL];
  __device__ inline void load(const QT* q) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) f[e] = Elt<QT>::load1(q + e);
  }
  __device__ inline float dot(const v4u& raw) const {
    float k[EPL];
    Elt<E>::unpack(raw, k);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) s = fmaf(f[e], k[e], s);
    return s;
  }
};
template <>
struct QPiece<bf16_t, bf16_t, 8> {
  uint32_t w[4];
  __device__ inline void load(const bf16_t* q) {
    const v4u v = *(const v4u*)q;
    w[0] = v.x;
    w[1] = v.y;
    w[2] = v.z;
    w[3] = v.w;
  }
  __device__ inline float dot(const v4u& raw) const {
    float s = 0.f;
    s = __builtin_amdgcn_fdot2_f32_bf16(as_bf2(w[0]), as_bf2(raw.x), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(as_bf2(w[1]), as_bf2(raw.y), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(as_bf2(w[2]), as_bf2(raw.z), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(as_bf2(w[3]), as_bf2(raw.w), s, false);
    return s;
  }
};

// Weight of an evicted token in attention-weighted merging: its calibrated
// attention weight relative to the head's largest, floored at e^-60.
__device__ inline float merge_weight(float c, float m) { return __expf(fmaxf(c - m, -60.f)); }

// ------------------------------------------------------------ policy -----
// Rewrite (0) or sparse loading (1) for a head with A aged tokens, k kept,
// window W: budget thresholds first, then the smaller memory-time integral
// over the horizon, in K/V rows, in exact 128-bit integers (the formulas
// are documented with hardkv_policy).
__host__ __device__ inline uint8_t plan_mode(const hardkv_policy& p, int A, int k, int W) {
  if (p.kind == HARDKV_POLICY_REWRITE) return HARDKV_MODE_REWRITE;
  if (p.kind == HARDKV_POLICY_SPARSE) return HARDKV_MODE_SPARSE;
  if (k <= p.l_lower) return HARDKV_MODE_REWRITE;
  if (k >= p.l_upper) return HARDKV_MODE_SPARSE;
  typedef unsigned __int128 u128;
  const u128 a = (u128)(uint32_t)A, kk = (u128)(uint32_t)k, w = (u128)(uint32_t)W;
  const u128 reuse = (u128)(uint32_t)(p.horizon - 1);
  const u128 foot_sparse = a + w, foot_rewrite = kk + w;
  const u128 select_rows = 3 * a + 2 * w, rewrite_rows = 2 * kk, reuse_rows = 2 * (kk + w);
  const u128 mti_sparse = foot_sparse * select_rows + reuse * foot_sparse * reuse_rows;
  const u128 mti_rewrite =
      (foot_sparse + kk) * (select_rows + rewrite_rows) + reuse * foot_rewrite * reuse_rows;
  return mti_rewrite < mti_sparse ? HARDKV_MODE_REWRITE : HARDKV_MODE_SPARSE;
}

inline int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

}  // namespace hk
