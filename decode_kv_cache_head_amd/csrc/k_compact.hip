// Index Regularization (HARD-KV, gist.science technical summary, section
// 2.C: Rewrite Cache moves the selected tokens into contiguous ranges,
// Flatten Index pads every head to the maximum length) and the condensed
// tier (section 2.A, Tier 3: evicted tokens merged into constant-size
// storage).
//
// Single step: a tile is a whole number of position-aligned chunks (about
// 1024 tokens, or one chunk when chunks are longer), processed in 64-row
// sub-tiles.  A workgroup finds its first destination slot by counting the
// kept tokens before its tile in the mask (one byte per token, L2-resident),
// so tiles are independent and the rewrite is one launch.  Rows are staged
// through LDS with 16-byte coalesced loads; kept rows are stored to their
// slots as bit copies, evicted rows are summed into per-chunk float32 sums by
// one thread per (tensor, dim), in ascending position order.  Sequences with
// no candidate tokens write count = 0 from the first tile slot.
//
// Sparse Loading (section 2.C, "Techniques"): a head whose mode byte says
// HARDKV_MODE_SPARSE gets its positions, count and chunks but no row copies;
// attention later loads its kept rows from the cache through the positions.
//
// Lifecycle (in place): k_compact_inplace runs one workgroup per (b, h) that
// sweeps its pool in sub-tiles in order, reading each sub-tile before any of
// its rows is written back and the next one while it is written.  A kept row
// only moves to a slot at or below its own, so the left compaction never
// overwrites a row that has not been read.  Evicted rows are added to the
// running sums of chunk pos / C.
#include <type_traits>

#include "inplace_core.h"

namespace hk {

// Per-token weights of attention-weighted merging for one (b, h): the
// token's calibrated value c from the selection's scores and statistics.
struct MergeW {
  const float* x;
  double shift, scale;
  float m;
  bool on;
  __device__ inline float at(int t) const { return merge_weight(cval(x[t], shift, scale), m); }
};

__device__ inline MergeW merge_w(const CompactArgs& a, int h, int64_t bh) {
  MergeW r{};
  r.on = a.merge == HARDKV_MERGE_WEIGHTED;
  if (r.on) {
    const bool l2 = aux_metric(a.metric, h);
    r.x = (l2 ? a.l2 : a.logit) + bh * a.cap_stride;
    const double* st = a.stats + bh * 4;
    r.shift = st[0];
    r.scale = st[1];
    r.m = (float)st[2];
  }
  return r;
}

__device__ inline int block_excl_scan_256(int v, int* sh, int& total) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (l >= o) incl += u;
  }
  __syncthreads();
  if (l == 63) sh[w] = incl;
  __syncthreads();
  int off = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < w) off += sh[i];
    total += sh[i];
  }
  return off + incl - v;
}

// Two exclusive prefix sums over the 256 threads in one pass (the same two
// barriers as one): returns v1's prefix, v0's goes to ex0, the totals to
// t0 / t1.  sh holds 8 ints.
__device__ inline int block_excl_scan2_256(int v0, int v1, int* sh, int& ex0, int& t0,
                                           int& t1) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  int i0 = v0, i1 = v1;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u0 = __shfl_up(i0, o, 64), u1 = __shfl_up(i1, o, 64);
    if (l >= o) {
      i0 += u0;
      i1 += u1;
    }
  }
  __syncthreads();
  if (l == 63) {
    sh[w] = i0;
    sh[4 + w] = i1;
  }
  __syncthreads();
  int o0 = 0, o1 = 0;
  t0 = 0;
  t1 = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < w) {
      o0 += sh[i];
      o1 += sh[4 + i];
    }
    t0 += sh[i];
    t1 += sh[4 + i];
  }
  ex0 = o0 + i0 - v0;
  return o1 + i1 - v1;
}

template <typename T, int D, bool P>
__global__ __launch_bounds__(256) void k_compact(CompactArgs a, int TT) {
  constexpr int RB = D * (int)sizeof(T);
  constexpr int CPR = RB / 16;
  constexpr int PIECES = 2 * 64 * CPR;     // K and V pieces of one 64-row sub-tile
  constexpr int PER = PIECES / 256;
  __shared__ __attribute__((aligned(16))) unsigned char sk[64 * RB];
  __shared__ __attribute__((aligned(16))) unsigned char sv[64 * RB];
  __shared__ int s_rank[64];
  __shared__ int s_sel[64];
  __shared__ float s_w[64];
  __shared__ int s_base;
  __shared__ int s_scan[4];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int n = a.cand.n(b, h);
  const int t0 = j * TT;
  const int64_t bh = (int64_t)b * a.hkv + h;
  if (t0 >= n) {
    if (j == 0 && tid == 0) a.out_count[bh] = 0;
    return;
  }
  const int tend = min(t0 + TT, n);
  const bool copy_rows = a.mode == nullptr || a.mode[bh] == HARDKV_MODE_REWRITE;
  const uint8_t* mk = a.mask + bh * a.cap_stride;
  const int64_t slot0 = a.offset ? (int64_t)a.offset[bh] : a.tier_table ? 0 : bh * a.cap_stride;
  char* ok = a.out_k + slot0 * RB;
  char* ov = a.out_v + slot0 * RB;
  int32_t* pos = a.out_pos + bh * a.cap_stride;
  // first destination slot of this tile: kept tokens before t0
  int base;
  {
    int c = 0;
#pragma unroll 8
    for (int t = tid; t < t0; t += 256) c += mk[t] != 0;
    int total;
    block_excl_scan_256(c, s_scan, total);
    base = total;
  }

  const bool summer = tid < 2 * D;
  const int tensor = tid / D, dim = tid % D;
  const MergeW mw = merge_w(a, h, bh);
  float acc = 0.f, wsum = 0.f;
  int cnt = 0;
  int cur = t0 / a.C;
  auto flush = [&](int ch) {
    float* dst = (tensor ? a.vsum : a.ksum) + (bh * a.chunk_stride + ch) * D + dim;
    *dst = mw.on ? (cnt > 0 ? acc * ((float)cnt / wsum) : 0.f) : acc;
    if (tid == 0) a.ccount[bh * a.chunk_stride + ch] = cnt;
  };

  for (int s0 = t0; s0 < tend; s0 += 64) {
    const int nr = min(64, tend - s0);
    if (tid < 64) {
      const bool sel = tid < nr && mk[s0 + tid] != 0;
      const unsigned long long bal = __ballot(sel);
      const int rk = base + __popcll(bal & ((1ull << tid) - 1ull));
      s_sel[tid] = sel;
      s_rank[tid] = rk;
      if (sel) pos[rk] = a.pos_off + s0 + tid;
      if (mw.on) s_w[tid] = tid < nr ? mw.at(s0 + tid) : 0.f;
      if (tid == 0) s_base = base + __popcll(bal);
    }
    v4u buf[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int tsr = k / (PER / 2), rem = (k % (PER / 2)) * 256 + tid, r = rem / CPR, c = rem % CPR;
      // rows past the sub-tile re-read its last row (in bounds, never stored)
      const int t = s0 + min(r, nr - 1);
      const char* src = tsr ? a.vrows.template row<P>(b, h, t) : a.krows.template row<P>(b, h, t);
      buf[k] = __builtin_nontemporal_load((const v4u*)(src + c * 16));
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int tsr = k / (PER / 2), rem = (k % (PER / 2)) * 256 + tid, r = rem / CPR, c = rem % CPR;
      *(v4u*)((tsr ? sv : sk) + r * RB + c * 16) = buf[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int tsr = k / (PER / 2), rem = (k % (PER / 2)) * 256 + tid, r = rem / CPR, c = rem % CPR;
      if (copy_rows && r < nr && s_sel[r]) {
        const int64_t drow = a.tier_table ? a.tier_slot(bh, s_rank[r]) : (int64_t)s_rank[r];
        if (drow >= 0)
          __builtin_nontemporal_store(*(const v4u*)((tsr ? sv : sk) + r * RB + c * 16),
                                      (v4u*)((tsr ? ov : ok) + drow * RB + c * 16));
      }
    }
    if (summer) {
      const T* src = (const T*)(tensor ? sv : sk);
      for (int r = 0; r < nr; ++r) {
        const int ch = (s0 + r) / a.C;
        if (ch != cur) {
          flush(cur);
          cur = ch;
          acc = 0.f;
          wsum = 0.f;
          cnt = 0;
        }
        if (!s_sel[r]) {
          const float x = Elt<T>::load1(src + r * D + dim);
          if (mw.on) {
            acc = fmaf(s_w[r], x, acc);
            wsum += s_w[r];
          } else {
            acc += x;
          }
          ++cnt;
        }
      }
    }
    base = s_base;
    __syncthreads();
  }
  if (summer) flush(cur);
  if (tid == 0 && tend == n) a.out_count[bh] = base;
}

// Fast path for chunks that are whole multiples of 64 rows.  One tile
// (<= 1024 rows, whole chunks) per workgroup: the ranks of all its rows are
// computed once (block scan of the mask), then every wave streams whole
// 64-row units of the tile (wave w takes units w, w + 4, ...) through
// registers in steps of 4 KB per tensor, the next step's loads issued before
// the current one is processed (ping-pong buffers), with no workgroup
// barrier until the tile ends.  Lane (g, c) of a wave owns 16-byte piece c
// of rows g, g + RGW, ... of a step; kept pieces go straight to their slot,
// evicted ones are added to per-lane float32 partial sums.  At the end of a
// unit the wave reduces its partials across its row groups (lane shuffles)
// into LDS; at the end of the tile the units of each chunk are added in unit
// order and stored: deterministic, and one barrier per tile instead of two
// per 64 rows.  In the fused step, tiles that keep under 1/8 of their rows
// run a copy of the streaming loop that skips the attention arithmetic of
// units without a kept row; denser tiles run the copy without that branch
// (it costs them more than it saves).  The fused step's tile also attends
// the condensed chunks it has just formed (a tile holds whole chunks, so
// every chunk's sum is final inside its tile): each non-empty chunk enters
// the tile's partial with key ksum / n, value vsum / n and logit
// q.(ksum / n) / sqrt(d) + ln n, from the float32 sums as stored, so the
// sums are never read back from memory.
template <typename T, int D, int G, bool P, bool ATTN, bool WMERGE>
__global__ __launch_bounds__(256) void k_compact_fast(CompactArgs a, int TT) {
  constexpr int RB = D * (int)sizeof(T);
  constexpr int CPR = RB / 16;         // pieces per row
  constexpr int EPC = Elt<T>::kPer16;  // elements per piece
  constexpr int RGW = 64 / CPR;        // row groups per wave
  constexpr int RPT = 4;               // rows per lane per step
  constexpr int SR = RPT * RGW;        // rows per step (4 KB of each tensor)
  constexpr int SPU = 64 / SR;         // steps per 64-row unit
  constexpr int NB = 2 * RPT;          // pieces per lane per step (K and V)
  constexpr int MAXU = 16;             // units per tile (TT <= 1024)
  constexpr int GA = ATTN ? G : 1;
  __shared__ int s_rank[1024];
  __shared__ float s_unit[MAXU][2][D];  // per-unit sums of the evicted rows
  __shared__ float s_unitw[WMERGE ? MAXU : 1];
  __shared__ int s_evc[MAXU];           // evicted rows per chunk of the tile
  __shared__ int s_scan[8];
  __shared__ unsigned s_kept_sub;       // bit u: unit u holds a kept row
  __shared__ int s_kept_tile;           // kept rows in the tile
  __shared__ float s_am[4][GA], s_al[4][GA];
  __shared__ float s_ao[ATTN ? 4 * G * D : 1];
  __shared__ float s_q[ATTN ? G * D : 1];          // the group's queries, float32
  __shared__ float s_cl[ATTN ? MAXU * G : 1];      // chunk logits (-inf: empty chunk)
  __shared__ float s_cf[ATTN ? MAXU * G : 1];      // chunk weights against the tile max
  __shared__ float s_cv[ATTN ? MAXU * G : 1];      // ... divided by the chunk's count
  __shared__ float s_M[GA];                         // tile max per query head
  __shared__ int s_tab[1024 / 16 + 2];              // block ids of the tile's kept slots
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int n = a.cand.n(b, h);
  const int t0 = j * TT;
  const int64_t bh = (int64_t)b * a.hkv + h;
  if (t0 >= n) {
    if (j == 0 && tid == 0) a.out_count[bh] = 0;
    return;
  }
  const int nrows = min(TT, n - t0);
  const bool copy_rows = a.mode == nullptr || a.mode[bh] == HARDKV_MODE_REWRITE;
  const uint8_t* mk = a.mask + bh * a.cap_stride;
  const int64_t slot0 = a.offset ? (int64_t)a.offset[bh] : a.tier_table ? 0 : bh * a.cap_stride;
  char* ok = a.out_k + slot0 * RB;
  char* ov = a.out_v + slot0 * RB;
  int32_t* pos = a.out_pos + bh * a.cap_stride;
  if (tid < MAXU) s_evc[tid] = 0;
  if (tid == 0) s_kept_sub = 0u;

  // kept tokens before the tile (the select's per-block counts when given,
  // tiles starting on block boundaries; else the mask bytes before it) and
  // the ranks of the tile's rows (rows 4 tid .. 4 tid + 3, one unit; -1 =
  // evicted): both counts are read together and scanned in one pass
  int base;
  {
    int c = 0;
    if (a.kept_blk) {
      // fewer blocks than kept_stride <= kKeptMaxBlks: one count per thread
      static_assert(kKeptMaxBlks <= 256, "one block count per thread");
      if (tid < t0 / kKeptBlk) c = a.kept_blk[bh * a.kept_stride + tid];
    } else {
#pragma unroll 8
      for (int t = tid; t < t0; t += 256) c += mk[t] != 0;
    }
    int c4 = 0, ev4 = 0, flags = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 4 * tid + q;
      const bool sel = r < nrows && mk[t0 + r] != 0;
      flags |= (int)sel << q;
      c4 += sel;
      ev4 += r < nrows && !sel;
    }
    int ex_unused, total;
    const int pre = block_excl_scan2_256(c, c4, s_scan, ex_unused, base, total);
    int rk = base + pre;
    if (tid == 0) s_kept_tile = total;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 4 * tid + q;
      if (r < nrows) {
        if ((flags >> q) & 1) {
          s_rank[r] = rk;
          pos[rk] = a.pos_off + t0 + r;
          ++rk;
        } else {
          s_rank[r] = -1;
        }
      }
    }
    if (c4) atomicOr(&s_kept_sub, 1u << (tid >> 4));  // unit of rows 4 tid..
    if (ev4) atomicAdd(&s_evc[(4 * tid) / a.C], ev4);
    if (t0 + nrows == n && tid == 255) a.out_count[bh] = rk;
  }
  __syncthreads();
  // block manager: the block ids of the tile's kept slots [base, base + kept)
  int tab0 = 0;
  if (a.tier_table && copy_rows) {
    tab0 = base >> a.tier_lbs;
    const int nt = s_kept_tile > 0 ? ((base + s_kept_tile - 1) >> a.tier_lbs) - tab0 + 1 : 0;
    if (tid < nt) {
      // a block id outside the pool (a tier never allocated) stores nothing
      const int id = tab0 + tid < a.tier_maxb ? a.tier_table[bh * a.tier_maxb + tab0 + tid] : -1;
      s_tab[tid] = id >= 0 && id < a.tier_nblocks ? id : -1;
    }
    __syncthreads();
  }
  // destination row of kept slot rk, -1: none
  auto dest_row = [&](int rk) -> int64_t {
    if (!a.tier_table) return rk;
    const int id = s_tab[(rk >> a.tier_lbs) - tab0];
    return id < 0 ? -1 : ((int64_t)id << a.tier_lbs) + (rk & ((1 << a.tier_lbs) - 1));
  };

  const int w = tid >> 6, lane = tid & 63;
  const int c = lane % CPR, rg = lane / CPR;
  const int nunits = (nrows + 63) / 64;
  const int my_units = nunits > w ? (nunits - w + 3) / 4 : 0;
  const int nsteps = my_units * SPU;
  MergeW mw{};
  if constexpr (WMERGE) mw = merge_w(a, h, bh);
  float acc[2][EPC];
  float wacc = 0.f;  // weighted merging: sum of this lane's evicted rows' weights
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[q][e] = 0.f;
  // attention over the kept rows (fused): running max, sum and numerator of
  // this lane's row group for every query head of the GQA group
  QPiece<T, T, EPC> qp[GA];
  float am[GA], al[GA], ao[GA][EPC];
  if constexpr (ATTN) {
    const T* qg = (const T*)a.q + ((int64_t)b * a.hq + (int64_t)h * G) * D;
    for (int i = tid; i < G * D; i += 256) s_q[i] = Elt<T>::load1(qg + i);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      qp[g].load(qg + g * D + c * EPC);
      am[g] = -INFINITY;
      al[g] = 0.f;
#pragma unroll
      for (int e = 0; e < EPC; ++e) ao[g][e] = 0.f;
    }
  }

  // step k of this wave: unit w + 4 (k / SPU), rows (k % SPU) * SR + rg + RGW i
  auto first_row = [&](int k) { return (w + 4 * (k / SPU)) * 64 + (k % SPU) * SR + rg; };
  auto load = [&](v4u (&buf)[NB], int k) {
    const int r0 = first_row(k);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = min(r0 + RGW * i, nrows - 1);
      // streamed once: non-temporal, so the pass does not flush what the
      // following kernels read (chunk sums, dense rows) out of the caches
      buf[i] = __builtin_nontemporal_load((const v4u*)(a.krows.template row<P>(b, h, t0 + r) + c * 16));
      buf[RPT + i] =
          __builtin_nontemporal_load((const v4u*)(a.vrows.template row<P>(b, h, t0 + r) + c * 16));
    }
  };
  auto process = [&](const v4u (&buf)[NB], int k, auto skip) {
    const int u = w + 4 * (k / SPU);
    const int r0 = first_row(k);
    // attention over the unit's rows; sparse tiles skip units with no kept row
    if constexpr (ATTN) if (!decltype(skip)::value || ((s_kept_sub >> u) & 1u)) {
      float sc[RPT][G], mr[G];
#pragma unroll
      for (int g = 0; g < G; ++g) mr[g] = -INFINITY;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int r = r0 + RGW * i;
        const bool kept = r < nrows && s_rank[min(r, nrows - 1)] >= 0;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float dot = group_sum<CPR>(qp[g].dot(buf[i]));
          sc[i][g] = kept ? dot * a.scale : -INFINITY;
          mr[g] = fmaxf(mr[g], sc[i][g]);
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float mn = fmaxf(am[g], mr[g]);
        const float alpha = am[g] == -INFINITY ? 0.f : __expf(am[g] - mn);
        al[g] *= alpha;
#pragma unroll
        for (int e = 0; e < EPC; ++e) ao[g][e] *= alpha;
        am[g] = mn;
      }
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        float f[EPC];
        Elt<T>::unpack(buf[RPT + i], f);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float pr = sc[i][g] == -INFINITY ? 0.f : __expf(sc[i][g] - am[g]);
          al[g] += pr;
#pragma unroll
          for (int e = 0; e < EPC; ++e) ao[g][e] = fmaf(pr, f[e], ao[g][e]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = r0 + RGW * i;
      if (r < nrows) {
        const int rk = s_rank[r];
        if (rk >= 0) {
          const int64_t dr = copy_rows ? dest_row(rk) : -1;
          if (dr >= 0) {
            __builtin_nontemporal_store(buf[i], (v4u*)(ok + dr * RB + c * 16));
            __builtin_nontemporal_store(buf[RPT + i], (v4u*)(ov + dr * RB + c * 16));
          }
        } else if (WMERGE) {
          const float wt = mw.at(t0 + r);
          wacc += wt;
          float f[EPC];
          Elt<T>::unpack(buf[i], f);
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[0][e] = fmaf(wt, f[e], acc[0][e]);
          Elt<T>::unpack(buf[RPT + i], f);
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[1][e] = fmaf(wt, f[e], acc[1][e]);
        } else {
          float f[EPC];
          Elt<T>::unpack(buf[i], f);
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[0][e] += f[e];
          Elt<T>::unpack(buf[RPT + i], f);
#pragma unroll
          for (int e = 0; e < EPC; ++e) acc[1][e] += f[e];
        }
      }
    }
    // end of the unit: its sums across this wave's row groups go to LDS
    if (k % SPU == SPU - 1) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          float v = acc[q][e];
#pragma unroll
          for (int o = CPR; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
          acc[q][e] = 0.f;
          if (lane < CPR) s_unit[u][q][c * EPC + e] = v;
        }
      if (WMERGE) {
        float v = wacc;
#pragma unroll
        for (int o = CPR; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
        if (lane == 0) s_unitw[u] = v;
        wacc = 0.f;
      }
    }
  };

  auto stream = [&](auto skip) {
    v4u A_[NB], B_[NB];
    if (nsteps > 0) load(A_, 0);
    for (int k = 0; k < nsteps; k += 2) {
      if (k + 1 < nsteps) load(B_, k + 1);
      process(A_, k, skip);
      if (k + 1 < nsteps) {
        if (k + 2 < nsteps) load(A_, k + 2);
        process(B_, k + 1, skip);
      }
    }
  };
  if (!ATTN || 8 * s_kept_tile >= nrows)
    stream(std::false_type{});
  else
    stream(std::true_type{});
  if constexpr (ATTN) {
    // join the row groups of each wave, then the four waves; one partial
    // (max, sum, numerator) per query head for this tile
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mw_ = across_groups_max<CPR>(am[g]);
      const float f = am[g] == -INFINITY ? 0.f : __expf(am[g] - mw_);
      al[g] = across_groups_sum<CPR>(al[g] * f);
#pragma unroll
      for (int e = 0; e < EPC; ++e) ao[g][e] = across_groups_sum<CPR>(ao[g][e] * f);
      am[g] = mw_;
    }
    if (lane < CPR) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < EPC; ++e) s_ao[(w * G + g) * D + lane * EPC + e] = ao[g][e];
    }
    if (lane == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        s_am[w][g] = am[g];
        s_al[w][g] = al[g];
      }
    }
  }
  __syncthreads();
  // chunks of the tile: units added in unit order
  {
    const int ch0 = t0 / a.C;
    const int upc = a.C / 64;
    const int nch = (nrows + a.C - 1) / a.C;
    for (int idx = tid; idx < nch * 2 * D; idx += 256) {
      const int cl = idx / (2 * D), q = (idx / D) & 1, dim = idx % D;
      const int u1 = min((cl + 1) * upc, nunits);
      float v = 0.f, wt = 0.f;
      for (int u = cl * upc; u < u1; ++u) {
        v += s_unit[u][q][dim];
        if (WMERGE) wt += s_unitw[u];
      }
      if (WMERGE) {
        const int ne = s_evc[cl];
        v = ne > 0 ? v * ((float)ne / wt) : 0.f;
      }
      (q ? a.vsum : a.ksum)[(bh * a.chunk_stride + ch0 + cl) * D + dim] = v;
      // the stored chunk sum, kept for the attention below in the slot of
      // the chunk's first unit (read above by this thread only)
      if (ATTN) s_unit[cl * upc][q][dim] = v;
    }
    if (tid < nch) a.ccount[bh * a.chunk_stride + ch0 + tid] = s_evc[tid];
  }
  if constexpr (ATTN) {
    const int upc = a.C / 64;
    const int nch = (nrows + a.C - 1) / a.C;
    __syncthreads();
    // chunk logits: wave w takes chunks w, w + 4, ...; each lane holds D / 64
    // dimensions of the chunk's key sum, the dot products are wave sums
    for (int cl = w; cl < MAXU; cl += 4) {
      const int ne = cl < nch ? s_evc[cl] : 0;  // uniform over the wave
      if (ne > 0) {
        const float* ks = s_unit[cl * upc][0];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float dot = 0.f;
#pragma unroll
          for (int e = lane; e < D; e += 64) dot = fmaf(s_q[g * D + e], ks[e], dot);
          dot = group_sum<64>(dot);
          if (lane == 0) s_cl[cl * G + g] = dot / (float)ne * a.scale + __logf((float)ne);
        }
      } else if (lane < G) {
        s_cl[cl * G + lane] = -INFINITY;
      }
    }
    __syncthreads();
    // per (chunk, query head): its weight against the head's maximum over the
    // tile (kept rows of the four waves and the chunks), and the value weight
    // (the chunk's value is vsum / n)
    if (tid < MAXU * G) {
      const int cl = tid / G, g = tid % G;
      float M = -INFINITY;
#pragma unroll
      for (int v = 0; v < 4; ++v) M = fmaxf(M, s_am[v][g]);
      for (int x = 0; x < nch; ++x) M = fmaxf(M, s_cl[x * G + g]);
      const float lg = s_cl[cl * G + g];
      const float f = cl < nch && lg != -INFINITY ? __expf(lg - M) : 0.f;
      s_cf[cl * G + g] = f;
      s_cv[cl * G + g] = f > 0.f ? f / (float)s_evc[cl] : 0.f;
      if (cl == 0) s_M[g] = M;
    }
    __syncthreads();
    float* part_out = a.part + (bh * a.max_tiles + j) * G * (D + 2);
    for (int i = tid; i < G * D; i += 256) {
      const int g = i / D, e = i % D;
      const float M = s_M[g];
      float O = 0.f, S = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if (s_am[v][g] != -INFINITY) {
            const float f = __expf(s_am[v][g] - M);
            O = fmaf(f, s_ao[(v * G + g) * D + e], O);
            S = fmaf(f, s_al[v][g], S);
          }
        }
        for (int cl = 0; cl < nch; ++cl) {
          O = fmaf(s_cv[cl * G + g], s_unit[cl * upc][1][e], O);
          S += s_cf[cl * G + g];
        }
      }
      float* pp = part_out + g * (D + 2);
      pp[2 + e] = O;
      if (e == 0) {
        pp[0] = M;
        pp[1] = S;
      }
    }
  }
}

template <typename T, int D, int G_unused, bool P>
static void launch_compact_t(const CompactArgs& a, hipStream_t st) {
  const int TT = compact_tile(a.C, a.max_cand);
  const int nt = max(1, ceil_div(a.max_cand, TT));  // tile 0 also writes count = 0
  if (compact_fusable(a.C)) {
    observe("k_compact_fast", st);
    if (a.merge == HARDKV_MERGE_WEIGHTED)
      hipLaunchKernelGGL((k_compact_fast<T, D, 1, P, false, true>), dim3(nt, a.hkv, a.B),
                         dim3(256), 0, st, a, TT);
    else
      hipLaunchKernelGGL((k_compact_fast<T, D, 1, P, false, false>), dim3(nt, a.hkv, a.B),
                         dim3(256), 0, st, a, TT);
  } else {
    observe("k_compact", st);
    hipLaunchKernelGGL((k_compact<T, D, P>), dim3(nt, a.hkv, a.B), dim3(256), 0, st, a, TT);
  }
}

void launch_compact(const CompactArgs& a, hipStream_t st) {
  HK_DISPATCH_P(a.dtype, a.D, 1, a.krows.table != nullptr, launch_compact_t, a, st);
}

template <typename T, int D, int G, bool P>
static void launch_compact_attn_t(const CompactArgs& a, hipStream_t st) {
  const int TT = compact_tile(a.C, a.max_cand);
  const int nt = max(1, ceil_div(a.max_cand, TT));
  observe("k_compact_attn", st);
  if (a.merge == HARDKV_MERGE_WEIGHTED)
    hipLaunchKernelGGL((k_compact_fast<T, D, G, P, true, true>), dim3(nt, a.hkv, a.B),
                       dim3(256), 0, st, a, TT);
  else
    hipLaunchKernelGGL((k_compact_fast<T, D, G, P, true, false>), dim3(nt, a.hkv, a.B),
                       dim3(256), 0, st, a, TT);
}

void launch_compact_attn(const CompactArgs& a, hipStream_t st) {
  HK_DISPATCH_P(a.dtype, a.D, a.G, a.krows.table != nullptr, launch_compact_attn_t, a, st);
}

// ------------------------------------------------------------ in place ----
// One workgroup of 512 threads per (b, h): compact_inplace_head
// (inplace_core.h) with its own LDS.
template <typename T, int D>
__global__ __launch_bounds__(512) void k_compact_inplace(CompactArgs a) {
  __shared__ InplaceLds<T, D> L;
  const int h = blockIdx.x, b = blockIdx.y;
  compact_inplace_head<T, D, true>(a, b, h, a.cand.n(b, h), L);
}

template <typename T, int D, int G_unused>
static void launch_compact_inplace_t(const CompactArgs& a, hipStream_t st) {
  observe("k_compact_inplace", st);
  hipLaunchKernelGGL((k_compact_inplace<T, D>), dim3(a.hkv, a.B), dim3(512), 0, st, a);
}

void launch_compact_inplace(const CompactArgs& a, hipStream_t st) {
  HK_DISPATCH(a.dtype, a.D, 1, launch_compact_inplace_t, a, st);
}

}  // namespace hk
