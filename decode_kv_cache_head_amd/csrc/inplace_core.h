// In-place compaction of one lifecycle pool (HARD-KV, gist.science technical
// summary, section 2.C Rewrite Cache; section 2.A Tier 3), shared by the
// standalone in-place kernel and the fused lifecycle step.
//
// One workgroup of 512 threads per (b, h) sweeps the pool in order, in
// sub-tiles of 32 KB per tensor (128 bf16 rows).  A sub-tile is staged in
// LDS; while its kept rows are written to their slots and its evicted rows
// are summed, the next sub-tile is already being loaded into registers.
// Reading ahead is safe: a kept row only moves to a slot at or below its
// own, so every slot written while sub-tile s is processed lies below the
// rows of sub-tile s + 1.  Evicted rows are added to the running sums of
// chunk pos / C in ascending position order, one thread per (tensor,
// dimension); a chunk's old sums are loaded when its first evicted row is
// met and stored back when the next chunk starts.  Pool rows are streamed
// with non-temporal loads and stores.
#pragma once

#include "internal.h"

namespace hk {

constexpr int kInplaceTab = 2048;  // block-table entries a workgroup keeps in LDS

// LDS of one in-place compaction: a sub-tile of K and of V rows, their mask
// bits and positions, and the head's block table row (block manager).
// TAB false: no block manager, no table row (a.pg.table must be null).
template <typename T, int D, bool TAB = true>
struct InplaceLds {
  static constexpr int RB = D * (int)sizeof(T);
  static constexpr int SUB = 32768 / RB;  // rows per sub-tile
  static constexpr int NW = SUB / 64;     // 64-row words of mask bits
  __attribute__((aligned(16))) unsigned char sk[SUB * RB];
  __attribute__((aligned(16))) unsigned char sv[SUB * RB];
  unsigned long long s_bal[NW];
  int s_pos[SUB];
  int32_t s_tab[TAB ? kInplaceTab : 1];
};

// The in-place compaction of head (b, h) with n pool rows, by a workgroup of
// 512 threads (see k_compact_inplace).
template <typename T, int D, bool TAB>
__device__ inline void compact_inplace_head(const CompactArgs& a, int b, int h, int n,
                                            InplaceLds<T, D, TAB>& L) {
  constexpr int NT = 512;
  constexpr int RB = D * (int)sizeof(T);
  constexpr int CPR = RB / 16;        // 16-byte pieces per row
  constexpr int SUB = 32768 / RB;     // rows per sub-tile
  constexpr int NW = SUB / 64;        // 64-row words of mask bits
  constexpr int PER = 2 * SUB * CPR / NT;  // pieces per thread (K then V)
  static_assert(NW >= 1 && NW * 64 <= NT && PER % 2 == 0, "sub-tile shape");
  unsigned char* sk = L.sk;
  unsigned char* sv = L.sv;
  unsigned long long* s_bal = L.s_bal;
  int* s_pos = L.s_pos;
  int32_t* s_tab = L.s_tab;
  const int tid = threadIdx.x, w = tid >> 6;
  const int64_t bh = (int64_t)b * a.hkv + h;
  const uint8_t* mk = a.mask + bh * a.cap_stride;
  int32_t* pos = a.out_pos + bh * a.cap_stride;
  // pool row r (read and written): the head's region, or row r % bs of block
  // table[r / bs] under the block manager, with the head's table row copied
  // into LDS when it is short (a missing block reads as block 0: the tables
  // always cover [0, count))
  const int32_t* ptab = TAB && a.pg.table ? a.pg.table + bh * a.pg.maxb : nullptr;
  const bool tab_lds = TAB && ptab && a.pg.maxb <= kInplaceTab;
  if (tab_lds) {
    for (int i = tid; i < a.pg.maxb; i += NT) s_tab[i] = ptab[i];
    __syncthreads();
  }
  auto prow = [&](char* base, int r) -> char* {
    if (!ptab) return base + (bh * a.cap_stride + r) * RB;
    int blk = tab_lds ? s_tab[r >> a.pg.lbs] : ptab[r >> a.pg.lbs];
    blk = blk < 0 || blk >= a.pg.nblocks ? 0 : blk;
    return base + (((int64_t)blk << a.pg.lbs) + (r & ((1 << a.pg.lbs) - 1))) * RB;
  };

  v4u buf[PER];
  bool sel = false;
  int mypos = 0;
  auto fetch = [&](int s0) {
    const int nr = min(SUB, n - s0);
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int idx = (k % (PER / 2)) * NT + tid, r = idx / CPR, c = idx % CPR;
      buf[k] = __builtin_nontemporal_load(
          (const v4u*)(prow(k < PER / 2 ? a.out_k : a.out_v, s0 + min(r, nr - 1)) + c * 16));
    }
    if (tid < SUB) {
      sel = tid < nr && mk[s0 + tid] != 0;
      mypos = tid < nr ? pos[s0 + tid] : 0;
    }
  };
  auto kept = [&](int r) { return ((s_bal[r >> 6] >> (r & 63)) & 1ull) != 0; };

  // running chunk sums of thread (tensor, dim)
  const bool summer = tid < 2 * D;
  const int tensor = tid / D, dim = tid % D;
  float* sums = (tensor ? a.vsum : a.ksum) + bh * a.chunk_stride * D + dim;
  int32_t* cc = a.ccount + bh * a.chunk_stride;
  float acc = 0.f, old = 0.f;
  int cnt = 0, oldc = 0, cur = -1;
  auto flush = [&]() {
    if (cur < 0 || cur >= a.chunk_stride) return;  // positions outside the chunk capacity
    sums[(int64_t)cur * D] = old + acc;
    if (tid == 0) cc[cur] = oldc + cnt;
  };

  int base = 0;
  if (n > 0) fetch(0);
  for (int s0 = 0; s0 < n; s0 += SUB) {
    const int nr = min(SUB, n - s0);
    if (w < NW) {
      const unsigned long long bal = __ballot(sel);
      if ((tid & 63) == 0) s_bal[w] = bal;
      s_pos[tid] = mypos;
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int idx = (k % (PER / 2)) * NT + tid, r = idx / CPR, c = idx % CPR;
      if (r < nr) *(v4u*)((k < PER / 2 ? sk : sv) + r * RB + c * 16) = buf[k];
    }
    __syncthreads();  // the sub-tile, its positions and mask bits are in LDS
    int total = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) total += __popcll(s_bal[v]);
    auto rank = [&](int r) {
      int rk = base;
#pragma unroll
      for (int v = 0; v < NW; ++v)
        if (v < (r >> 6)) rk += __popcll(s_bal[v]);
      return rk + __popcll(s_bal[r >> 6] & ((1ull << (r & 63)) - 1ull));
    };
    if (s0 + SUB < n) fetch(s0 + SUB);  // in flight during the writes below
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int idx = (k % (PER / 2)) * NT + tid, r = idx / CPR, c = idx % CPR;
      if (r < nr && kept(r)) {
        const int rk = rank(r);
        if (rk != s0 + r)
          __builtin_nontemporal_store(*(const v4u*)((k < PER / 2 ? sk : sv) + r * RB + c * 16),
                                      (v4u*)(prow(k < PER / 2 ? a.out_k : a.out_v, rk) + c * 16));
      }
    }
    if (tid < nr && kept(tid)) pos[rank(tid)] = s_pos[tid];
    if (summer) {
      const T* src = (const T*)(tensor ? sv : sk) + dim;
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        const int lo = v * 64;
        if (lo >= nr) break;
        unsigned long long ev = ~s_bal[v];
        if (nr - lo < 64) ev &= (1ull << (nr - lo)) - 1ull;
        while (ev) {
          const int r = lo + __ffsll((long long)ev) - 1;
          ev &= ev - 1ull;
          const int ch = s_pos[r] / a.C;
          if (ch != cur) {
            flush();
            cur = ch;
            acc = 0.f;
            cnt = 0;
            if (cur < a.chunk_stride) {
              old = sums[(int64_t)cur * D];
              if (tid == 0) oldc = cc[cur];
            }
          }
          acc += Elt<T>::load1(src + r * D);
          ++cnt;
        }
      }
    }
    base += total;
    __syncthreads();  // LDS is read before the next sub-tile is stored
  }
  if (summer) flush();
  if (tid == 0) a.out_count[bh] = base;
}

}  // namespace hk
