// Step (1) of the HARD-KV four-step pipeline (gist.science technical
// summary, section 2.A): linear append to the dense tier.  The dense tier
// is a ring of W slots per (b, h); the token that the new one displaces
// (position P - W) has aged out of the window and moves to the end of the
// sparse pool, whose positions therefore stay ascending.
//
// Head-wise block manager (section 2.C: a head-wise block manager for
// head-adaptive budgets under static shapes): with it, a head's pool rows
// live in blocks of a shared pool, found through the head's block table.
// k_pool_grow hands out blocks before the append, k_pool_shrink takes back
// the blocks a compaction emptied; both run as one workgroup with prefix
// scans in (b, h) order, so the allocation is deterministic.
#include "internal.h"

namespace hk {

// Pool row r of head bh: its region slot, or row r % bs of its table's
// block r / bs under the block manager (nullptr when that block is missing).
__device__ inline char* pool_row(const AppendArgs& a, char* base, int64_t bh, int r, int rb) {
  if (!a.pg.table) return base + (bh * a.sparse_cap + r) * rb;
  const int blk = a.pg.table[bh * a.pg.maxb + (r >> a.pg.lbs)];
  if (blk < 0 || blk >= a.pg.nblocks) return nullptr;
  return base + (((int64_t)blk << a.pg.lbs) + (r & ((1 << a.pg.lbs) - 1))) * rb;
}

template <typename T, int D>
__global__ __launch_bounds__(64) void k_append(AppendArgs a) {
  constexpr int RB = D * (int)sizeof(T);
  constexpr int CPR = RB / 16;
  static_assert(2 * CPR <= 64, "one 16-byte piece per thread");
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int64_t bh = (int64_t)b * a.hkv + h;
  if (a.q64) {
    // the score's float64 queries: this head's GQA group, 16-byte pieces
    constexpr int EPC = Elt<T>::kPer16;
    const int G = a.hq / a.hkv;
    const int64_t q0 = ((int64_t)b * a.hq + (int64_t)h * G) * D;
    for (int p = tid; p < G * D / EPC; p += 64) {
      float f[EPC];
      Elt<T>::unpack(*(const v4u*)((const T*)a.q + q0 + p * EPC), f);
#pragma unroll
      for (int e = 0; e < EPC; ++e) a.q64[q0 + p * EPC + e] = (double)f[e];
    }
  }
  const int P = a.seq_len[b];
  if (P < a.W || a.W <= 0) return;
  const int cnt = a.pool_count[bh];
  // the aged token must fit the pool and the chunk capacity (P < ctx_cap)
  const bool room = cnt >= 0 && cnt < a.sparse_cap && P < a.ctx_cap;
  char* dk = room ? pool_row(a, a.pool_k, bh, cnt, RB) : nullptr;
  char* dv = room ? pool_row(a, a.pool_v, bh, cnt, RB) : nullptr;
  // block manager out of blocks: the token goes straight into its chunk
  const bool to_chunk = room && dk == nullptr;
  const int slot = P % a.W;
  char* rk = a.ring_k + (bh * a.W + slot) * RB;
  char* rv = a.ring_v + (bh * a.W + slot) * RB;
  const int tsr = tid / CPR, c = tid % CPR;
  const bool mine = tid < 2 * CPR;
  v4u old{};
  if (mine) old = *(const v4u*)((tsr ? rv : rk) + c * 16);
  if (to_chunk) {
    const int ch = (P - a.W) / a.C;  // < chunk_cap because P < ctx_cap
    for (int i = tid; i < 2 * D; i += 64) {
      const int ts = i / D, dim = i % D;
      float* dst = (ts ? a.vsum : a.ksum) + (bh * a.chunk_cap + ch) * D + dim;
      *dst += Elt<T>::load1((const T*)(ts ? rv : rk) + dim);
    }
    if (tid == 0) a.ccount[bh * a.chunk_cap + ch] += 1;
  }
  __syncthreads();  // every read of the old ring row is done
  if (mine) {
    if (dk) *(v4u*)((tsr ? dv : dk) + c * 16) = old;
    *(v4u*)((tsr ? rv : rk) + c * 16) =
        *(const v4u*)((const char*)(tsr ? a.v_new : a.k_new) + bh * RB + c * 16);
  }
  if (tid == 0 && dk) {
    a.pool_pos[bh * a.sparse_cap + cnt] = P - a.W;
    a.pool_count[bh] = cnt + 1;
  }
}

// Exclusive scan of v over a 1024-thread workgroup; total = sum of all v.
__device__ inline int scan_1024(int v, int* sh, int& total) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (l >= o) incl += u;
  }
  if (l == 63) sh[w] = incl;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int x = sh[i];
    if (i < w) before += x;
    total += x;
  }
  __syncthreads();  // sh is free again
  return before + incl - v;
}

// Block manager, before the append: every head whose append row starts a
// block it does not hold requests one; requests are served in (b, h) order
// from the top of the free stack while it lasts.  One workgroup.
__global__ __launch_bounds__(1024) void k_pool_grow(AppendArgs a) {
  __shared__ int sh[16];
  __shared__ int s_top, s_served;
  const int tid = threadIdx.x, nh = a.B * a.hkv;
  const PoolPaging& pg = a.pg;
  if (tid == 0) {
    const int t = *pg.free_top;
    s_top = t < 0 ? 0 : (t > pg.nblocks ? pg.nblocks : t);
    s_served = 0;
  }
  __syncthreads();
  for (int h0 = 0; h0 < nh; h0 += 1024) {
    const int bh = h0 + tid;
    int want = 0;
    int64_t idx = 0;
    if (bh < nh) {
      const int P = a.seq_len[bh / a.hkv];
      const int cnt = a.pool_count[bh];
      const bool room = a.W > 0 && P >= a.W && cnt >= 0 && cnt < a.sparse_cap && P < a.ctx_cap;
      if (room && (cnt & ((1 << pg.lbs) - 1)) == 0) {
        idx = (int64_t)bh * pg.maxb + (cnt >> pg.lbs);
        want = pg.table[idx] < 0;
      }
    }
    int total;
    const int rank = scan_1024(want, sh, total);
    const int k = s_served + rank;
    if (want && k < s_top) pg.table[idx] = pg.free_ids[s_top - 1 - k];
    __syncthreads();
    if (tid == 0) s_served += total;
    __syncthreads();
  }
  if (tid == 0) *pg.free_top = s_top - (s_served < s_top ? s_served : s_top);
}

// Block manager, after the compaction: every head returns the blocks past
// ceil(count / bs), in (b, h) order and ascending table index.  One workgroup.
__global__ __launch_bounds__(1024) void k_pool_shrink(PoolPaging pg, const int32_t* count, int nh) {
  __shared__ int sh[16];
  __shared__ int s_top, s_pushed;
  const int tid = threadIdx.x;
  if (tid == 0) {
    const int t = *pg.free_top;
    s_top = t < 0 ? 0 : (t > pg.nblocks ? pg.nblocks : t);
    s_pushed = 0;
  }
  __syncthreads();
  for (int h0 = 0; h0 < nh; h0 += 1024) {
    const int bh = h0 + tid;
    int keep = 0, nrel = 0;
    int32_t* tab = pg.table + (int64_t)(bh < nh ? bh : 0) * pg.maxb;
    if (bh < nh) {
      int c = count[bh];
      c = c < 0 ? 0 : c;
      keep = (int)(((int64_t)c + (1 << pg.lbs) - 1) >> pg.lbs);
      // held blocks past `keep`: eight independent loads per round
      for (int i = keep; i < pg.maxb; i += 8) {
        int e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) e[j] = i + j < pg.maxb ? tab[i + j] : -1;
        int run = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (run == j && e[j] >= 0) ++run;
        nrel += run;
        if (run < 8) break;
      }
    }
    int total;
    const int rank = scan_1024(nrel, sh, total);
    // eight independent loads per round, then their stores
    for (int j0 = 0; j0 < nrel; j0 += 8) {
      int e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = j0 + j < nrel ? tab[keep + j0 + j] : -1;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j0 + j >= nrel) break;
        const int at = s_top + s_pushed + rank + j0 + j;
        if (at < pg.nblocks) pg.free_ids[at] = e[j];
        tab[keep + j0 + j] = -1;
      }
    }
    __syncthreads();
    if (tid == 0) s_pushed += total;
    __syncthreads();
  }
  if (tid == 0) {
    const int t = s_top + s_pushed;
    *pg.free_top = t > pg.nblocks ? pg.nblocks : t;
  }
}

template <typename T, int D, int G_unused>
static void launch_append_t(const AppendArgs& a, hipStream_t st) {
  observe("k_append", st);
  hipLaunchKernelGGL((k_append<T, D>), dim3(a.hkv, a.B), dim3(64), 0, st, a);
}

void launch_append(const AppendArgs& a, hipStream_t st) {
  HK_DISPATCH(a.dtype, a.D, 1, launch_append_t, a, st);
}

void launch_pool_grow(const AppendArgs& a, hipStream_t st) {
  observe("k_pool_grow", st);
  hipLaunchKernelGGL(k_pool_grow, dim3(1), dim3(1024), 0, st, a);
}

void launch_pool_shrink(const PoolPaging& pg, const int32_t* count, int n_heads, hipStream_t st) {
  observe("k_pool_shrink", st);
  hipLaunchKernelGGL(k_pool_shrink, dim3(1), dim3(1024), 0, st, pg, count, n_heads);
}

}  // namespace hk
