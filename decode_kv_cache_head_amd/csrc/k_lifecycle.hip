// Step (1) of the HARD-KV four-step pipeline (gist.science technical
// summary, section 2.A): linear append to the dense tier.  The dense tier
// is a ring of W slots per (b, h); the token that the new one displaces
// (position P - W) has aged out of the window and moves to the end of the
// sparse pool, whose positions therefore stay ascending.
#include "internal.h"

namespace hk {

template <typename T, int D>
__global__ __launch_bounds__(64) void k_append(AppendArgs a) {
  constexpr int RB = D * (int)sizeof(T);
  constexpr int CPR = RB / 16;
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int64_t bh = (int64_t)b * a.hkv + h;
  const int P = a.seq_len[b];
  if (P < a.W || a.W <= 0) return;
  const int cnt = a.pool_count[bh];
  // the aged token must fit the pool and the chunk capacity (P < ctx_cap)
  const bool room = cnt >= 0 && cnt < a.sparse_cap && P < a.ctx_cap;
  const int slot = P % a.W;
  for (int i = tid; i < 2 * CPR; i += 64) {
    const int tsr = i / CPR, c = i % CPR;
    char* ring = (tsr ? a.ring_v : a.ring_k) + (bh * a.W + slot) * RB + c * 16;
    const v4u old = *(const v4u*)ring;
    if (room) *(v4u*)((tsr ? a.pool_v : a.pool_k) + (bh * a.sparse_cap + cnt) * RB + c * 16) = old;
    *(v4u*)ring = *(const v4u*)((const char*)(tsr ? a.v_new : a.k_new) + bh * RB + c * 16);
  }
  if (tid == 0 && room) {
    a.pool_pos[bh * a.sparse_cap + cnt] = P - a.W;
    a.pool_count[bh] = cnt + 1;
  }
}

__global__ void k_advance(int32_t* seq_len, int B) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < B) seq_len[i] += 1;
}

template <typename T, int D, int G_unused>
static void launch_append_t(const AppendArgs& a, hipStream_t st) {
  observe("k_append", st);
  hipLaunchKernelGGL((k_append<T, D>), dim3(a.hkv, a.B), dim3(64), 0, st, a);
}

void launch_append(const AppendArgs& a, hipStream_t st) {
  HK_DISPATCH(a.dtype, a.D, 1, launch_append_t, a, st);
}

void launch_advance(int32_t* seq_len, int B, hipStream_t st) {
  observe("k_advance", st);
  hipLaunchKernelGGL(k_advance, dim3(ceil_div(B, 256)), dim3(256), 0, st, seq_len, B);
}

}  // namespace hk
