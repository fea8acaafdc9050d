"""Decode-step benchmark of the HARD-KV hot path on one MI355X.

One step = one pass of the whole path over one batch: score -> calibrate ->
top-p select -> compact (rewrite + condense, with attention over the kept
rows folded in) -> dense/condensed attention -> merge, for every (sequence,
KV head) of one layer, through the C ABI's hardkv_step.  Default workload:
Qwen3-8B attention shape (32 query heads, 8 KV heads, head_dim 128), batch
32, 16384-token contexts in a paged bf16 cache (16-token blocks), dense
window 256, chunk 64, top-p 0.95.  Inputs are synthetic N(0, 1) and resident
in HBM before timing.

Prints one JSON line.  In the timed region the library's launch observer
records a HIP event on the launch stream before every kernel, so each
kernel's average duration is measured live; the same loop without the
observer is timed as a cross-check.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/s + HBM GB/s (% of peak), Qwen3-8B shape, 16k ctx, batch 32"
HBM_PEAK_GBS = 8000.0
QWEN3_8B_LAYERS = 36   # decoder layers of the public Qwen3-8B / Qwen3-32B models
QWEN3_32B_LAYERS = 64
KERNEL_SOURCES = {"k_prep": "k_score.hip", "k_score": "k_score.hip",
                  "k_calibrate": "k_select.hip", "k_select": "k_select.hip",
                  "k_calsel": "k_select.hip",
                  "k_compact_attn": "k_compact.hip", "k_compact_fast": "k_compact.hip",
                  "k_compact": "k_compact.hip", "k_attn": "k_attn.hip",
                  "k_attn_merge": "k_attn.hip"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen8b_b32_16k_paged")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--block-size", type=int, default=None,
                    help="override the cache layout (0 = contiguous)")
    ap.add_argument("--no-amortization", action="store_true",
                    help="skip the selection-reuse timings")
    return ap.parse_args()


def kernel_bytes(w, A, k, kernel, fused):
    """Bytes the method must move per launch (sums over every (b, h)).

    A[b, h]: aged candidates, k[b, h]: kept tokens (numpy int arrays);
    row = d * element size, nch = ceil(A / C), W' = dense rows.  Per (b, h):
      k_prep         q widened to float64                [+ A*row, key-dissimilarity heads]
      k_score        A*row (keys) + 4A (logits)         [+ 4A second metric, other heads]
      k_calibrate    4A (scores)                         [+ 4A]
      k_select       4A (scores) + A (mask)              [+ 4A]
      k_calsel       4A (scores) + A (mask)              [+ 4A] (both in one)
      k_compact*     2A*row (K, V) + A (mask) + 2k*row + 4k (rows, positions)
                     + nch*(8d + 4) (chunk sums, counts)
      k_attn         fused: 2W'*row + nch*(8d + 4); unfused: + 2k*row
    plus q once per query head (score, attention) and o (attention).
    """
    import numpy as np
    d = w.d
    es = 4 if w.dtype == 0 else 2
    row = d * es
    l2 = np.array([m != 0 for m in w.metrics])[None, :]
    kd = np.array([m == 3 for m in w.metrics])[None, :]
    T = np.array(w.T)[:, None]
    nch = -(-A // w.C)
    dense = np.minimum(T, w.W) + 0 * A
    q_bytes = w.B * w.Hq * d * es
    o_bytes = w.B * w.Hq * d * 4
    if kernel == "k_prep":
        return int(q_bytes + w.B * w.Hq * d * 8 + (A * row * kd).sum())
    if kernel == "k_score":
        return int((A * row + 4 * A + 4 * A * l2).sum() + w.B * w.Hq * d * 8)
    if kernel == "k_calibrate":
        return int((4 * A + 4 * A * l2).sum())
    if kernel == "k_select":
        return int((4 * A + A + 4 * A * l2).sum())
    if kernel == "k_calsel":
        return int((4 * A + A + 4 * A * l2).sum())
    if kernel in ("k_compact", "k_compact_fast", "k_compact_attn"):
        extra = q_bytes if kernel == "k_compact_attn" else 0
        return int((2 * A * row + A + 2 * k * row + 4 * k + nch * (8 * d + 4)).sum() + extra)
    if kernel == "k_attn":
        sparse = 0 if fused else 2 * k * row
        return int((2 * dense * row + sparse + nch * (8 * d + 4)).sum() + q_bytes)
    if kernel == "k_attn_merge":
        return o_bytes
    return 0


def source_hash(kernel):
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES[kernel], "common.h", "internal.h"):
        h.update(open(os.path.join(ROOT, "decode_kv_cache_head_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel, workload):
    """HBM bytes per launch from committed counter runs, if they were taken on
    the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(p):
        return None
    t = json.load(open(p))
    if t.get("source_hash") != source_hash(kernel):
        return None
    return int(t["fetch_bytes"] * t["fetch_scale"] + t["write_bytes"] * t["write_scale"])


def cpu_baseline(case, w, seconds):
    """The CPU oracle (one BLAS thread) on the same workload: whole passes
    over every (sequence, KV head) until about `seconds` of oracle time."""
    import numpy as np
    import oracle as O
    from decode_kv_cache_head_amd import synth as S
    from threadpoolctl import threadpool_limits

    G = w.G
    heads = []
    for b in range(w.B):
        for h in range(w.Hkv):
            q = case.q[b, h * G:(h + 1) * G].float().cpu().numpy().astype(np.float64)
            heads.append((b, h, q))
    spent, passes, done = 0.0, 0, 0
    with threadpool_limits(limits=1):
        while True:
            for b, h, q in heads:
                K = S.head_rows(case, b, h, "k").float().cpu().numpy()
                V = S.head_rows(case, b, h, "v").float().cpu().numpy()
                t0 = time.perf_counter()
                O.step_head(q, K, V, w.T[b], w.W, w.C, w.p, int(w.metrics[h]))
                spent += time.perf_counter() - t0
                done += 1
                if passes and spent >= seconds:
                    break
            else:
                passes += 1
                if spent >= seconds:
                    break
                continue
            break
    step_s = spent / done * len(heads)
    return {"value": round(w.B / step_s, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} (sequence, KV head) oracle steps = {done / len(heads):.2f} passes "
                      f"over all {len(heads)} heads of the same workload, {spent:.1f} s of "
                      f"single-thread oracle time; input copies to host not timed",
            "ms_per_step": round(step_s * 1e3, 1)}


def time_ms(fn, steps, warmup=2):
    import torch
    for _ in range(warmup):
        fn()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(steps):
        fn()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def amortization(w, case, steps, horizons=(1, 2, 4, 8, 16, 32)):
    """Serving one selection over several decode steps (section 2.C,
    "Trade-off Management"; section 4, "Scalability": the rewrite's cost is
    amortized within a few steps).  Times, per step of one layer:
      select  hardkv_step (every head rewritten) / hardkv_step_policy with
              every head sparse-loaded;
      reuse   hardkv_decode_attn over those tiers (window W: the cost of a
              reuse step up to one more dense row per step since the selection);
      dense   hardkv_decode_attn over the whole context with no selection
              (window = context), the uncompressed reference;
    and the average step time over a horizon of N steps (one selection, N - 1
    reuses), the first N where it beats dense attention, and how many heads
    the memory-time-integral policy sends to each mode."""
    import numpy as np
    import torch
    from decode_kv_cache_head_amd import hardkv as H
    dev = case.q.device
    desc = H.make_desc(w.B, w.Hq, w.Hkv, w.d, w.dtype, w.W, w.C, w.p, case.ctx_cap,
                       w.block_size, case.max_blocks)
    ws = H.alloc_workspace(desc, dev)
    cache = H.cache_struct(case.k, case.v, case.ctx_len, case.block_table)
    out = torch.empty((w.B, w.Hq, w.d), device=dev)
    t_rw = H.alloc_tiers(desc, dev, mode=True)
    t_sp = H.alloc_tiers(desc, dev, mode=True)
    sparse = H.policy(H.POLICY_SPARSE)
    sel_rw = time_ms(lambda: H.step(desc, case.q, cache, case.metric, t_rw, out, ws), steps)
    sel_sp = time_ms(lambda: H.step_policy(desc, sparse, case.q, cache, case.metric, t_sp, out,
                                           ws), steps)
    reuse_rw = time_ms(lambda: H.decode_attn(desc, case.q, cache, t_rw, out, ws), steps)
    reuse_sp = time_ms(lambda: H.decode_attn(desc, case.q, cache, t_sp, out, ws), steps)
    d_dense = H.make_desc(w.B, w.Hq, w.Hkv, w.d, w.dtype, case.ctx_cap, w.C, w.p, case.ctx_cap,
                          w.block_size, case.max_blocks, desc.sparse_cap, desc.chunk_cap)
    ws_dense = H.alloc_workspace(d_dense, dev)
    t_none = H.Tiers(t_rw.k, t_rw.v, t_rw.pos, torch.zeros_like(t_rw.count), t_rw.ksum,
                     t_rw.vsum, t_rw.ccount)
    dense = time_ms(lambda: H.decode_attn(d_dense, case.q, cache, t_none, out, ws_dense), steps)
    A = np.maximum(np.array(w.T) - w.W, 0)
    k = t_rw.count.cpu().numpy()
    # the reuse step is the attention launch alone (plus its merge): its
    # algorithmic bytes (rewritten rows, dense rows, chunks, q) per second
    reuse_bytes = kernel_bytes(w, np.repeat(A[:, None], w.Hkv, axis=1), k, "k_attn", False)

    def avg(sel, reuse, n):
        return (sel + (n - 1) * reuse) / n

    def breakeven(sel, reuse):
        if reuse >= dense:
            return None
        return int(math.floor((sel - dense) / (dense - reuse))) + 2 if sel > dense else 1

    # the packed rewritten tier (one region sized to the kept rows, Flatten
    # Index to the sum) against the per-head regions of the maximum length
    kept_rows = int(t_rw.count.sum().item())
    d_pack = H.make_desc(w.B, w.Hq, w.Hkv, w.d, w.dtype, w.W, w.C, w.p, case.ctx_cap,
                         w.block_size, case.max_blocks, packed_rows=max(kept_rows, 1))
    t_pack = H.alloc_tiers(d_pack, dev)
    sel_pack = time_ms(lambda: H.step(d_pack, case.q, cache, case.metric, t_pack, out, ws), steps)
    reuse_pack = time_ms(lambda: H.decode_attn(d_pack, case.q, cache, t_pack, out, ws), steps)
    row_bytes = w.d * (4 if w.dtype == 0 else 2)
    del t_pack
    mti = {}
    t_mti = H.alloc_tiers(desc, dev, mode=True)
    for n in horizons:
        H.step_policy(desc, H.policy(H.POLICY_MTI, n), case.q, cache, case.metric, t_mti, out, ws)
        torch.cuda.synchronize()
        mti[str(n)] = int(t_mti.mode.sum().item())
    return {
        "kept_fraction": round(float(k.sum() / max(int(A.sum()) * w.Hkv, 1)), 4),
        "median_kept_tokens": int(np.median(k)),
        "select_ms": {"rewrite": round(sel_rw, 4), "sparse": round(sel_sp, 4)},
        "reuse_ms": {"rewrite": round(reuse_rw, 4), "sparse": round(reuse_sp, 4)},
        "dense_attention_ms": round(dense, 4),
        "reuse_attention_hbm": {"algorithmic_gb": round(reuse_bytes / 1e9, 4),
                                "gbs": round(reuse_bytes / (reuse_rw * 1e-3) / 1e9, 1),
                                "frac_of_peak": round(reuse_bytes / (reuse_rw * 1e-3) / 1e9
                                                      / HBM_PEAK_GBS, 4)},
        "avg_step_ms": {str(n): {"rewrite": round(avg(sel_rw, reuse_rw, n), 4),
                                 "sparse": round(avg(sel_sp, reuse_sp, n), 4)}
                        for n in horizons},
        "breakeven_horizon_vs_dense": {"rewrite": breakeven(sel_rw, reuse_rw),
                                       "sparse": breakeven(sel_sp, reuse_sp)},
        "mti_sparse_heads_by_horizon": mti,
        "heads": int(w.B * w.Hkv),
        "packed_tier": {"select_ms": round(sel_pack, 4), "reuse_ms": round(reuse_pack, 4),
                        "kv_bytes": 2 * kept_rows * row_bytes,
                        "per_head_regions_kv_bytes": 2 * w.B * w.Hkv * desc.sparse_cap * row_bytes},
    }


def lifecycle(dev, reps=5, steady_steps=48, pool_block=0):
    """The multi-step lifecycle (hardkv_step_inplace) of one layer at the
    Qwen3-32B attention shape: 64 sequences, 64 query / 8 KV heads, d = 128,
    12288-token prefill, window 512, chunk 64, p = 0.95, fresh N(0, 1) query,
    key and value every step.  Step 1 re-selects over the whole aged pool
    (restored from a copy before each timed repetition); later steps run on
    the pool that the selections left.  pool_block > 0: the pool under the
    head-wise block manager (blocks of that many rows, as many blocks as the
    per-head regions would hold)."""
    import torch
    from decode_kv_cache_head_amd import hardkv as H
    B, Hq, Hkv, d, T0, W, C, p = 64, 64, 8, 128, 12288, 512, 64, 0.95
    steps_cap = 1 + steady_steps + 8 + 8  # step 1, steady steps, graph replays
    desc = H.make_desc(B, Hq, Hkv, d, H.BF16, W, C, p, T0 + steps_cap)
    A = T0 - W
    ws = H.alloc_workspace(desc, dev)
    out = torch.empty((B, Hq, d), device=dev)
    g = torch.Generator(device=dev).manual_seed(4242)
    k0 = torch.empty((B, Hkv, A, d), dtype=torch.bfloat16, device=dev)
    v0 = torch.empty_like(k0)
    for i in range(0, B, 8):
        k0[i:i + 8] = torch.randn((8, Hkv, A, d), generator=g, device=dev).to(torch.bfloat16)
        v0[i:i + 8] = torch.randn((8, Hkv, A, d), generator=g, device=dev).to(torch.bfloat16)
    ring_k = torch.randn((B, Hkv, W, d), generator=g, device=dev).to(torch.bfloat16)
    ring_v = torch.randn((B, Hkv, W, d), generator=g, device=dev).to(torch.bfloat16)
    r0k, r0v = ring_k.clone(), ring_v.clone()
    seq = torch.full((B,), T0, dtype=torch.int32, device=dev)
    if pool_block:
        maxb = -(-desc.sparse_cap // pool_block)
        st = H.paged_state(desc, k0, v0, ring_k, ring_v, seq, pool_block, B * Hkv * maxb)
        saved = [x.clone() for x in (st.pool_table, st.free_ids, st.free_top)]
        used = B * Hkv * (-(-A // pool_block))
        pk0, pv0 = st.tiers.k[:used].clone(), st.tiers.v[:used].clone()
    else:
        t = H.alloc_tiers(desc, dev)
        t.k[:, :, :A] = k0
        t.v[:, :, :A] = v0
        st = H.State(ring_k, ring_v, t, seq)
    t = st.tiers
    qs = [torch.randn((B, Hq, d), generator=g, device=dev).to(torch.bfloat16) for _ in range(4)]
    kn = torch.randn((B, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
    vn = torch.randn((B, Hkv, d), generator=g, device=dev).to(torch.bfloat16)

    def reset():
        if pool_block:
            t.k[:used].copy_(pk0)
            t.v[:used].copy_(pv0)
            for x, x0 in zip((st.pool_table, st.free_ids, st.free_top), saved):
                x.copy_(x0)
        else:
            t.k[:, :, :A].copy_(k0)
            t.v[:, :, :A].copy_(v0)
        t.pos[:, :, :A] = torch.arange(A, dtype=torch.int32, device=dev)
        t.count.fill_(A)
        t.ksum.zero_()
        t.vsum.zero_()
        t.ccount.zero_()
        ring_k.copy_(r0k)
        ring_v.copy_(r0v)
        seq.fill_(T0)

    def pool_mb():
        rows = st.blocks_held() * pool_block if pool_block else B * Hkv * desc.sparse_cap
        return round(rows * d * 2 * 2 / 2**20, 1)

    mb0 = pool_mb()
    s1 = []
    for r in range(reps + 1):
        reset()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        H.step_inplace(desc, qs[0], kn, vn, None, st, out, ws)
        e1.record()
        torch.cuda.synchronize()
        if r:
            s1.append(e0.elapsed_time(e1))
    pool1 = int(t.count.float().median().item())
    mb1 = pool_mb()
    for i in range(steady_steps - 8):
        H.step_inplace(desc, qs[i % 4], kn, vn, None, st, out, ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(8):
        H.step_inplace(desc, qs[i % 4], kn, vn, None, st, out, ws)
    e1.record()
    torch.cuda.synchronize()
    steady = e0.elapsed_time(e1) / 8
    pool_steady = int(t.count.float().median().item())
    mb_steady = pool_mb()
    # the same steady step captured once in a HIP graph and replayed
    qg = qs[0].clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        H.step_inplace(desc, qg, kn, vn, None, st, out, ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(8):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    steady_graph = e0.elapsed_time(e1) / 8
    del graph
    step1 = sum(s1) / len(s1)
    res = {"shape": "qwen3-32b attention, B=64, T0=12288, W=512, C=64, p=0.95, one layer",
           "pool_block": pool_block,
           "step1_ms": round(step1, 4), "step1_pool_median_after": pool1,
           "aged_pool_before_step1": A, "steady_ms": round(steady, 4),
           "steady_graph_replay_ms": round(steady_graph, 4),
           "steady_after_steps": steady_steps,
           "steady_pool_median": pool_steady,
           "pool_kv_mb": {"before": mb0, "after_step1": mb1, "steady": mb_steady},
           "step1_tokens_per_s": round(B / (step1 * 1e-3), 1),
           "steady_tokens_per_s": round(B / (steady * 1e-3), 1),
           # attention + compression only, every layer of the model, steady state
           "steady_model_tokens_per_s_attention_only": {
               "layers": QWEN3_32B_LAYERS,
               "value": round(B / (steady * 1e-3) / QWEN3_32B_LAYERS, 1)}}
    del t, st, k0, v0, ws
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the path shards by "
              "(sequence, KV head) with no exchange, which is described but not run here.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from decode_kv_cache_head_amd import hardkv as H
    from decode_kv_cache_head_amd import synth as S

    H.load()
    dev = torch.device("cuda:0")
    w = S.workload(args.workload)
    if args.block_size is not None:
        from dataclasses import replace
        w = replace(w, block_size=args.block_size)
    print(f"[bench] generating {w.name}", file=sys.stderr, flush=True)
    case = S.make_case(w, dev)
    desc = H.make_desc(w.B, w.Hq, w.Hkv, w.d, w.dtype, w.W, w.C, w.p, case.ctx_cap,
                       w.block_size, case.max_blocks)
    ws = H.alloc_workspace(desc, dev)
    cache = H.cache_struct(case.k, case.v, case.ctx_len, case.block_table)
    tiers = H.alloc_tiers(desc, dev)
    out = torch.empty((w.B, w.Hq, w.d), device=dev)
    stream = torch.cuda.current_stream()

    def step():
        H.step(desc, case.q, cache, case.metric, tiers, out, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: every kernel bracketed by events on the launch stream
    with H.KernelTimer() as kt:
        for _ in range(args.steps):
            kt.mark(stream)
            step()
        kt.mark(stream)
    torch.cuda.synchronize()
    marks = [i for i, (n, _) in enumerate(kt.events) if n is None]
    step_ms = [kt.events[a][1].elapsed_time(kt.events[b][1]) for a, b in zip(marks, marks[1:])]
    ms_per_step = float(np.mean(step_ms))
    per_kernel = {}
    for name, ms in kt.durations():
        per_kernel.setdefault(name, []).append(ms)
    kernel_ms = {n: float(np.mean(v)) for n, v in per_kernel.items()}
    launches = {n: len(v) // args.steps for n, v in per_kernel.items()}
    print(f"[bench] step {ms_per_step:.3f} ms {kernel_ms}", file=sys.stderr, flush=True)

    # the step captured once into a HIP graph and replayed (static shapes,
    # no host synchronisation or allocation inside the step)
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        graph.replay()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for _ in range(args.steps):
        graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    graph_ms = g0.elapsed_time(g1) / args.steps
    del graph

    # the same loop without the observer (cross-check of the step time)
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record(stream)
    for _ in range(args.steps):
        step()
    f1.record(stream)
    torch.cuda.synchronize()
    plain_ms = f0.elapsed_time(f1) / args.steps

    if args.copy_calib:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # reference: a plain device-to-device copy of 2 GiB (read + write)
    src = torch.empty(1 << 31, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * (1 << 31) * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst

    A = np.maximum(np.array(w.T)[:, None] - w.W, 0) * np.ones((1, w.Hkv), np.int64)
    k = tiers.count.cpu().numpy().astype(np.int64)
    fused = "k_compact_attn" in kernel_ms
    alg = {n: kernel_bytes(w, A, k, n, fused) for n in kernel_ms}
    gbs = {n: alg[n] / (kernel_ms[n] * 1e-3) / 1e9 for n in kernel_ms}
    dom = max(kernel_ms, key=lambda n: kernel_ms[n])
    traffic = traffic_from_profile(dom, w.name)
    roof = {"bound": "hbm", "kernel": dom,
            "achieved": round(gbs[dom], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs[dom] / HBM_PEAK_GBS, 4),
            "traffic": traffic, "algorithmic_bytes": alg[dom],
            "avg_launch_ms": round(kernel_ms[dom], 4)}
    step_bytes = sum(alg.values())
    tok_s = w.B / (ms_per_step * 1e-3)
    res = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "ctx": max(w.T), "q_heads": w.Hq,
                   "kv_heads": w.Hkv, "head_dim": w.d, "kv_dtype": "bf16" if w.dtype else "f32",
                   "layout": f"paged{w.block_size}" if w.block_size else "contiguous",
                   "dense_window": w.W, "chunk": w.C, "top_p": w.p, "layers": 1},
        "roofline": roof,
        "kernel_ms": {n: round(v, 4) for n, v in kernel_ms.items()},
        "kernel_launches_per_step": launches,
        "kernel_hbm_gbs": {n: round(v, 1) for n, v in gbs.items()},
        "kernel_peak_frac": {n: round(v / HBM_PEAK_GBS, 4) for n, v in gbs.items()},
        "step_algorithmic_gb": round(step_bytes / 1e9, 4),
        "step_hbm_gbs": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "step_ms_without_observer": round(plain_ms, 4),
        "graph_replay_ms_per_step": round(graph_ms, 4),
        "device_copy_gbs": round(copy_gbs, 1),
        "kept_fraction": round(float(k.sum() / max(A.sum(), 1)), 4),
        # attention + compression only, every layer of the model at this shape
        "model_tokens_per_s_attention_only": {
            "layers": QWEN3_8B_LAYERS, "value": round(tok_s / QWEN3_8B_LAYERS, 1)},
        "dtype_note": "bf16 q/K/V in HBM; float64 score accumulation, 2^-47 fixed-point "
                      "top-p masses, float32 attention",
    }
    if not args.no_amortization and args.block_size is None:
        # the step with attention sinks and / or attention-weighted merging
        var = {}
        for tag, kw in (("sinks4", dict(sinks=4)), ("weighted_merge", dict(merge=1)),
                        ("sinks4_weighted_merge", dict(sinks=4, merge=1))):
            dv = H.make_desc(w.B, w.Hq, w.Hkv, w.d, w.dtype, w.W, w.C, w.p, case.ctx_cap,
                             w.block_size, case.max_blocks, desc.sparse_cap, desc.chunk_cap,
                             **kw)
            wsv = H.alloc_workspace(dv, dev)
            var[tag] = round(time_ms(lambda: H.step(dv, case.q, cache, case.metric, tiers, out,
                                                    wsv), args.steps), 4)
        # every head on the observation-window metric: 4 queries, pooling radius 3
        dv = H.make_desc(w.B, w.Hq, w.Hkv, w.d, w.dtype, w.W, w.C, w.p, case.ctx_cap,
                         w.block_size, case.max_blocks, desc.sparse_cap, desc.chunk_cap,
                         obs_window=4, pool_radius=3)
        wsv = H.alloc_workspace(dv, dev)
        q_hist = torch.randn((w.B, 3, w.Hq, w.d), device=dev).to(case.q.dtype)
        cache_w = H.cache_struct(case.k, case.v, case.ctx_len, case.block_table, q_hist)
        metric_w = torch.full((w.Hkv,), H.METRIC_WINDOW, dtype=torch.int8, device=dev)
        var["window4_pool3"] = round(time_ms(lambda: H.step(dv, case.q, cache_w, metric_w, tiers,
                                                            out, wsv), args.steps), 4)
        # every head on the key norm, calibrated by the spread or the entropy rule
        metric_n = torch.full((w.Hkv,), H.METRIC_L2, dtype=torch.int8, device=dev)
        for tag, rule in (("keynorm_spread", H.CALIB_SPREAD), ("keynorm_entropy", H.CALIB_ENTROPY)):
            dv = H.make_desc(w.B, w.Hq, w.Hkv, w.d, w.dtype, w.W, w.C, w.p, case.ctx_cap,
                             w.block_size, case.max_blocks, desc.sparse_cap, desc.chunk_cap,
                             calibration=rule)
            wsv = H.alloc_workspace(dv, dev)
            var[tag] = round(time_ms(lambda: H.step(dv, case.q, cache, metric_n, tiers, out, wsv),
                                     args.steps), 4)
        # every head on the key-dissimilarity metric (one more pass for the key sums)
        metric_k = torch.full((w.Hkv,), H.METRIC_KEYDIFF, dtype=torch.int8, device=dev)
        var["keydiff_spread"] = round(time_ms(lambda: H.step(desc, case.q, cache, metric_k, tiers,
                                                             out, ws), args.steps), 4)
        res["variant_step_ms"] = var
    if not args.no_amortization:
        print("[bench] selection reuse", file=sys.stderr, flush=True)
        am = {w.name: amortization(w, case, args.steps)}
        if args.workload == "qwen8b_b32_16k_paged" and args.block_size is None:
            wp = S.workload("qwen8b_b32_16k_paged_peaked")
            am[wp.name] = amortization(wp, S.make_case(wp, dev), args.steps)
            torch.cuda.empty_cache()
        res["amortization"] = am
        print("[bench] lifecycle", file=sys.stderr, flush=True)
        res["lifecycle"] = lifecycle(dev)
        res["lifecycle_block_manager"] = lifecycle(dev, pool_block=64)
    if not args.no_cpu:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(case, w, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
