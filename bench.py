"""Decode-step benchmark of the HARD-KV hot path on one MI355X.

One step = one pass of the whole path over one batch: score -> calibrate ->
top-p select -> compact (rewrite + condense) -> three-tier attention, for
every (sequence, KV head) of one layer.  Default workload: Qwen3-8B attention
shape (32 query heads, 8 KV heads, head_dim 128), batch 32, 16384-token
contexts in a paged bf16 cache (16-token blocks), dense window 256, chunk 64,
top-p 0.95.  Inputs are synthetic N(0, 1) and resident in HBM before timing.

Prints one JSON line (rank 0).  The timed region runs the five ABI calls of
the path back to back on one stream with HIP events between them, so every
stage's average duration is measured live; the fused hardkv_step over the
same inputs is timed separately and reported next to it.
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
KERNEL_OF_STAGE = {"score": "k_score", "calibrate": "k_calibrate", "select": "k_select",
                   "compact": "k_compact", "attn": "k_attn"}
STAGE_SOURCES = {"score": "k_score.hip", "calibrate": "k_select.hip", "select": "k_select.hip",
                 "compact": "k_compact.hip", "attn": "k_attn.hip"}


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
    return ap.parse_args()


def algorithmic_bytes(w, A, k, stage):
    """Bytes the method must move per step (sums over every (b, h)).

    A[b, h]: aged candidates, k[b, h]: kept tokens (numpy int arrays).
    row = d * element size.  Per (b, h):
      score     A*row (keys) + 4A (logits)            [+ 4A norms on L2 heads]
      calibrate 4A (read scores)                      [+ 4A on L2 heads]
      select    4A (read scores) + A (mask)           [+ 4A on L2 heads]
      compact   2A*row (K, V) + A (mask) + 2k*row + 4k (rows, positions)
                + nch*(8d + 4) (chunk sums and counts)
      attn      2(k + W')*row + nch*(8d + 4), W' = dense rows
    plus q (and o for attention) once per query head.
    """
    import numpy as np
    d = w.d
    es = 4 if w.dtype == 0 else 2
    row = d * es
    l2 = np.array([m == 1 for m in w.metrics])[None, :]
    T = np.array(w.T)[:, None]
    nch = -(-A // w.C)
    dense = np.minimum(T, w.W) + 0 * A
    q_bytes = w.B * w.Hq * d * es
    if stage == "score":
        return int((A * row + 4 * A + 4 * A * l2).sum() + q_bytes)
    if stage == "calibrate":
        return int((4 * A + 4 * A * l2).sum())
    if stage == "select":
        return int((4 * A + A + 4 * A * l2).sum())
    if stage == "compact":
        return int((2 * A * row + A + 2 * k * row + 4 * k + nch * (8 * d + 4)).sum())
    if stage == "attn":
        return int((2 * (k + dense) * row + nch * (8 * d + 4)).sum() + q_bytes + w.B * w.Hq * d * 4)
    raise KeyError(stage)


def source_hash(stage):
    h = hashlib.sha256()
    for f in (STAGE_SOURCES[stage], "common.h", "internal.h"):
        h.update(open(os.path.join(ROOT, "decode_kv_cache_head_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile(stage, workload):
    """HBM bytes per launch from committed counter runs, if they were taken on
    the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_{KERNEL_OF_STAGE[stage]}_{workload}.json")
    if not os.path.exists(p):
        return None
    t = json.load(open(p))
    if t.get("source_hash") != source_hash(stage):
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
    cap = desc.sparse_cap
    logit = torch.empty((w.B, w.Hkv, cap), device=dev)
    l2 = torch.empty((w.B, w.Hkv, cap), device=dev)
    stats = torch.empty((w.B, w.Hkv, 4), dtype=torch.float64, device=dev)
    mask = torch.empty((w.B, w.Hkv, cap), dtype=torch.uint8, device=dev)
    count = torch.empty((w.B, w.Hkv), dtype=torch.int32, device=dev)
    tiers = H.alloc_tiers(desc, dev)
    out = torch.empty((w.B, w.Hq, w.d), device=dev)
    stream = torch.cuda.current_stream()

    stages = ["score", "calibrate", "select", "compact", "attn"]

    def one_pass(ev=None):
        if ev:
            ev[0].record(stream)
        H.score(desc, case.q, cache, case.metric, logit, l2, ws)
        if ev:
            ev[1].record(stream)
        H.calibrate(desc, case.ctx_len, case.metric, logit, l2, stats, ws)
        if ev:
            ev[2].record(stream)
        H.topp_select(desc, case.ctx_len, case.metric, logit, l2, stats, mask, count, ws)
        if ev:
            ev[3].record(stream)
        H.compact(desc, cache, mask, tiers, ws)
        if ev:
            ev[4].record(stream)
        H.decode_attn(desc, case.q, cache, tiers, out, ws)
        if ev:
            ev[5].record(stream)

    for _ in range(args.warmup):
        one_pass()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_pass(evs[i])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    stage_ms = {s: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)]))
                for j, s in enumerate(stages)}
    ms_per_step = float(np.mean([evs[i][0].elapsed_time(evs[i][5]) for i in range(args.steps)]))
    print(f"[bench] staged step {ms_per_step:.3f} ms (wall {wall * 1e3:.3f} ms) {stage_ms}",
          file=sys.stderr, flush=True)

    # the fused entry point over the same inputs
    for _ in range(args.warmup):
        H.step(desc, case.q, cache, case.metric, tiers, out, ws)
    torch.cuda.synchronize()
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record(stream)
    for _ in range(args.steps):
        H.step(desc, case.q, cache, case.metric, tiers, out, ws)
    f1.record(stream)
    torch.cuda.synchronize()
    fused_ms = f0.elapsed_time(f1) / args.steps

    if args.copy_calib:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # reference: a plain device-to-device copy of 2 GiB (read + write), the
    # bandwidth a streaming kernel can reach on this machine
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
    alg = {s: algorithmic_bytes(w, A, k, s) for s in stages}
    gbs = {s: alg[s] / (stage_ms[s] * 1e-3) / 1e9 for s in stages}
    dom = max(stages, key=lambda s: stage_ms[s])
    traffic = traffic_from_profile(dom, w.name)
    roof = {"bound": "hbm", "kernel": KERNEL_OF_STAGE[dom],
            "achieved": round(gbs[dom], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs[dom] / HBM_PEAK_GBS, 4),
            "traffic": traffic, "algorithmic_bytes": alg[dom],
            "avg_launch_ms": round(stage_ms[dom], 4)}
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
        "stage_ms": {s: round(v, 4) for s, v in stage_ms.items()},
        "stage_hbm_gbs": {s: round(v, 1) for s, v in gbs.items()},
        "stage_peak_frac": {s: round(v / HBM_PEAK_GBS, 4) for s, v in gbs.items()},
        "fused_step_ms": round(fused_ms, 4),
        "device_copy_gbs": round(copy_gbs, 1),
        "fused_tokens_s": round(w.B / (fused_ms * 1e-3), 1),
        "kept_fraction": round(float(k.sum() / max(A.sum(), 1)), 4),
        "dtype_note": "bf16 q/K/V in HBM; float64 score accumulation, 2^-47 fixed-point "
                      "top-p masses, float32 attention",
    }
    if not args.no_cpu:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(case, w, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
