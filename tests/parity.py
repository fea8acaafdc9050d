"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare it with the CPU oracle head by head.

Comparison rules (written here, used by every GPU test):
  * scores: float32 logits / key norms equal; a 1-ulp difference is allowed
    on a tiny fraction of tokens (float64 sums in another order can round
    the other way at a float32 midpoint).
  * selected set: identical, except tokens that are borderline for the top-p
    cutoff: their exclusive prefix mass is within 1e-6 relative of p, or
    their weight is within 1e-6 relative of the weight of the last kept or
    first dropped token.  Every such token is counted and reported.
  * rewritten tier: slot count equals the oracle budget when the sets agree;
    positions and the K/V bit patterns of every slot equal the source rows.
  * condensed tier: counts exact, sums within 1e-5 * sum|x| (float32 on the
    GPU, float64 in the oracle); chunks that hold a mismatched token excused.
  * attention: per query row, max|o_gpu - o_ref| / max|o_ref| <= 2e-3, the
    oracle run on the GPU's own tiers when the sets differ.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
from decode_kv_cache_head_amd import hardkv as H
from decode_kv_cache_head_amd import synth as S

ATTN_TOL = 2e-3
SUM_TOL = 1e-5
BORDER = 1e-6


def desc_for(case: S.Case, top_p=None, sparse_cap=None, chunk_cap=None) -> H.Desc:
    w = case.w
    return H.make_desc(w.B, w.Hq, w.Hkv, w.d, w.dtype, w.W, w.C,
                       w.p if top_p is None else top_p, case.ctx_cap, w.block_size,
                       case.max_blocks, sparse_cap, chunk_cap, w.sinks, w.merge,
                       obs_window=w.obs_window, pool_radius=w.pool_radius,
                       calibration=w.calibration, select_block=w.select_block)


def cache_of(case: S.Case) -> H.Cache:
    return H.cache_struct(case.k, case.v, case.ctx_len, case.block_table, case.q_hist)


def run_stages(case: S.Case, desc: H.Desc):
    """Each ABI entry point on its own, in pipeline order."""
    w = case.w
    dev = case.q.device
    B, Hkv, cap = w.B, w.Hkv, desc.sparse_cap
    ws = H.alloc_workspace(desc, dev)
    cache = cache_of(case)
    logit = torch.full((B, Hkv, cap), float("nan"), device=dev)
    l2 = torch.full((B, Hkv, cap), float("nan"), device=dev)
    stats = torch.zeros((B, Hkv, 4), dtype=torch.float64, device=dev)
    mask = torch.full((B, Hkv, cap), 7, dtype=torch.uint8, device=dev)
    count = torch.full((B, Hkv), -1, dtype=torch.int32, device=dev)
    tiers = H.alloc_tiers(desc, dev)
    out = torch.full((B, w.Hq, w.d), float("nan"), device=dev)
    H.score(desc, case.q, cache, case.metric, logit, l2, ws)
    H.calibrate(desc, case.ctx_len, case.metric, logit, l2, stats, ws)
    H.topp_select(desc, case.ctx_len, case.metric, logit, l2, stats, mask, count, ws)
    H.compact_scored(desc, cache, case.metric, logit, l2, stats, mask, tiers, ws)
    H.decode_attn(desc, case.q, cache, tiers, out, ws)
    torch.cuda.synchronize()
    return dict(logit=logit, l2=l2, stats=stats, mask=mask, count=count, tiers=tiers, out=out)


def run_step(case: S.Case, desc: H.Desc, ws=None, tiers=None, out=None):
    w = case.w
    dev = case.q.device
    ws = H.alloc_workspace(desc, dev) if ws is None else ws
    tiers = H.alloc_tiers(desc, dev) if tiers is None else tiers
    out = torch.empty((w.B, w.Hq, w.d), device=dev) if out is None else out
    H.step(desc, case.q, cache_of(case), case.metric, tiers, out, ws)
    torch.cuda.synchronize()
    return dict(tiers=tiers, out=out)


def oracle_head(case: S.Case, b: int, h: int, p: float):
    w = case.w
    G = w.G
    q = case.q[b, h * G:(h + 1) * G].float().cpu().numpy().astype(np.float64)
    K = S.head_rows(case, b, h, "k").float().cpu().numpy()
    V = S.head_rows(case, b, h, "v").float().cpu().numpy()
    hist = None
    if case.q_hist is not None:
        hist = case.q_hist[b, :, h * G:(h + 1) * G].float().cpu().numpy().astype(np.float64)
    ref = O.step_head(q, K, V, w.T[b], w.W, w.C, p, int(w.metrics[h]), w.sinks, w.merge,
                      q_hist=hist, radius=w.pool_radius, calib=w.calibration,
                      select_block=w.select_block)
    return q, K, V, ref


def _ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    ia = a.astype(np.float32).view(np.int32).astype(np.int64)
    ib = b.astype(np.float32).view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


def borderline_tokens(ref: O.HeadResult, p: float, tokens) -> np.ndarray:
    """tokens: candidate indices (position - sinks)."""
    sel = ref.sel
    A = ref.A
    p32 = float(np.float32(p))
    rank = np.empty(A, np.int64)
    rank[sel.order] = np.arange(A)
    w = ref.cal.w
    cuts = [w[sel.order[sel.k - 1]]] if sel.k >= 1 else []
    if sel.k < A:
        cuts.append(w[sel.order[sel.k]])
    ok = []
    for t in tokens:
        i = rank[t]
        mass = abs(sel.prefix_excl[i] - p32) <= BORDER * p32
        order = any(abs(w[t] - c) <= BORDER * c for c in cuts)
        ok.append(mass or order)
    return np.array(ok, bool)


def borderline_blocks(ref: O.HeadResult, p: float, tokens) -> np.ndarray:
    """Block-granular selection: tokens (candidate indices) whose block is
    borderline for the cutoff: its exclusive prefix mass in block rank order
    within 1e-6 relative of p, or its mass within 1e-6 relative of the last
    kept or first dropped block's."""
    bsel = ref.extra["blocks"]
    p32 = float(np.float32(p))
    bs_ids = ref.sinks + np.asarray(tokens, np.int64)
    rank = np.empty(len(bsel.blocks), np.int64)
    rank[bsel.order] = np.arange(len(bsel.blocks))
    cuts = []
    if bsel.k >= 1:
        cuts.append(bsel.mass[bsel.order[bsel.k - 1]])
    if bsel.k < len(bsel.blocks):
        cuts.append(bsel.mass[bsel.order[bsel.k]])
    ok = []
    for pos in bs_ids:
        j = int(np.searchsorted(bsel.blocks, pos // ref.extra["block_size"]))
        i = rank[j]
        mass = abs(bsel.prefix_excl[i] - p32) <= BORDER * p32
        order = any(abs(bsel.mass[j] - c) <= BORDER * c for c in cuts)
        ok.append(mass or order)
    return np.array(ok, bool)


def check_head(case, b, h, gpu, p, report, stages=True, desc=None, skip_slots=False):
    """Compare every stage of (b, h) with the oracle; returns mismatch count.
    skip_slots: the head is sparse-loaded, its k / v slots hold no rows."""
    w = case.w
    q, K, V, ref = oracle_head(case, b, h, p)
    A = ref.A
    s0 = ref.sinks  # sink count: candidate index i is position s0 + i
    G, d = w.G, w.d
    is_l2 = int(w.metrics[h]) != O.METRIC_QK  # the second score array holds the metric
    if stages:
        lg = gpu["logit"][b, h, :A].cpu().numpy()
        u = _ulp_diff(lg, ref.ell)
        assert u.max(initial=0) <= 1, f"logit off by {u.max()} ulp at ({b},{h})"
        report["logit_1ulp"] += int((u == 1).sum())
        if is_l2:
            u2 = _ulp_diff(gpu["l2"][b, h, :A].cpu().numpy(), ref.s)
            assert u2.max(initial=0) <= 1
            report["l2_1ulp"] += int((u2 == 1).sum())
        st = gpu["stats"][b, h].cpu().numpy()
        if A:
            assert st[2] == ref.cal.m or (u.max(initial=0) > 0 or is_l2)
            assert abs(st[0] - ref.cal.shift) <= 1e-12 * max(1.0, abs(ref.cal.shift))
            assert abs(st[1] - ref.cal.scale) <= 1e-12 * max(1.0, abs(ref.cal.scale))
            assert abs(st[3] - ref.cal.Z) <= 1e-12 * ref.cal.Z
        gm = gpu["mask"][b, h, :A].cpu().numpy()
        assert set(np.unique(gm).tolist()) <= {0, 1}
        assert int(gpu["count"][b, h]) == int(gm.sum())
    tiers = gpu["tiers"]
    k_gpu = int(tiers.count[b, h])
    pos_gpu = tiers.pos[b, h, :k_gpu].cpu().numpy().astype(np.int64)
    assert np.all(np.diff(pos_gpu) > 0) and (k_gpu == 0 or (pos_gpu[0] >= s0 and pos_gpu[-1] < s0 + A))
    if stages:
        assert np.array_equal(pos_gpu, s0 + np.nonzero(gm)[0])
    diff = np.setxor1d(pos_gpu, ref.pos)
    if w.select_block:
        # whole blocks on the GPU too
        kept_blocks = np.unique(pos_gpu // w.select_block)
        cand = s0 + np.arange(A)
        assert np.array_equal(pos_gpu, cand[np.isin(cand // w.select_block, kept_blocks)])
    if diff.size:
        bl = (borderline_blocks(ref, p, diff - s0) if w.select_block else
              borderline_tokens(ref, p, diff - s0))
        assert bl.all(), f"non-borderline set mismatch at ({b},{h}): {diff[~bl][:10]}"
        report["borderline"] += int(diff.size)
    else:
        assert k_gpu == ref.sel.k
    report["selected"] += k_gpu
    report["candidates"] += A
    # rewritten rows are bit copies of the source rows (a sparse-loaded head
    # has no rows in its slots)
    if skip_slots:
        report["sparse_heads"] += 1
    else:
        kt = tiers.slots(b, h, "k")
        vt = tiers.slots(b, h, "v")
        idx = torch.as_tensor(pos_gpu, device=kt.device).long()
        src_k = S.head_rows(case, b, h, "k")[idx]
        src_v = S.head_rows(case, b, h, "v")[idx]
        bits = torch.int16 if kt.dtype == torch.bfloat16 else torch.int32
        assert torch.equal(kt.view(bits), src_k.view(bits))
        assert torch.equal(vt.view(bits), src_v.view(bits))
    # condensed tier
    nch = -(-A // w.C) if A else 0
    cc = tiers.ccount[b, h, :nch].cpu().numpy()
    ks = tiers.ksum[b, h, :nch].double().cpu().numpy()
    vs = tiers.vsum[b, h, :nch].double().cpu().numpy()
    evicted_gpu = np.setdiff1d(s0 + np.arange(A), pos_gpu)
    wts = None
    if w.merge == O.MERGE_WEIGHTED:
        wts = O.merge_weights(ref.cal.c[evicted_gpu - s0], ref.cal.m)
    allpos = np.arange(w.T[b])
    if diff.size:
        ek, ev, ec = O.condense(K, V, evicted_gpu, allpos, w.C, nch, wts, origin=s0)
    else:
        ek, ev, ec = ref.ksum, ref.vsum, ref.cnt
    assert np.array_equal(cc, ec)
    # bound: SUM_TOL times the same merge of |x| (n * weighted mean of |x|)
    ak, av = _abs_scale(K, V, evicted_gpu, w.C, nch, wts, s0)
    assert np.all(np.abs(ks - ek) <= SUM_TOL * ak + 1e-30)
    assert np.all(np.abs(vs - ev) <= SUM_TOL * av + 1e-30)
    # attention
    o_gpu = gpu["out"][b, h * G:(h + 1) * G].double().cpu().numpy()
    if diff.size:
        Kc = K[pos_gpu]
        Vc = V[pos_gpu]
        dense = O.dense_positions(w.T[b], s0, A)
        o_ref = O.attend_head(q, K[dense], V[dense], Kc, Vc, ks, vs, cc)
        report["staged_attn"] += 1
    else:
        o_ref = ref.out
    err = np.abs(o_gpu - o_ref).max(axis=1) / np.abs(o_ref).max(axis=1)
    assert np.all(err <= ATTN_TOL), f"attention rel err {err.max():.3g} at ({b},{h})"
    report["max_attn_err"] = max(report["max_attn_err"], float(err.max()))
    return int(diff.size)


def _abs_scale(K, V, evicted, C, nch, wts, origin):
    """Per chunk, the merge of |k| and |v| over its evicted tokens: the scale
    of the float32 sums' rounding error.  Mean merging: plain sums of |x|
    (np.add.at, so a 64k-token head costs milliseconds); weighted merging:
    the oracle's own weighted merge of |x|."""
    if wts is not None:
        ak, av, _ = O.condense(np.abs(K), np.abs(V), evicted, np.arange(len(K)), C, nch, wts,
                               origin=origin)
        return ak, av
    d = K.shape[1]
    ak = np.zeros((nch, d))
    av = np.zeros((nch, d))
    j = (np.asarray(evicted, np.int64) - origin) // C
    np.add.at(ak, j, np.abs(K[evicted].astype(np.float64)))
    np.add.at(av, j, np.abs(V[evicted].astype(np.float64)))
    return ak, av


def new_report():
    return dict(logit_1ulp=0, l2_1ulp=0, borderline=0, selected=0, candidates=0, staged_attn=0,
                max_attn_err=0.0, heads=0, sparse_heads=0)


def check_case(case, gpu, p, heads=None, stages=True, skip_slots=None):
    """skip_slots: optional [B][Hkv] array, non-zero = sparse-loaded head."""
    rep = new_report()
    w = case.w
    if heads is None:
        heads = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    for b, h in heads:
        check_head(case, b, h, gpu, p, rep, stages,
                   skip_slots=skip_slots is not None and bool(skip_slots[b, h]))
        rep["heads"] += 1
    return rep


def check_all_heads_invariants(case, desc, gpu):
    """Cheap properties on every (b, h), checked on the device: kept +
    evicted = aged, counts within capacity, positions strictly increasing."""
    w = case.w
    t = gpu["tiers"]
    A = torch.clamp(case.ctx_len.long() - w.W - w.sinks, min=0)
    cnt = t.count.long()
    assert torch.all(cnt >= 0) and torch.all(cnt <= A[:, None])
    nch_max = desc.chunk_cap
    idx = torch.arange(nch_max, device=cnt.device)
    nch = (A + w.C - 1) // w.C
    valid = idx[None, :] < nch[:, None]
    evicted = (t.ccount.long() * valid[:, None, :]).sum(-1)
    assert torch.equal(evicted + cnt, A[:, None].expand_as(cnt))
    pos = t.pos.long()
    slot = torch.arange(desc.sparse_cap, device=pos.device)
    live = slot[None, None, 1:] < cnt[..., None]
    assert torch.all((pos[..., 1:] > pos[..., :-1]) | ~live)
    # sink positions never leave the dense tier
    assert torch.all((pos >= w.sinks) | ~(slot[None, None, :] < cnt[..., None]))
