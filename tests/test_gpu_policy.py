"""GPU parity of the rewrite-versus-sparse-loading path (gist.science
technical summary, section 2.C: Sparse Loading, Memory-Time Integral with
budget thresholds) and of steps that reuse a selection.

  * hardkv_plan and the plan fused into hardkv_step_policy choose exactly
    the oracle's mode for every head (integer decision, bit-exact).
  * A sparse-loaded head gets the oracle's positions, count and chunks, its
    k / v slots are not touched, and its attention output is the oracle's
    and bit-identical to the rewritten head's (same values, same order).
  * Reuse steps (window W + i, same tiers) match the oracle's reuse
    attention, for rewritten and sparse-loaded heads alike.
Comparison rules: tests/parity.py.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle as O
from decode_kv_cache_head_amd import hardkv as H
from decode_kv_cache_head_amd import synth as S

from parity import (ATTN_TOL, cache_of, check_all_heads_invariants, check_case, desc_for,
                    new_report, borderline_tokens, run_step)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def small(name, **kw):
    base = dict(name=name, B=3, Hq=8, Hkv=2, d=128, T=(2100, 777, 40), dtype=S.DT_BF16, W=64,
                C=64, p=0.9)
    base.update(kw)
    return S.Workload(**base)


def oracle_modes(case, desc, count, pol):
    w = case.w
    modes = np.empty((w.B, w.Hkv), np.uint8)
    for b in range(w.B):
        A = min(max(int(case.ctx_len[b]) - desc.dense_window - desc.sinks, 0), desc.sparse_cap)
        for h in range(w.Hkv):
            modes[b, h] = O.plan_head(A, int(count[b, h]), desc.dense_window, pol.kind,
                                      pol.horizon, pol.l_lower, pol.l_upper)
    return modes


def run_policy(case, desc, pol, sentinel=True):
    w = case.w
    dev = case.q.device
    ws = H.alloc_workspace(desc, dev)
    tiers = H.alloc_tiers(desc, dev, mode=True)
    if sentinel:
        tiers.k.view(torch.int16 if tiers.k.dtype == torch.bfloat16 else torch.int32).fill_(0x5A5A)
        tiers.v.view(torch.int16 if tiers.v.dtype == torch.bfloat16 else torch.int32).fill_(0x5A5A)
    tiers.mode.fill_(7)
    out = torch.full((w.B, w.Hq, w.d), float("nan"), device=dev)
    H.step_policy(desc, pol, case.q, cache_of(case), case.metric, tiers, out, ws)
    torch.cuda.synchronize()
    return dict(tiers=tiers, out=out)


def check_sparse_slots_untouched(g):
    t = g["tiers"]
    view = torch.int16 if t.k.dtype == torch.bfloat16 else torch.int32
    sp = t.mode.bool()
    assert torch.all(t.k.view(view)[sp] == 0x5A5A)
    assert torch.all(t.v.view(view)[sp] == 0x5A5A)


def check_policy_case(case, desc, pol, ref_step=None):
    """step_policy against the oracle: modes exact, tiers and attention to
    the usual rules, output bit-identical to the all-rewrite step."""
    w = case.w
    g = run_policy(case, desc, pol)
    modes = g["tiers"].mode.cpu().numpy()
    want = oracle_modes(case, desc, g["tiers"].count.cpu().numpy(), pol)
    assert np.array_equal(modes, want), (modes, want)
    check_sparse_slots_untouched(g)
    check_all_heads_invariants(case, desc, g)
    rep = check_case(case, g, w.p, stages=False, skip_slots=g["tiers"].mode.cpu().numpy())
    if ref_step is None:
        ref_step = run_step(case, desc)
    assert torch.equal(g["out"], ref_step["out"])
    assert torch.equal(g["tiers"].count, ref_step["tiers"].count)
    return g, rep, modes


def test_plan_exact_on_large_budgets(gpu):
    # hardkv_plan on counts drawn over the whole int32 range of A: the
    # 128-bit integrals decide exactly as the oracle's Python integers
    B, Hkv = 64, 8
    W = 4096
    desc = H.make_desc(B, Hkv * 4, Hkv, 128, H.BF16, W, 1 << 20, 0.9, 2_000_000_000,
                       sparse_cap=2_000_000_000 - W, chunk_cap=2000)
    assert H.validate(desc) == H.OK
    g = torch.Generator().manual_seed(11)
    ctx = torch.randint(1, 2_000_000_000, (B,), generator=g, dtype=torch.int64)
    ctx[:4] = torch.tensor([1, W, W + 1, 2_000_000_000])
    A = torch.clamp(ctx - W, min=0)
    frac = torch.rand((B, Hkv), generator=g, dtype=torch.float64)
    frac[:, 0] = 0.0
    frac[:, 1] = 1.0
    count = torch.floor(A[:, None].double() * frac).long()
    ctx_d = ctx.to(torch.int32).to(gpu)
    cnt_d = count.to(torch.int32).to(gpu)
    mode = torch.full((B, Hkv), 9, dtype=torch.uint8, device=gpu)
    seen = set()
    for pol in [H.policy(H.POLICY_REWRITE), H.policy(H.POLICY_SPARSE),
                H.policy(H.POLICY_MTI, 1), H.policy(H.POLICY_MTI, 2), H.policy(H.POLICY_MTI, 7),
                H.policy(H.POLICY_MTI, 100), H.policy(H.POLICY_MTI, 2 ** 31 - 1),
                H.policy(H.POLICY_MTI, 5, 1 << 28, 1 << 30)]:
        H.plan(desc, pol, ctx_d, cnt_d, mode)
        torch.cuda.synchronize()
        got = mode.cpu().numpy()
        want = np.array([[O.plan_head(int(A[b]), int(count[b, h]), W, pol.kind, pol.horizon,
                                      pol.l_lower, pol.l_upper) for h in range(Hkv)]
                         for b in range(B)], np.uint8)
        assert np.array_equal(got, want), pol.horizon
        seen |= set(got.ravel().tolist())
    assert seen == {0, 1}


GRID = [
    dict(dtype=S.DT_BF16, d=128, Hq=8, Hkv=2, C=64, p=0.9),
    dict(dtype=S.DT_BF16, d=128, Hq=8, Hkv=2, C=64, p=0.5, block_size=16),
    dict(dtype=S.DT_F32, d=128, Hq=4, Hkv=2, C=7, p=0.8),
    dict(dtype=S.DT_F32, d=64, Hq=16, Hkv=2, C=100, p=0.99, block_size=32),
    dict(dtype=S.DT_BF16, d=128, Hq=16, Hkv=4, C=64, p=0.9, peaked_heads=(0, 2),
         metric=(S.METRIC_QK, S.METRIC_QK, S.METRIC_L2, S.METRIC_L2), block_size=16),
    dict(dtype=S.DT_BF16, d=128, Hq=8, Hkv=2, C=64, p=0.8, sinks=4, merge=1, block_size=16),
    dict(dtype=S.DT_F32, d=64, Hq=8, Hkv=2, C=7, p=0.9, sinks=33, merge=1),
]


@pytest.mark.parametrize("i", range(len(GRID)))
def test_step_policy_all_sparse_and_mixed(gpu, i):
    w = small(f"pol{i}", **GRID[i])
    say("policy grid", i, w)
    case = S.make_case(w, gpu)
    desc = desc_for(case)
    ref = run_step(case, desc)
    _, rep, modes = check_policy_case(case, desc, H.policy(H.POLICY_SPARSE), ref)
    assert modes.all()
    say("sparse", rep)
    # a mixture: thresholds put the smaller budgets on rewrite
    cnt = ref["tiers"].count.cpu().numpy()
    mid = int(np.median(cnt[cnt > 0])) if (cnt > 0).any() else 1
    for pol in (H.policy(H.POLICY_MTI, 1, mid), H.policy(H.POLICY_MTI, 64),
                H.policy(H.POLICY_MTI, 3, 0, mid)):
        _, rep, modes = check_policy_case(case, desc, pol, ref)
        say("mti", pol.horizon, pol.l_lower, pol.l_upper, modes.ravel().tolist(), rep)


def test_staged_sparse_loading(gpu):
    # hardkv_plan -> hardkv_compact (mode honoured) -> hardkv_decode_attn
    # (sparse heads gather from the cache), against the oracle and the
    # all-rewrite staged path
    for kw in (dict(C=64, block_size=16), dict(C=7, dtype=S.DT_F32, d=64)):
        w = small("staged_sparse", **kw)
        case = S.make_case(w, gpu)
        desc = desc_for(case)
        dev = gpu
        B, Hkv, cap = w.B, w.Hkv, desc.sparse_cap
        ws = H.alloc_workspace(desc, dev)
        cache = cache_of(case)
        logit = torch.empty((B, Hkv, cap), device=dev)
        l2 = torch.empty((B, Hkv, cap), device=dev)
        stats = torch.empty((B, Hkv, 4), dtype=torch.float64, device=dev)
        mask = torch.empty((B, Hkv, cap), dtype=torch.uint8, device=dev)
        count = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
        H.score(desc, case.q, cache, case.metric, logit, l2, ws)
        H.calibrate(desc, case.ctx_len, case.metric, logit, l2, stats, ws)
        H.topp_select(desc, case.ctx_len, case.metric, logit, l2, stats, mask, count, ws)
        outs = {}
        for kind in (H.POLICY_REWRITE, H.POLICY_SPARSE, H.POLICY_MTI):
            pol = H.policy(kind, 4)
            tiers = H.alloc_tiers(desc, dev, mode=True)
            view = torch.int16 if tiers.k.dtype == torch.bfloat16 else torch.int32
            tiers.k.view(view).fill_(0x5A5A)
            tiers.v.view(view).fill_(0x5A5A)
            out = torch.full((B, w.Hq, w.d), float("nan"), device=dev)
            H.plan(desc, pol, case.ctx_len, count, tiers.mode)
            H.compact(desc, cache, mask, tiers, ws)
            H.decode_attn(desc, case.q, cache, tiers, out, ws)
            torch.cuda.synchronize()
            g = dict(tiers=tiers, out=out)
            want = oracle_modes(case, desc, count.cpu().numpy(), pol)
            assert np.array_equal(tiers.mode.cpu().numpy(), want)
            check_sparse_slots_untouched(g)
            check_case(case, g, w.p, stages=False, skip_slots=tiers.mode.cpu().numpy())
            outs[kind] = out
        assert torch.equal(outs[H.POLICY_REWRITE], outs[H.POLICY_SPARSE])
        assert torch.equal(outs[H.POLICY_REWRITE], outs[H.POLICY_MTI])


def _reuse_check(case, desc, g, T_sel, steps, report, oracle_sel):
    """Reuse the tiers of a selection at T_sel for later steps: window
    W + i, context T_sel + i, fresh queries; compare with the oracle's reuse
    attention where the GPU kept the oracle's set, else with the oracle's
    attention over the GPU's own tiers (borderline tokens, see parity.py)."""
    w = case.w
    dev = case.q.device
    G = w.G
    tiers = g["tiers"]
    for i in steps:
        ctx = (T_sel + i).to(torch.int32)
        d_i = H.make_desc(w.B, w.Hq, w.Hkv, w.d, w.dtype, w.W + i, w.C, w.p, case.ctx_cap,
                          w.block_size, case.max_blocks, desc.sparse_cap, desc.chunk_cap,
                          w.sinks, w.merge)
        ws = H.alloc_workspace(d_i, dev)
        qn = S._randn((w.B, w.Hq, w.d), w, dev, "reuse_q", i).to(case.q.dtype)
        out = torch.full((w.B, w.Hq, w.d), float("nan"), device=dev)
        H.decode_attn(d_i, qn, H.cache_struct(case.k, case.v, ctx, case.block_table), tiers,
                      out, ws)
        torch.cuda.synchronize()
        for b in range(w.B):
            Ts = int(T_sel[b])
            Tn = int(ctx[b])
            A = max(Ts - w.W - w.sinks, 0)
            dense = O.dense_positions(Tn, w.sinks, A)
            for h in range(w.Hkv):
                K = S.head_rows(case, b, h, "k").float().cpu().numpy()
                V = S.head_rows(case, b, h, "v").float().cpu().numpy()
                q = qn[b, h * G:(h + 1) * G].double().cpu().numpy()
                k_gpu = int(tiers.count[b, h])
                pos = tiers.pos[b, h, :k_gpu].cpu().numpy().astype(np.int64)
                sel = oracle_sel[(b, h)]
                if np.array_equal(pos, sel.pos):
                    o_ref = O.reuse_head(q, K, V, Tn, sel)
                    report["oracle_reuse"] += 1
                else:
                    nch = -(-A // w.C) if A else 0
                    o_ref = O.attend_head(q, K[dense], V[dense], K[pos], V[pos],
                                          tiers.ksum[b, h, :nch].double().cpu().numpy(),
                                          tiers.vsum[b, h, :nch].double().cpu().numpy(),
                                          tiers.ccount[b, h, :nch].cpu().numpy())
                    report["staged_attn"] += 1
                o = out[b, h * G:(h + 1) * G].double().cpu().numpy()
                err = np.abs(o - o_ref).max(axis=1) / np.abs(o_ref).max(axis=1)
                assert np.all(err <= ATTN_TOL), (i, b, h, err.max())
                report["max_attn_err"] = max(report["max_attn_err"], float(err.max()))
                report["heads"] += 1


@pytest.mark.parametrize("kw", [dict(C=64, block_size=16), dict(C=7, dtype=S.DT_F32),
                                dict(C=64, peaked_heads=(1,), W=128),
                                dict(C=64, block_size=16, sinks=5, merge=1)])
def test_reuse_steps(gpu, kw):
    # sequences long enough to grow by 40 tokens past the selection
    R = 40
    w = small("reuse", T=(2100 + R, 777 + R, 100 + R), **kw)
    case = S.make_case(w, gpu)
    T_sel = (case.ctx_len - R).to(torch.int32)
    wsel = dataclasses.replace(w, T=tuple(int(t) for t in T_sel.cpu()))
    sel_case = S.Case(wsel, case.q, case.k, case.v, T_sel, case.block_table, case.metric,
                      case.ctx_cap, case.max_blocks, case.extra)
    desc = desc_for(case)
    # the selection at T - R, checked against the oracle as usual
    ref = run_step(sel_case, desc)
    check_case(sel_case, ref, w.p, stages=False)
    oracle_sel = {}
    for b in range(w.B):
        for h in range(w.Hkv):
            q = case.q[b, h * w.G:(h + 1) * w.G].double().cpu().numpy()
            K = S.head_rows(case, b, h, "k").float().cpu().numpy()
            V = S.head_rows(case, b, h, "v").float().cpu().numpy()
            oracle_sel[(b, h)] = O.step_head(q, K, V, wsel.T[b], w.W, w.C, w.p,
                                             int(w.metrics[h]), w.sinks, w.merge)
    rep = new_report()
    rep["oracle_reuse"] = 0
    full = S.Case(w, case.q, case.k, case.v, case.ctx_len, case.block_table, case.metric,
                  case.ctx_cap, case.max_blocks, case.extra)
    for pol in (H.policy(H.POLICY_REWRITE), H.policy(H.POLICY_SPARSE),
                H.policy(H.POLICY_MTI, 8)):
        g = run_policy(sel_case, desc, pol)
        assert torch.equal(g["out"], ref["out"])
        _reuse_check(full, desc, g, T_sel, (1, 2, 17, R), rep, oracle_sel)
    say("reuse", rep)
    assert rep["heads"] == 3 * 4 * w.B * w.Hkv
    assert rep["oracle_reuse"] > rep["heads"] // 2


def test_headline_policy_b32_16k_paged(gpu):
    """Full headline size: the MTI plan on every head equals the oracle's
    decision for the GPU budgets, sparse heads leave their slots alone, the
    output equals the all-rewrite step bit for bit, and sampled heads match
    the oracle."""
    w = S.workload("qwen8b_b32_16k_paged")
    case = S.make_case(w, gpu)
    desc = desc_for(case)
    say("headline policy", w.name)
    ref = run_step(case, desc)
    cnt = ref["tiers"].count.cpu().numpy()
    for pol in (H.policy(H.POLICY_MTI, 22), H.policy(H.POLICY_MTI, 23),
                H.policy(H.POLICY_MTI, 4, 0, int(np.median(cnt)))):
        g = run_policy(case, desc, pol)
        modes = g["tiers"].mode.cpu().numpy()
        assert np.array_equal(modes, oracle_modes(case, desc, g["tiers"].count.cpu().numpy(),
                                                  pol))
        check_sparse_slots_untouched(g)
        assert torch.equal(g["out"], ref["out"])
        say("modes", pol.horizon, pol.l_upper, int(modes.sum()), "of", modes.size, "sparse")
    heads = [(0, 0), (7, 3), (31, 7)]
    rep = check_case(case, g, w.p, heads=heads, stages=False, skip_slots=modes)
    say(rep)
