"""GPU parity of the packed rewritten tier (gist.science technical summary,
section 2.C: head-wise allocation under static shapes, Flatten Index to the
sum).  The heads' kept rows are laid end to end in one region; heads past
its end are served by sparse loading.

  * offsets and the overflow modes equal the oracle's pack_heads, exactly;
  * every rewritten head's rows are bit copies of its cache rows, and rows
    of the region past the last packed head are untouched;
  * the attention output equals the per-head layout's bit for bit (the same
    values are attended in the same order), and the oracle's.
Comparison rules: tests/parity.py.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from decode_kv_cache_head_amd import hardkv as H
from decode_kv_cache_head_amd import synth as S

from parity import (cache_of, check_all_heads_invariants, check_case, desc_for, run_stages,
                    run_step)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def small(name, **kw):
    base = dict(name=name, B=3, Hq=8, Hkv=2, d=128, T=(2100, 777, 40), dtype=S.DT_BF16, W=64,
                C=64, p=0.9)
    base.update(kw)
    return S.Workload(**base)


def packed_desc(case, rows):
    d = desc_for(case)
    d.packed_rows = rows
    return d


def bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def run_packed(case, desc, pol=None):
    w = case.w
    dev = case.q.device
    ws = H.alloc_workspace(desc, dev)
    tiers = H.alloc_tiers(desc, dev)
    bits(tiers.k).fill_(0x5A5A)
    bits(tiers.v).fill_(0x5A5A)
    out = torch.full((w.B, w.Hq, w.d), float("nan"), device=dev)
    if pol is None:
        H.step(desc, case.q, cache_of(case), case.metric, tiers, out, ws)
    else:
        H.step_policy(desc, pol, case.q, cache_of(case), case.metric, tiers, out, ws)
    torch.cuda.synchronize()
    return dict(tiers=tiers, out=out)


def check_packing(case, desc, g, plan_modes):
    """Offsets / modes against the oracle; untouched rows past the packed heads."""
    t = g["tiers"]
    counts = t.count.cpu().numpy()
    off, modes = O.pack_heads(counts, plan_modes, desc.packed_rows)
    got_m = t.mode.cpu().numpy()
    assert np.array_equal(got_m, modes)
    assert np.array_equal(t.offset.cpu().numpy(), off)
    used = [int(off.ravel()[i] + counts.ravel()[i]) for i in range(counts.size)
            if modes.ravel()[i] == O.MODE_REWRITE]
    end = max(used, default=0)
    assert torch.all(bits(t.k)[end:] == 0x5A5A) and torch.all(bits(t.v)[end:] == 0x5A5A)
    return got_m


GRID = [
    dict(C=64),
    dict(C=64, block_size=16, p=0.5),
    dict(C=7, dtype=S.DT_F32, d=64),
    dict(C=64, block_size=16, sinks=4, merge=1, metric=(S.METRIC_QK, S.METRIC_L2)),
    dict(C=128, Hkv=4, Hq=16, peaked_heads=(1, 2), T=(3000, 1200, 300)),
]


@pytest.mark.parametrize("i", range(len(GRID)))
def test_packed_step_matches_per_head_layout(gpu, i):
    w = small(f"pack{i}", **GRID[i])
    say("pack grid", i, w)
    case = S.make_case(w, gpu)
    ref = run_step(case, desc_for(case))
    total = int(ref["tiers"].count.sum())
    rewrite_all = np.zeros((w.B, w.Hkv), np.uint8)
    for rows in (total + 17, total, max(total // 2, 1), 1):
        desc = packed_desc(case, rows)
        g = run_packed(case, desc)
        modes = check_packing(case, desc, g, rewrite_all)
        assert torch.equal(g["out"], ref["out"])
        check_all_heads_invariants(case, desc, g)
        rep = check_case(case, g, w.p, stages=False, skip_slots=modes)
        say("rows", rows, "of", total, "sparse heads", int(modes.sum()), rep["max_attn_err"])
        if rows >= total:
            assert modes.sum() == 0


def test_packed_with_policy_and_staged(gpu):
    w = small("pack_pol", C=64, block_size=16, peaked_heads=(0,), T=(2500, 1500, 900))
    case = S.make_case(w, gpu)
    ref = run_step(case, desc_for(case))
    total = int(ref["tiers"].count.sum())
    for pol in (H.policy(H.POLICY_MTI, 8), H.policy(H.POLICY_MTI, 1, 200)):
        for rows in (total, total // 3):
            desc = packed_desc(case, rows)
            g = run_packed(case, desc, pol)
            counts = g["tiers"].count.cpu().numpy()
            A = np.maximum(np.array(w.T) - w.W, 0)
            plan = np.array([[O.plan_head(int(A[b]), int(counts[b, h]), w.W, pol.kind,
                                          pol.horizon, pol.l_lower, pol.l_upper)
                              for h in range(w.Hkv)] for b in range(w.B)], np.uint8)
            modes = check_packing(case, desc, g, plan)
            assert torch.equal(g["out"], ref["out"])
            check_case(case, g, w.p, stages=False, skip_slots=modes)
    # staged: plan -> pack -> compact -> decode_attn
    desc = packed_desc(case, total // 2)
    dev = gpu
    B, Hkv, cap = w.B, w.Hkv, desc.sparse_cap
    ws = H.alloc_workspace(desc, dev)
    cache = cache_of(case)
    logit = torch.empty((B, Hkv, cap), device=dev)
    l2 = torch.empty((B, Hkv, cap), device=dev)
    stats = torch.empty((B, Hkv, 4), dtype=torch.float64, device=dev)
    mask = torch.empty((B, Hkv, cap), dtype=torch.uint8, device=dev)
    count = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    tiers = H.alloc_tiers(desc, dev)
    bits(tiers.k).fill_(0x5A5A)
    bits(tiers.v).fill_(0x5A5A)
    out = torch.empty((B, w.Hq, w.d), device=dev)
    H.score(desc, case.q, cache, case.metric, logit, l2, ws)
    H.calibrate(desc, case.ctx_len, case.metric, logit, l2, stats, ws)
    H.topp_select(desc, case.ctx_len, case.metric, logit, l2, stats, mask, count, ws)
    pol = H.policy(H.POLICY_MTI, 8)
    H.plan(desc, pol, case.ctx_len, count, tiers.mode)
    torch.cuda.synchronize()
    plan = tiers.mode.cpu().numpy().copy()
    H.pack(desc, count, tiers)
    H.compact(desc, cache, mask, tiers, ws)
    H.decode_attn(desc, case.q, cache, tiers, out, ws)
    torch.cuda.synchronize()
    g = dict(tiers=tiers, out=out)
    modes = check_packing(case, desc, g, plan)
    # the staged path sums attention in another order than the fused step:
    # compare with the staged per-head layout
    assert torch.equal(out, run_stages(case, desc_for(case))["out"])
    check_case(case, g, w.p, stages=False, skip_slots=modes)


def test_packed_headline_b32_16k(gpu):
    """Full headline size with a region of 90 % of the kept rows: the first
    heads in (b, h) order are packed, the rest sparse-loaded; the output is
    the per-head layout's, bit for bit."""
    w = S.workload("qwen8b_b32_16k_paged")
    case = S.make_case(w, gpu)
    ref = run_step(case, desc_for(case))
    total = int(ref["tiers"].count.sum())
    desc = packed_desc(case, int(total * 0.9))
    g = run_packed(case, desc)
    modes = check_packing(case, desc, g, np.zeros((w.B, w.Hkv), np.uint8))
    assert 0 < modes.sum() < modes.size
    assert torch.equal(g["out"], ref["out"])
    check_all_heads_invariants(case, desc, g)
    per_head_rows = w.B * w.Hkv * desc.sparse_cap
    say("packed rows", desc.packed_rows, "per-head rows", per_head_rows, "sparse heads",
        int(modes.sum()))
    check_case(case, g, w.p, heads=[(0, 0), (31, 7), (20, 3)], stages=False, skip_slots=modes)
