"""GPU parity of the rewritten tier under its head-wise block manager
(gist.science technical summary, section 2.C "Metadata": a head-wise block
manager allocates head-adaptive budgets under static shapes).

The rewritten tier is a pool of blocks of tier_block rows with a stack of
free block ids; every selection returns each head's blocks and hands out
ceil(k / tier_block) new ones per rewritten head, in (b, h) order; heads
that do not fit are sparse-loaded.

  * table, held counts, the free stack and the modes equal the oracle's
    tier_alloc exactly, step after step (blocks recycled);
  * every rewritten head's rows, read through its table, are bit copies of
    its cache rows; positions, counts, chunks and the attention output equal
    the per-head layout's bit for bit and the oracle's;
  * a pool shared by two tiers (two layers) conserves its blocks;
  * the standalone calls (tier_alloc, compact, decode_attn) agree with the
    step, and a later attention call reads the tier through the table.
Comparison rules: tests/parity.py.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from decode_kv_cache_head_amd import hardkv as H
from decode_kv_cache_head_amd import synth as S

from parity import cache_of, check_all_heads_invariants, check_case, desc_for, run_step

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def small(name, **kw):
    base = dict(name=name, B=3, Hq=8, Hkv=2, d=128, T=(2100, 777, 40), dtype=S.DT_BF16, W=64,
                C=64, p=0.9)
    base.update(kw)
    return S.Workload(**base)


def bm_desc(case, tb, nblocks):
    d = desc_for(case)
    d.tier_block = tb
    d.tier_blocks = nblocks
    return d


def bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def host_state(t: H.Tiers):
    return (t.table.cpu().numpy().astype(np.int64), t.held.cpu().numpy().astype(np.int64),
            t.free_ids.cpu().numpy().astype(np.int64), int(t.free_top.item()),
            t.mode.cpu().numpy())


def expect_alloc(before, counts, modes_in, desc):
    """The oracle's allocation from the state before the step."""
    table, held, ids, top, _ = before
    cap = max(desc.ctx_cap - desc.dense_window - desc.sinks, 0)
    return O.tier_alloc(table, held, ids, top, counts, modes_in, desc.tier_block, cap)


def check_alloc(t: H.Tiers, want):
    table, held, ids, top, modes = want
    g_table, g_held, g_ids, g_top, g_modes = host_state(t)
    assert g_top == top
    assert np.array_equal(g_held, held)
    assert np.array_equal(g_modes, modes)
    assert np.array_equal(g_ids[:top], ids[:top])
    B, Hkv = held.shape
    for b in range(B):
        for h in range(Hkv):
            n = int(held[b, h])
            assert np.array_equal(g_table[b, h, :n], table[b, h, :n]), (b, h)


def check_conserved(tiers_list, nblocks):
    live = []
    for t in tiers_list:
        tab, held = t.table.cpu().numpy(), t.held.cpu().numpy()
        for b in range(held.shape[0]):
            for h in range(held.shape[1]):
                live += tab[b, h, :held[b, h]].tolist()
    top = int(tiers_list[0].free_top.item())
    stack = tiers_list[0].free_ids[:top].cpu().tolist()
    assert sorted(live + stack) == list(range(nblocks))


def fresh_tiers(desc, dev):
    t = H.alloc_tiers(desc, dev)
    bits(t.k).fill_(0x5A5A)
    bits(t.v).fill_(0x5A5A)
    H.tier_init(desc, t)
    torch.cuda.synchronize()
    return t


@pytest.mark.parametrize("tb,paged", [(16, False), (64, True), (1024, False)])
def test_step_matches_regions_and_oracle(gpu, tb, paged):
    w = small(f"tier{tb}", block_size=16 if paged else 0)
    case = S.make_case(w, gpu)
    ref = run_step(case, desc_for(case))
    desc = bm_desc(case, tb, 1000)
    t = fresh_tiers(desc, gpu)
    before = host_state(t)
    g = run_step(case, desc, tiers=t)
    say(w.name, "counts", t.count.cpu().tolist(), "held", t.held.cpu().tolist())
    want = expect_alloc(before, t.count.cpu().numpy(), np.zeros((w.B, w.Hkv), np.uint8), desc)
    check_alloc(t, want)
    assert torch.equal(t.count, ref["tiers"].count)
    assert torch.equal(g["out"], ref["out"])
    for b in range(w.B):
        for h in range(w.Hkv):
            n = int(t.count[b, h])
            assert torch.equal(t.pos[b, h, :n], ref["tiers"].pos[b, h, :n])
            assert torch.equal(bits(t.slots(b, h, "k")), bits(ref["tiers"].slots(b, h, "k")))
            assert torch.equal(bits(t.slots(b, h, "v")), bits(ref["tiers"].slots(b, h, "v")))
    for b in range(w.B):
        nch = -(-max(w.T[b] - w.W, 0) // w.C)
        for h in range(w.Hkv):
            for f in ("ksum", "vsum", "ccount"):
                assert torch.equal(getattr(t, f)[b, h, :nch], getattr(ref["tiers"], f)[b, h, :nch])
    check_all_heads_invariants(case, desc, g)
    rep = check_case(case, g, w.p, stages=False)
    say(rep)
    check_conserved([t], desc.tier_blocks)


def test_recycling_and_exhaustion_over_steps(gpu):
    """Five selections on one tier with a pool too small for every head:
    blocks come back and go out again in the documented order; heads that do
    not fit are sparse-loaded and still attend exactly (equal to the
    per-head layout's output)."""
    nblocks = 260
    for step in range(5):
        w = small("recycle", B=4, T=(3000, 1900, 2600, 700), p=0.5 + 0.1 * step, seed=40 + step)
        case = S.make_case(w, gpu)
        desc = bm_desc(case, 16, nblocks)
        if step == 0:
            t = fresh_tiers(desc, gpu)
        before = host_state(t)
        g = run_step(case, desc, tiers=t)
        ref = run_step(case, desc_for(case))
        want = expect_alloc(before, t.count.cpu().numpy(), np.zeros((w.B, w.Hkv), np.uint8),
                            desc)
        check_alloc(t, want)
        sparse = t.mode.cpu().numpy()
        say("step", step, "held", t.held.cpu().tolist(), "sparse heads", int(sparse.sum()),
            "free", int(t.free_top.item()))
        assert torch.equal(g["out"], ref["out"])
        check_conserved([t], nblocks)
        rep = check_case(case, g, w.p, stages=False, skip_slots=sparse)
        say(rep)
        if step >= 1:
            assert sparse.sum() > 0  # the small pool runs out at these budgets


def test_pool_shared_by_two_layers(gpu):
    nblocks = 400
    w0 = small("layer0", B=2, T=(2500, 1800), seed=7)
    w1 = small("layer1", B=2, T=(2200, 2900), seed=8)
    c0, c1 = S.make_case(w0, gpu), S.make_case(w1, gpu)
    d0, d1 = bm_desc(c0, 32, nblocks), bm_desc(c1, 32, nblocks)
    t0 = fresh_tiers(d0, gpu)
    t1 = H.alloc_tiers(d1, gpu, blocks=(t0.k, t0.v, t0.free_ids, t0.free_top))
    H.tier_init(d1, t1)  # t1's own table and held counts (and the still-full shared stack)
    for rnd in range(3):
        for c, d, t in ((c0, d0, t0), (c1, d1, t1)):
            before = host_state(t)
            g = run_step(c, d, tiers=t)
            want = expect_alloc(before, t.count.cpu().numpy(),
                                np.zeros((c.w.B, c.w.Hkv), np.uint8), d)
            check_alloc(t, want)
            ref = run_step(c, desc_for(c))
            assert torch.equal(g["out"], ref["out"])
            check_conserved([t0, t1], nblocks)
    say("free after 3 rounds", int(t0.free_top.item()))


def test_staged_calls_and_reuse_attention(gpu):
    """select -> tier_alloc -> compact -> decode_attn by hand equals the step;
    a second attention call over the same tiers (selection reuse) reads the
    rows through the table and equals the per-head layout's."""
    w = small("staged", block_size=16)
    case = S.make_case(w, gpu)
    desc = bm_desc(case, 16, 1000)
    dev = gpu
    B, Hkv, cap = w.B, w.Hkv, desc.sparse_cap
    ws = H.alloc_workspace(desc, dev)
    cache = cache_of(case)
    logit = torch.empty((B, Hkv, cap), device=dev)
    l2 = torch.empty((B, Hkv, cap), device=dev)
    stats = torch.zeros((B, Hkv, 4), dtype=torch.float64, device=dev)
    mask = torch.empty((B, Hkv, cap), dtype=torch.uint8, device=dev)
    count = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    t = fresh_tiers(desc, dev)
    out = torch.empty((B, w.Hq, w.d), device=dev)
    H.score(desc, case.q, cache, case.metric, logit, l2, ws)
    H.calibrate(desc, case.ctx_len, case.metric, logit, l2, stats, ws)
    H.topp_select(desc, case.ctx_len, case.metric, logit, l2, stats, mask, count, ws)
    t.mode.zero_()
    H.tier_alloc(desc, count, t)
    H.compact_scored(desc, cache, case.metric, logit, l2, stats, mask, t, ws)
    H.decode_attn(desc, case.q, cache, t, out, ws)
    torch.cuda.synchronize()
    step = run_step(case, bm_desc(case, 16, 1000), tiers=fresh_tiers(desc, dev))
    ref = run_step(case, desc_for(case))
    assert torch.equal(t.count, step["tiers"].count)
    assert torch.equal(t.held, step["tiers"].held)
    for b in range(B):
        for h in range(Hkv):
            n = int(t.held[b, h])
            assert torch.equal(t.table[b, h, :n], step["tiers"].table[b, h, :n])
    err = ((out - ref["out"]).abs().amax(-1) / ref["out"].abs().amax(-1)).max().item()
    say("staged vs step attention rel err", err)
    assert err <= 1e-4
    # selection reuse: attention alone over the block-managed tiers
    out2 = torch.empty_like(out)
    H.decode_attn(desc, case.q, cache, t, out2, ws)
    ref2 = torch.empty_like(out)
    H.decode_attn(desc_for(case), case.q, cache, ref["tiers"], ref2, H.alloc_workspace(
        desc_for(case), dev))
    torch.cuda.synchronize()
    assert torch.equal(out2, ref2)


def test_headline_shape_with_block_manager(gpu):
    """The 16k paged headline workload with 64-row tier blocks: every head
    against the oracle, the allocation against the oracle's rule."""
    w = S.workload("qwen8b_b32_16k_paged")
    case = S.make_case(w, gpu)
    desc = bm_desc(case, 64, 32 * 8 * 256)
    t = fresh_tiers(desc, gpu)
    before = host_state(t)
    g = run_step(case, desc, tiers=t)
    want = expect_alloc(before, t.count.cpu().numpy(), np.zeros((w.B, w.Hkv), np.uint8), desc)
    check_alloc(t, want)
    check_all_heads_invariants(case, desc, g)
    rep = check_case(case, g, w.p, stages=False)
    say(rep)
    assert rep["heads"] == w.B * w.Hkv
    check_conserved([t], desc.tier_blocks)
