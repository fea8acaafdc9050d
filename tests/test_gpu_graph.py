"""hardkv_step captured into a HIP graph (static shapes, persistent pointers:
gist.science technical summary, section 2.C "Metadata" and section 5).

The step is captured once and replayed with new query and cache contents
written into the same buffers between replays; every replay must equal an
eager hardkv_step on the same inputs (tiers bit for bit, attention output
bit for bit since the same kernels run in the same order)."""
import sys

import pytest
import torch

from decode_kv_cache_head_amd import hardkv as H
from decode_kv_cache_head_amd import synth as S

from parity import cache_of, check_case, desc_for

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,kw", [
    ("qwen8b_b1_16k", dict(B=2, T=(5000, 3333))),
    ("qwen8b_b32_16k_paged", dict(B=4, T=(4000, 2500, 300, 1024))),
    # every non-logit metric (key sums formed in the first launch) and both
    # calibration rules
    ("qwen8b_b32_16k_paged", dict(B=3, T=(4000, 2500, 1024), metric=(
        S.METRIC_KEYDIFF, S.METRIC_QK, S.METRIC_L2, S.METRIC_KEYDIFF) * 2)),
    ("qwen8b_b1_16k", dict(B=2, T=(5000, 3333), calibration=1, metric=(
        S.METRIC_L2, S.METRIC_KEYDIFF, S.METRIC_QK, S.METRIC_L2) * 2)),
    ("qwen8b_b32_16k_paged", dict(B=3, T=(4000, 2500, 1024), metric=(
        S.METRIC_RKV, S.METRIC_QK, S.METRIC_KEYDIFF, S.METRIC_RKV) * 2)),
])
def test_step_graph_replay_matches_eager(gpu, name, kw):
    w = S.workload(name, **kw)
    case = S.make_case(w, gpu)
    desc = desc_for(case)
    ws = H.alloc_workspace(desc, gpu)
    tiers = H.alloc_tiers(desc, gpu)
    out = torch.empty((w.B, w.Hq, w.d), device=gpu)
    cache = cache_of(case)
    # warm up on a side stream, then capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        H.step(desc, case.q, cache, case.metric, tiers, out, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        H.step(desc, case.q, cache, case.metric, tiers, out, ws)
    torch.cuda.synchronize()
    ref_tiers = H.alloc_tiers(desc, gpu)
    ref_out = torch.empty_like(out)
    ref_ws = H.alloc_workspace(desc, gpu)
    gen = torch.Generator(device=gpu).manual_seed(5)
    for rep in range(4):
        # new contents in the captured buffers (eager work between replays)
        case.q.copy_((torch.randn(case.q.shape, generator=gen, device=gpu) * (1 + rep)).to(case.q.dtype))
        case.k.copy_(torch.randn(case.k.shape, generator=gen, device=gpu).to(case.k.dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        H.step(desc, case.q, cache, case.metric, ref_tiers, ref_out, ref_ws)
        torch.cuda.synchronize()
        assert torch.equal(tiers.count, ref_tiers.count), rep
        for b in range(w.B):
            for h in range(w.Hkv):
                n = int(ref_tiers.count[b, h])
                assert torch.equal(tiers.pos[b, h, :n], ref_tiers.pos[b, h, :n])
                assert torch.equal(tiers.k[b, h, :n], ref_tiers.k[b, h, :n])
        assert torch.equal(out, ref_out), rep
        if rep == 3:   # and the replayed step is right, not only repeatable
            rep_ = check_case(case, dict(tiers=tiers, out=out), w.p, stages=False)
            print(rep_, file=sys.stderr, flush=True)



def test_step_graph_replay_with_tier_block_manager(gpu):
    """The step with the rewritten tier under its block manager, captured
    once and replayed: the allocation (blocks returned and handed out again
    on the device every replay), the tiers read through the tables and the
    output equal eager steps on an identical pool, replay after replay, with
    the pool small enough that some heads are sparse-loaded."""
    w = S.workload("qwen8b_b32_16k_paged", B=4, T=(4000, 2500, 3000, 1024))
    case = S.make_case(w, gpu)
    desc = desc_for(case)
    desc.tier_block = 32
    desc.tier_blocks = 600
    ws = H.alloc_workspace(desc, gpu)
    out = torch.empty((w.B, w.Hq, w.d), device=gpu)
    cache = cache_of(case)
    tiers = H.alloc_tiers(desc, gpu)
    ref_tiers = H.alloc_tiers(desc, gpu)
    H.tier_init(desc, tiers)
    H.tier_init(desc, ref_tiers)
    ref_out = torch.empty_like(out)
    ref_ws = H.alloc_workspace(desc, gpu)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        H.step(desc, case.q, cache, case.metric, tiers, out, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    H.step(desc, case.q, cache, case.metric, ref_tiers, ref_out, ref_ws)  # same history
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        H.step(desc, case.q, cache, case.metric, tiers, out, ws)
    torch.cuda.synchronize()
    gen = torch.Generator(device=gpu).manual_seed(6)
    sparse_seen = 0
    for rep in range(5):
        case.q.copy_((torch.randn(case.q.shape, generator=gen, device=gpu) * (1 + rep)).to(case.q.dtype))
        case.k.copy_(torch.randn(case.k.shape, generator=gen, device=gpu).to(case.k.dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        H.step(desc, case.q, cache, case.metric, ref_tiers, ref_out, ref_ws)
        torch.cuda.synchronize()
        for f in ("count", "mode", "held", "free_top"):
            assert torch.equal(getattr(tiers, f), getattr(ref_tiers, f)), (rep, f)
        top = int(tiers.free_top.item())
        assert torch.equal(tiers.free_ids[:top], ref_tiers.free_ids[:top]), rep
        for b in range(w.B):
            for h in range(w.Hkv):
                n = int(ref_tiers.count[b, h])
                nb = int(ref_tiers.held[b, h])
                assert torch.equal(tiers.table[b, h, :nb], ref_tiers.table[b, h, :nb])
                assert torch.equal(tiers.pos[b, h, :n], ref_tiers.pos[b, h, :n])
                if nb:
                    assert torch.equal(tiers.slots(b, h, "k"), ref_tiers.slots(b, h, "k"))
        assert torch.equal(out, ref_out), rep
        sparse_seen += int(tiers.mode.sum())
    assert sparse_seen > 0  # the pool ran out on some replays

def _lifecycle(dev, seed, B, Hq, Hkv, d, T0, W, C, p, steps, pool_block=0):
    g = torch.Generator(device=dev).manual_seed(seed)
    desc = H.make_desc(B, Hq, Hkv, d, H.BF16, W, C, p, T0 + steps)
    A = T0 - W
    K = torch.randn((B, Hkv, T0, d), generator=g, device=dev).to(torch.bfloat16)
    V = torch.randn((B, Hkv, T0, d), generator=g, device=dev).to(torch.bfloat16)
    tiers = H.alloc_tiers(desc, dev, zero=True)
    tiers.k[:, :, :A] = K[:, :, :A]
    tiers.v[:, :, :A] = V[:, :, :A]
    tiers.pos[:, :, :A] = torch.arange(A, dtype=torch.int32, device=dev)
    tiers.count.fill_(A)
    ring_k = torch.empty((B, Hkv, W, d), dtype=torch.bfloat16, device=dev)
    ring_v = torch.empty_like(ring_k)
    for t in range(T0 - W, T0):
        ring_k[:, :, t % W] = K[:, :, t]
        ring_v[:, :, t % W] = V[:, :, t]
    seq = torch.full((B,), T0, dtype=torch.int32, device=dev)
    if pool_block:
        maxb = -(-desc.sparse_cap // pool_block)
        return desc, H.paged_state(desc, K[:, :, :A], V[:, :, :A], ring_k, ring_v, seq, pool_block,
                                   B * Hkv * maxb)
    return desc, H.State(ring_k, ring_v, tiers, seq)


@pytest.mark.parametrize("pool_block", [0, 64])
def test_lifecycle_graph_replayed_300_steps(gpu, pool_block):
    """hardkv_step_inplace captured once and replayed for 300 consecutive
    decode steps (new query, key and value copied into the captured buffers
    before each replay) equals the same 300 steps run eagerly: every step's
    attention output and the final ring, pool, chunk sums and lengths bit
    for bit; with the block manager also its tables and free stack."""
    B, Hq, Hkv, d, T0, W, C, p, steps = 2, 16, 2, 128, 1200, 64, 32, 0.9, 300
    desc, st_g = _lifecycle(gpu, 21, B, Hq, Hkv, d, T0, W, C, p, steps, pool_block)
    _, st_e = _lifecycle(gpu, 21, B, Hq, Hkv, d, T0, W, C, p, steps, pool_block)
    ws_g, ws_e = H.alloc_workspace(desc, gpu), H.alloc_workspace(desc, gpu)
    q = torch.zeros((B, Hq, d), dtype=torch.bfloat16, device=gpu)
    kn = torch.zeros((B, Hkv, d), dtype=torch.bfloat16, device=gpu)
    vn = torch.zeros_like(kn)
    out_g = torch.empty((B, Hq, d), device=gpu)
    out_e = torch.empty_like(out_g)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):  # recorded only: the state is not advanced here
        H.step_inplace(desc, q, kn, vn, None, st_g, out_g, ws_g)
    torch.cuda.synchronize()
    gen = torch.Generator(device=gpu).manual_seed(22)
    for s in range(steps):
        q.copy_((torch.randn(q.shape, generator=gen, device=gpu) * 1.5).to(q.dtype))
        kn.copy_(torch.randn(kn.shape, generator=gen, device=gpu).to(kn.dtype))
        vn.copy_(torch.randn(vn.shape, generator=gen, device=gpu).to(vn.dtype))
        g.replay()
        H.step_inplace(desc, q, kn, vn, None, st_e, out_e, ws_e)
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), s
    assert torch.equal(st_g.seq_len, st_e.seq_len)
    assert int(st_g.seq_len[0]) == T0 + steps
    assert torch.equal(st_g.ring_k, st_e.ring_k) and torch.equal(st_g.ring_v, st_e.ring_v)
    tg, te = st_g.tiers, st_e.tiers
    assert torch.equal(tg.count, te.count)
    for b in range(B):
        for h in range(Hkv):
            n = int(te.count[b, h])
            assert torch.equal(tg.pos[b, h, :n], te.pos[b, h, :n])
            assert torch.equal(st_g.pool_rows(b, h, "k"), st_e.pool_rows(b, h, "k"))
            assert torch.equal(st_g.pool_rows(b, h, "v"), st_e.pool_rows(b, h, "v"))
    if pool_block:
        assert torch.equal(st_g.pool_table, st_e.pool_table)
        assert torch.equal(st_g.free_top, st_e.free_top)
        top = int(st_e.free_top.item())
        assert torch.equal(st_g.free_ids[:top], st_e.free_ids[:top])
        assert st_e.blocks_held() + top == st_e.free_ids.numel()
    assert torch.equal(tg.ccount, te.ccount)
    assert torch.equal(tg.ksum, te.ksum) and torch.equal(tg.vsum, te.vsum)
    # tokens kept flowing into the condensed tier over the replays
    assert int(tg.ccount.sum()) > B * Hkv * (T0 - W) // 4
    print("pool after", steps, "steps:", te.count.tolist(), file=sys.stderr, flush=True)


def test_lifecycle_graph_replayed_10000_steps(gpu):
    """One capture of hardkv_step_inplace replayed for 10000 consecutive
    decode steps (the pages stress graph compatibility over tens of
    thousands of decoding steps) against the same steps run eagerly: every
    step's attention output and the final state bit for bit.  The inputs of
    all steps are drawn up front and copied into the captured buffers before
    each replay; outputs are kept per step and compared at the end."""
    B, Hq, Hkv, d, T0, W, C, p, steps = 2, 16, 2, 128, 700, 64, 32, 0.9, 10000
    desc, st_g = _lifecycle(gpu, 31, B, Hq, Hkv, d, T0, W, C, p, steps)
    _, st_e = _lifecycle(gpu, 31, B, Hq, Hkv, d, T0, W, C, p, steps)
    ws_g, ws_e = H.alloc_workspace(desc, gpu), H.alloc_workspace(desc, gpu)
    gen = torch.Generator(device=gpu).manual_seed(32)
    Q = (torch.randn((steps, B, Hq, d), generator=gen, device=gpu) * 1.5).to(torch.bfloat16)
    KN = torch.randn((steps, B, Hkv, d), generator=gen, device=gpu).to(torch.bfloat16)
    VN = torch.randn((steps, B, Hkv, d), generator=gen, device=gpu).to(torch.bfloat16)
    q = torch.zeros_like(Q[0])
    kn = torch.zeros_like(KN[0])
    vn = torch.zeros_like(VN[0])
    out_g = torch.empty((B, Hq, d), device=gpu)
    outs_g = torch.empty((steps, B, Hq, d), device=gpu)
    outs_e = torch.empty_like(outs_g)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):  # recorded only: the state is not advanced here
        H.step_inplace(desc, q, kn, vn, None, st_g, out_g, ws_g)
    torch.cuda.synchronize()
    for s in range(steps):
        q.copy_(Q[s])
        kn.copy_(KN[s])
        vn.copy_(VN[s])
        g.replay()
        outs_g[s].copy_(out_g)
        H.step_inplace(desc, Q[s], KN[s], VN[s], None, st_e, outs_e[s], ws_e)
        if s % 2000 == 1999:
            torch.cuda.synchronize()
            print(f"replayed {s + 1} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    same = (outs_g.view(steps, -1).view(torch.int32) == outs_e.view(steps, -1).view(torch.int32)).all(1)
    assert bool(same.all()), f"first differing step {int((~same).nonzero()[0])}"
    assert int(st_g.seq_len[0]) == T0 + steps and torch.equal(st_g.seq_len, st_e.seq_len)
    assert torch.equal(st_g.ring_k, st_e.ring_k) and torch.equal(st_g.ring_v, st_e.ring_v)
    tg, te = st_g.tiers, st_e.tiers
    assert torch.equal(tg.count, te.count)
    assert torch.equal(tg.ccount, te.ccount)
    assert torch.equal(tg.ksum, te.ksum) and torch.equal(tg.vsum, te.vsum)
    for b in range(B):
        for h in range(Hkv):
            n = int(te.count[b, h])
            assert torch.equal(tg.pos[b, h, :n], te.pos[b, h, :n])
            assert torch.equal(tg.k[b, h, :n], te.k[b, h, :n])
    # every token is in exactly one tier after 10000 steps
    tot = te.count.long() + te.ccount.long().sum(-1) + W
    assert torch.all(tot == T0 + steps)
    print("pool after", steps, "steps:", te.count.tolist(), file=sys.stderr, flush=True)
