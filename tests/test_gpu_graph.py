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
