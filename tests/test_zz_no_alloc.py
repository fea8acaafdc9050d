"""hardkv_step_noalloc (the library-held workspace) against hardkv_step with
a caller workspace: two calls in a row, the second on a smaller input, each
compared with the plain step on the same inputs.  Both run the same kernels
in the same order, so every tier and the attention output must match bit
for bit (the comparison rules of the oracle tests are looser)."""
import sys

import pytest
import torch

from decode_kv_cache_head_amd import hardkv as H
from decode_kv_cache_head_amd import synth as S

from parity import cache_of, desc_for

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _assert_same_tiers(case, desc, a, b):
    w = case.w
    assert torch.equal(a.count, b.count)
    A = torch.clamp(case.ctx_len.long() - w.W - w.sinks, min=0)
    for bb in range(w.B):
        nch = -(-int(A[bb]) // w.C)
        assert torch.equal(a.ccount[bb, :, :nch], b.ccount[bb, :, :nch])
        assert torch.equal(a.ksum[bb, :, :nch].view(torch.int32), b.ksum[bb, :, :nch].view(torch.int32))
        assert torch.equal(a.vsum[bb, :, :nch].view(torch.int32), b.vsum[bb, :, :nch].view(torch.int32))
        for h in range(w.Hkv):
            n = int(a.count[bb, h])
            assert torch.equal(a.pos[bb, h, :n], b.pos[bb, h, :n])
            bits = torch.int16 if a.k.dtype == torch.bfloat16 else torch.int32
            assert torch.equal(a.k[bb, h, :n].view(bits), b.k[bb, h, :n].view(bits))
            assert torch.equal(a.v[bb, h, :n].view(bits), b.v[bb, h, :n].view(bits))


def _compare(case):
    w = case.w
    dev = case.q.device
    desc = desc_for(case)
    assert H.workspace_size(desc) <= H.SCRATCH_BYTES
    ref_t = H.alloc_tiers(desc, dev)
    ref_o = torch.empty((w.B, w.Hq, w.d), device=dev)
    H.step(desc, case.q, cache_of(case), case.metric, ref_t, ref_o, H.alloc_workspace(desc, dev))
    t = H.alloc_tiers(desc, dev)
    o = torch.full((w.B, w.Hq, w.d), float("nan"), device=dev)
    H.step_noalloc(desc, case.q, cache_of(case), case.metric, t, o)
    torch.cuda.synchronize()
    _assert_same_tiers(case, desc, ref_t, t)
    assert torch.equal(ref_o.view(torch.int32), o.view(torch.int32))
    say(w.name, "kept", int(t.count.sum()), "of", int(torch.clamp(case.ctx_len.long() - w.W, min=0).sum()) * w.Hkv)


def test_noalloc_step_matches_step_twice(gpu):
    # first call: the headline shape (54 MiB of the 64 MiB array)
    big = S.workload("qwen8b_b32_16k_paged")
    say("noalloc call 1:", big.name)
    _compare(S.make_case(big, gpu))
    # second call: a smaller, ragged batch with key-norm heads; the array
    # still holds the first call's scores, masks and partials
    small = S.Workload("noalloc_small", 3, 16, 2, 128, (2100, 777, 40), S.DT_BF16, 64, 64, 0.9,
                       metric=(S.METRIC_QK, S.METRIC_L2))
    say("noalloc call 2:", small.name)
    _compare(S.make_case(small, gpu))


def test_noalloc_step_refuses_an_oversized_workspace(gpu):
    w = S.workload("qwen8b_b32_ragged_paged")
    case = S.make_case(S.workload("qwen8b_b32_ragged_paged", B=1, T=(512,)), gpu)
    desc = desc_for(case)
    big = H.make_desc(w.B, w.Hq, w.Hkv, w.d, w.dtype, w.W, w.C, w.p, 32768, 16, 2048)
    assert H.workspace_size(big) > H.SCRATCH_BYTES
    t = H.alloc_tiers(desc, gpu)
    o = torch.empty((1, w.Hq, w.d), device=gpu)
    with pytest.raises(H.HardKVError) as e:
        H.step_noalloc(big, case.q, cache_of(case), None, t, o)
    assert e.value.code == H.ERR_WORKSPACE
