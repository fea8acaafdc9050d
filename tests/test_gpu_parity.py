"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small cases check every (b, h) and every stage.  At full size the product
call hardkv_step is compared with the oracle on every head of the headline,
ragged and 64k workloads; the stage-by-stage calls and the option variants
on sampled heads, with cheap invariants on every head.
Comparison rules: tests/parity.py.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle as O
from decode_kv_cache_head_amd import hardkv as H
from decode_kv_cache_head_amd import synth as S

from parity import (cache_of, check_all_heads_invariants, check_case, desc_for, oracle_head,
                    run_stages, run_step)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def small(name, **kw):
    base = dict(name=name, B=3, Hq=8, Hkv=2, d=128, T=(2100, 777, 40), dtype=S.DT_BF16, W=64,
                C=64, p=0.9)
    base.update(kw)
    return S.Workload(**base)


def test_tiny_workload(gpu):
    w = S.workload("tiny")
    case = S.make_case(w, gpu)
    desc = desc_for(case)
    say("tiny", w)
    g = run_stages(case, desc)
    rep = check_case(case, g, w.p)
    say(rep)
    assert rep["heads"] == 2 and rep["selected"] > 0
    # the planted heavy keys are kept
    for h in range(w.Hkv):
        kept = set(g["tiers"].pos[0, h, :int(g["tiers"].count[0, h])].tolist())
        assert set(case.extra[("planted", 0, h)]) <= kept


GRID = [
    dict(dtype=S.DT_BF16, d=128, Hq=8, Hkv=2, C=64, p=0.9),
    dict(dtype=S.DT_BF16, d=128, Hq=8, Hkv=2, C=64, p=0.5, block_size=16),
    dict(dtype=S.DT_BF16, d=64, Hq=8, Hkv=8, C=32, p=0.95),
    dict(dtype=S.DT_F32, d=128, Hq=4, Hkv=2, C=7, p=0.8),
    dict(dtype=S.DT_F32, d=64, Hq=16, Hkv=2, C=100, p=0.99, block_size=32),
    dict(dtype=S.DT_BF16, d=128, Hq=16, Hkv=2, C=1, p=0.7, metric=(S.METRIC_QK, S.METRIC_L2)),
    dict(dtype=S.DT_BF16, d=128, Hq=8, Hkv=4, C=64, p=0.9,
         metric=(S.METRIC_L2, S.METRIC_QK, S.METRIC_L2, S.METRIC_L2), block_size=16),
    dict(dtype=S.DT_F32, d=128, Hq=8, Hkv=2, C=128, p=0.9, T=(3000, 1100, 200)),
    dict(dtype=S.DT_BF16, d=64, Hq=8, Hkv=1, C=64, p=0.85, block_size=64),
    dict(dtype=S.DT_F32, d=64, Hq=4, Hkv=4, C=192, p=0.6, T=(2500, 1000, 70)),
    dict(dtype=S.DT_BF16, d=128, Hq=8, Hkv=2, C=1024, p=0.9, T=(2600, 1300, 1090)),
    # attention sinks and attention-weighted merging
    dict(dtype=S.DT_BF16, d=128, Hq=8, Hkv=2, C=64, p=0.9, sinks=4, merge=1, block_size=16),
    dict(dtype=S.DT_F32, d=64, Hq=4, Hkv=2, C=7, p=0.8, sinks=37, merge=1),
    dict(dtype=S.DT_BF16, d=128, Hq=16, Hkv=2, C=128, p=0.7, sinks=300,
         metric=(S.METRIC_QK, S.METRIC_L2)),
    dict(dtype=S.DT_BF16, d=64, Hq=8, Hkv=4, C=64, p=0.95, sinks=1, merge=1,
         metric=(S.METRIC_L2, S.METRIC_QK, S.METRIC_L2, S.METRIC_QK)),
    dict(dtype=S.DT_BF16, d=128, Hq=8, Hkv=2, C=192, p=0.6, merge=1, T=(2500, 1000, 400)),
    # observation-window metric (pooled max over earlier queries)
    dict(dtype=S.DT_BF16, d=128, Hq=8, Hkv=2, C=64, p=0.9, block_size=16,
         metric=(S.METRIC_WINDOW, S.METRIC_QK), obs_window=4, pool_radius=3),
    dict(dtype=S.DT_F32, d=64, Hq=8, Hkv=4, C=7, p=0.8, obs_window=2,
         metric=(S.METRIC_WINDOW, S.METRIC_L2, S.METRIC_WINDOW, S.METRIC_QK)),
    dict(dtype=S.DT_BF16, d=128, Hq=16, Hkv=2, C=128, p=0.95, pool_radius=5,
         metric=(S.METRIC_WINDOW, S.METRIC_WINDOW)),
    dict(dtype=S.DT_BF16, d=64, Hq=8, Hkv=1, C=64, p=0.7, obs_window=8, pool_radius=64, merge=1,
         sinks=3, metric=(S.METRIC_WINDOW,)),
    dict(dtype=S.DT_BF16, d=128, Hq=8, Hkv=2, C=64, p=0.9, metric=(S.METRIC_WINDOW, S.METRIC_QK)),
    # entropy-matched calibration of key-norm and window heads
    dict(dtype=S.DT_BF16, d=128, Hq=8, Hkv=2, C=64, p=0.9, metric=(S.METRIC_L2, S.METRIC_QK),
         calibration=1),
    dict(dtype=S.DT_F32, d=64, Hq=8, Hkv=4, C=7, p=0.8, obs_window=2, calibration=1,
         metric=(S.METRIC_WINDOW, S.METRIC_L2, S.METRIC_WINDOW, S.METRIC_QK)),
    dict(dtype=S.DT_BF16, d=128, Hq=8, Hkv=2, C=64, p=0.95, T=(9000, 5000, 300),
         metric=(S.METRIC_L2, S.METRIC_L2), calibration=1),
    dict(dtype=S.DT_BF16, d=128, Hq=8, Hkv=2, C=64, p=0.9, block_size=16, sinks=4, merge=1,
         metric=(S.METRIC_WINDOW, S.METRIC_L2), obs_window=4, pool_radius=3, calibration=1),
    # key-dissimilarity heads (the candidates' key sum formed before the score)
    dict(dtype=S.DT_BF16, d=128, Hq=8, Hkv=2, C=64, p=0.9, metric=(S.METRIC_KEYDIFF, S.METRIC_QK)),
    dict(dtype=S.DT_F32, d=64, Hq=8, Hkv=4, C=7, p=0.8, obs_window=2, calibration=1,
         metric=(S.METRIC_KEYDIFF, S.METRIC_L2, S.METRIC_WINDOW, S.METRIC_KEYDIFF)),
    dict(dtype=S.DT_BF16, d=128, Hq=16, Hkv=2, C=64, p=0.95, block_size=16, sinks=4, merge=1,
         T=(9000, 2100, 300), metric=(S.METRIC_KEYDIFF, S.METRIC_KEYDIFF)),
    dict(dtype=S.DT_BF16, d=64, Hq=8, Hkv=2, C=32, p=0.7, calibration=1,
         metric=(S.METRIC_QK, S.METRIC_KEYDIFF)),
    # R-KV redundancy heads (the candidates' unit-key sum formed before the score)
    dict(dtype=S.DT_BF16, d=128, Hq=8, Hkv=2, C=64, p=0.9, metric=(S.METRIC_RKV, S.METRIC_QK)),
    dict(dtype=S.DT_F32, d=64, Hq=8, Hkv=4, C=7, p=0.8, calibration=1,
         metric=(S.METRIC_RKV, S.METRIC_KEYDIFF, S.METRIC_L2, S.METRIC_RKV)),
    dict(dtype=S.DT_BF16, d=128, Hq=16, Hkv=2, C=64, p=0.95, block_size=16, sinks=4, merge=1,
         T=(9000, 2100, 300), metric=(S.METRIC_RKV, S.METRIC_RKV)),
    dict(dtype=S.DT_BF16, d=64, Hq=8, Hkv=2, C=32, p=0.7, T=(2100, 777, 2),
         metric=(S.METRIC_QK, S.METRIC_RKV)),
    # block-granular selection: whole position-aligned blocks ranked by mass
    dict(dtype=S.DT_BF16, d=128, Hq=8, Hkv=2, C=64, p=0.9, block_size=16, select_block=16),
    dict(dtype=S.DT_F32, d=64, Hq=8, Hkv=4, C=7, p=0.8, select_block=8, sinks=5,
         metric=(S.METRIC_L2, S.METRIC_QK, S.METRIC_RKV, S.METRIC_QK)),
    dict(dtype=S.DT_BF16, d=128, Hq=16, Hkv=2, C=64, p=0.95, block_size=16, select_block=64,
         merge=1, T=(9000, 2100, 300)),
    dict(dtype=S.DT_BF16, d=64, Hq=8, Hkv=2, C=32, p=0.6, select_block=1, calibration=1,
         metric=(S.METRIC_QK, S.METRIC_L2)),
]


@pytest.mark.parametrize("i", range(len(GRID)))
def test_small_grid_all_heads_all_stages(gpu, i):
    w = small(f"grid{i}", **GRID[i])
    say("grid", i, w)
    case = S.make_case(w, gpu)
    desc = desc_for(case)
    g = run_stages(case, desc)
    rep = check_case(case, g, w.p)
    say(rep)
    check_all_heads_invariants(case, desc, g)
    # the fused hardkv_step (its own launches) against the oracle too
    s = run_step(case, desc)
    check_all_heads_invariants(case, desc, s)
    rep2 = check_case(case, s, w.p, stages=False)
    say("step", rep2)


def test_p_one_is_full_attention(gpu):
    w = small("pone", p=1.0, T=(1500, 300, 65))
    case = S.make_case(w, gpu)
    desc = desc_for(case)
    g = run_step(case, desc)
    for b in range(w.B):
        assert torch.equal(g["tiers"].count[b].long(),
                           torch.full((w.Hkv,), max(w.T[b] - w.W, 0), device=gpu))
        for h in range(w.Hkv):
            G = w.G
            q = case.q[b, h * G:(h + 1) * G].double().cpu()
            K = S.head_rows(case, b, h, "k").double().cpu()
            V = S.head_rows(case, b, h, "v").double().cpu()
            ref = torch.nn.functional.scaled_dot_product_attention(
                q[None, :, None], K[None, None].expand(1, G, -1, -1).contiguous(),
                V[None, None].expand(1, G, -1, -1).contiguous())[0, :, 0]
            o = g["out"][b, h * G:(h + 1) * G].double().cpu()
            err = ((o - ref).abs().amax(1) / ref.abs().amax(1)).max().item()
            assert err <= 2e-3, err


ROW_TILE_CASES = [
    dict(Hq=16, Hkv=2),                                   # G = 8
    dict(Hq=8, Hkv=2, block_size=16),                     # G = 4, paged rows
    dict(Hq=16, Hkv=2, peaked_heads=(0,), temp_range=(0.3, 0.5)),
    dict(Hq=8, Hkv=2, peaked_heads=(1,), block_size=16),
]


@pytest.mark.parametrize("i", range(len(ROW_TILE_CASES)))
def test_row_tiles_ragged_and_peaked_full_attention(gpu, i):
    """bf16 rows with d = 128 and G >= 4 (the matrix-core attention): tier
    lengths that end at every offset of a 32-entry step, a 64- and 128-entry
    wave and a 256- and 512-entry tile, flat and peaked heads (Zipf-planted
    keys with logits up to 24 above the rest).  p = 1 keeps every token, so
    the output is full attention (float64 SDPA), both from the step (the
    kept rows attended inside the compaction pass) and from a standalone
    attention call over the step's tiers (the kept rows in 512-entry tiles).
    Bound 1e-4 of max|o|: each weight enters the value product as a bf16 pair
    whose sum is within 2^-18 of it, products of bf16 values are exact in
    float32 and the float32 sums run over at most 1300 terms."""
    W = 64
    T = (40,) + tuple(W + n for n in (1, 31, 32, 33, 63, 65, 127, 129, 255, 257, 511, 513, 1000,
                                      1240))
    w = small(f"rowtiles{i}", B=len(T), T=T, W=W, p=1.0, **ROW_TILE_CASES[i])
    say("row tiles", w)
    case = S.make_case(w, gpu)
    desc = desc_for(case)
    ws = H.alloc_workspace(desc, gpu)
    g = run_step(case, desc, ws=ws)
    alone = torch.full_like(g["out"], float("nan"))
    H.decode_attn(desc, case.q, cache_of(case), g["tiers"], alone, ws)
    torch.cuda.synchronize()
    worst = 0.0
    for b in range(w.B):
        for h in range(w.Hkv):
            G = w.G
            q = case.q[b, h * G:(h + 1) * G].double().cpu()
            K = S.head_rows(case, b, h, "k").double().cpu()
            V = S.head_rows(case, b, h, "v").double().cpu()
            ref = torch.nn.functional.scaled_dot_product_attention(
                q[None, :, None], K[None, None].expand(1, G, -1, -1).contiguous(),
                V[None, None].expand(1, G, -1, -1).contiguous())[0, :, 0]
            for name, res in (("step", g["out"]), ("decode_attn", alone)):
                o = res[b, h * G:(h + 1) * G].double().cpu()
                err = ((o - ref).abs().amax(1) / ref.abs().amax(1)).max().item()
                worst = max(worst, err)
                assert err <= 1e-4, (name, b, h, err)
    say("worst relative error", worst)


@pytest.mark.parametrize("Hq", [8, 16])
def test_condensed_tier_attention_precision(gpu, Hq):
    """Most of the mass in the condensed tier (p = 0.3, C = 16, G = 4 and 8):
    the GPU's attention against the oracle's float64 attention over the
    GPU's own tiers, so only the attention arithmetic is compared.  Bound
    1e-4 of max|o|: chunk sums and weights enter the matrix products as two
    bf16 terms each (relative error below 2^-17 per element), which moves a
    chunk logit by about 1e-5."""
    w = small(f"chunkprec{Hq}", Hq=Hq, Hkv=2, C=16, p=0.3, T=(4000, 1500, 300))
    case = S.make_case(w, gpu)
    desc = desc_for(case)
    g = run_step(case, desc)
    tiers = g["tiers"]
    G = w.G
    worst = 0.0
    for b in range(w.B):
        for h in range(w.Hkv):
            T = w.T[b]
            A = max(T - w.W, 0)
            nch = -(-A // w.C)
            q = case.q[b, h * G:(h + 1) * G].double().cpu().numpy()
            K = S.head_rows(case, b, h, "k").double().cpu().numpy()
            V = S.head_rows(case, b, h, "v").double().cpu().numpy()
            k = int(tiers.count[b, h])
            pos = tiers.pos[b, h, :k].long().cpu().numpy()
            ks = tiers.ksum[b, h, :nch].double().cpu().numpy()
            vs = tiers.vsum[b, h, :nch].double().cpu().numpy()
            cc = tiers.ccount[b, h, :nch].cpu().numpy()
            dense = O.dense_positions(T, 0, A)
            ref = O.attend_head(q, K[dense], V[dense], K[pos], V[pos], ks, vs, cc)
            o = g["out"][b, h * G:(h + 1) * G].double().cpu().numpy()
            err = float((np.abs(o - ref).max(1) / np.abs(ref).max(1)).max())
            worst = max(worst, err)
            assert err <= 1e-4, (b, h, err)
    say("worst relative error", worst)


def test_score_filter_with_tied_and_near_tied_query_heads(gpu):
    """The matrix-core score filter (bf16, d = 128, G = 8, no metric array):
    KV head 0's query heads come in identical pairs, so every token has at
    least two candidate heads; head 1's pairs differ in one element by one
    bf16 step, so their float32 dots sit within the filter's band and the
    float64 dots decide.  Logits must equal the oracle's float64 maximum
    under the usual rule (at most 1 ulp, on a tiny fraction)."""
    w = small("scorefilter", Hq=16, Hkv=2, T=(6000, 2500, 700), p=0.9)
    case = S.make_case(w, gpu)
    q = case.q.clone()
    G = w.G
    for b in range(w.B):
        for j in range(0, G, 2):
            q[b, j + 1] = q[b, j]                      # head 0: exact ties
            q[b, G + j + 1] = q[b, G + j]              # head 1: one element one bf16 step up
            e = (7 * j) % w.d
            bits = q[b, G + j + 1, e].view(torch.int16) + 1
            q[b, G + j + 1, e] = bits.view(torch.bfloat16)
    case.q.copy_(q)
    desc = desc_for(case)
    g = run_stages(case, desc)
    rep = check_case(case, g, w.p)
    say(rep)
    assert rep["logit_1ulp"] <= 0.001 * rep["candidates"]


@pytest.mark.parametrize("Hq", [8, 16])
@pytest.mark.parametrize("e", [63, -60])
def test_score_filter_outside_float32_range(gpu, e, Hq):
    """Queries and keys scaled by 2^e (exact in bf16).  At e = 63 the
    products reach 2^126 and their float32 sums overflow; at e = -60 the
    products are float32 subnormals (2^-120).  At G = 8 (the matrix-core
    filter) the filter's float32 band is then no bound and every head must
    stay a candidate; at G = 4 the score is float64 throughout.  Either way
    the logits must equal the oracle's float64 maximum (at most 1 ulp, on a
    tiny fraction; equal infinities where the maximum leaves float32's
    range)."""
    w = small(f"scorerange{e}_{Hq}", Hq=Hq, Hkv=2, B=2, T=(3000, 700), p=0.9)
    case = S.make_case(w, gpu)
    f = 2.0 ** e
    case.q.mul_(f)
    case.k.mul_(f)
    desc = desc_for(case)
    shape = (w.B, w.Hkv, desc.sparse_cap)
    logit = torch.full(shape, float("nan"), device=gpu)
    l2 = torch.full(shape, float("nan"), device=gpu)
    ws = H.alloc_workspace(desc, gpu)
    H.score(desc, case.q, cache_of(case), case.metric, logit, l2, ws)
    torch.cuda.synchronize()
    G, n_ulp, n_all = w.G, 0, 0
    for b in range(w.B):
        A = max(w.T[b] - w.W, 0)
        for h in range(w.Hkv):
            q = case.q[b, h * G:(h + 1) * G].float().cpu().numpy()
            K = S.head_rows(case, b, h, "k").float().cpu().numpy()[:A]
            with np.errstate(over="ignore"):
                ref, _ = O.score_head(q, K)
            got = logit[b, h, :A].cpu().numpy()
            inf = np.isinf(ref)
            assert np.array_equal(np.isinf(got), inf), (b, h)
            assert np.array_equal(got[inf], ref[inf]), (b, h)
            ia = got[~inf].view(np.int32).astype(np.int64)
            ib = ref[~inf].view(np.int32).astype(np.int64)
            diff = np.abs(ia - ib)
            assert diff.max(initial=0) <= 1, (b, h, diff.max())
            n_ulp += int((diff == 1).sum())
            n_all += A
    say("1-ulp logits", n_ulp, "of", n_all)
    assert n_ulp <= 0.001 * n_all


def test_selection_beyond_65536_candidates(gpu):
    """Heads of 139936 candidates (more than 2^17): the selection's
    fixed-point masses take 2^-45 units there, so a head's total stays within
    2^63.  Sequence 0's keys are one row repeated: every weight is 1 (in
    2^-47 units the total would pass 2^64) and the kept set is the first
    ceil(p n) positions.  Sequence 1 is N(0, 1).  Both against the oracle."""
    w = small("longheads", B=2, T=(140000, 140000), p=0.9)
    case = S.make_case(w, gpu)
    for h in range(w.Hkv):
        case.k[0, h, :w.T[0]] = case.k[0, h, :1].clone()
    desc = desc_for(case)
    g = run_stages(case, desc)
    rep = check_case(case, g, w.p)
    say(rep)
    n = w.T[0] - w.W
    k = math.ceil(float(np.float32(w.p)) * n)
    for h in range(w.Hkv):
        assert int(g["tiers"].count[0, h]) == k
        pos = g["tiers"].pos[0, h, :k].cpu().numpy()
        assert np.array_equal(pos, np.arange(k)), h


def test_edge_cases(gpu):
    # every sequence shorter than the window, a single-token context, and a
    # context exactly one token past the window
    w = small("edge", T=(1, 64, 65, 63), B=4, p=0.6)
    case = S.make_case(w, gpu)
    desc = desc_for(case)
    g = run_stages(case, desc)
    rep = check_case(case, g, w.p)
    assert rep["candidates"] == 2  # only the 65-token sequence ages one token (x2 heads)
    # a window of zero: everything is a candidate
    w0 = small("w0", T=(300, 129), B=2, W=0, C=16, p=0.9)
    c0 = S.make_case(w0, gpu)
    check_case(c0, run_stages(c0, desc_for(c0)), w0.p)


@pytest.mark.parametrize("p", [0.5, 0.93])
def test_tied_scores_take_the_lowest_positions(gpu, p):
    """Keys copied from 5 rows: every score is shared by hundreds of tokens,
    so the top-p cutoff falls inside a group of equal scores, and the oracle
    takes that group's lowest positions first.  The selected positions must
    equal the oracle's exactly (no borderline allowance), through the
    standalone calibrate + select and through the fused step."""
    w = small("ties", T=(9000, 1500, 700), p=p)  # 8936 candidates: 16 per thread
    case = S.make_case(w, gpu)
    g = torch.Generator().manual_seed(11)
    for b in range(w.B):
        for h in range(w.Hkv):
            rows = case.k[b, h, :5].clone()
            idx = torch.randint(0, 5, (w.T[b],), generator=g).to(gpu)
            case.k[b, h, :w.T[b]] = rows[idx]
    desc = desc_for(case)
    st = run_stages(case, desc)
    sp = run_step(case, desc)
    strict = 0
    for b in range(w.B):
        for h in range(w.Hkv):
            _, _, _, ref = oracle_head(case, b, h, p)
            A = ref.A
            if A == 0 or not np.array_equal(st["logit"][b, h, :A].cpu().numpy(), ref.ell):
                continue  # a 1-ulp score difference: the ordinary rules apply (check_case)
            assert len(np.unique(ref.ell)) <= 5
            for run in (st, sp):
                k = int(run["tiers"].count[b, h])
                pos = run["tiers"].pos[b, h, :k].cpu().numpy()
                assert np.array_equal(pos, ref.pos), (b, h, k, ref.sel.k)
            strict += 1
    say("heads checked strictly", strict)
    assert strict >= 4
    check_case(case, st, p)
    check_case(case, sp, p, stages=False)


def test_capacity_larger_than_needed(gpu):
    w = small("cap", T=(900, 500), B=2)
    case = S.make_case(w, gpu)
    desc = desc_for(case, sparse_cap=2000, chunk_cap=64)
    g = run_stages(case, desc)
    check_case(case, g, w.p)


def test_determinism(gpu):
    w = small("det", T=(3000, 2500, 1999), metric=(S.METRIC_QK, S.METRIC_L2))
    case = S.make_case(w, gpu)
    desc = desc_for(case)
    a = run_stages(case, desc)
    b = run_stages(case, desc)
    for f in ("logit", "stats", "mask", "count"):
        x, y = a[f], b[f]
        if f == "mask":
            for bb in range(w.B):
                A = max(w.T[bb] - w.W, 0)
                assert torch.equal(x[bb, :, :A], y[bb, :, :A])
        elif f == "logit":
            for bb in range(w.B):
                A = max(w.T[bb] - w.W, 0)
                assert torch.equal(x[bb, :, :A], y[bb, :, :A])
        else:
            assert torch.equal(x, y)
    for f in ("ksum", "vsum", "ccount"):
        for bb in range(w.B):
            nch = -(-max(w.T[bb] - w.W, 0) // w.C)
            assert torch.equal(getattr(a["tiers"], f)[bb, :, :nch], getattr(b["tiers"], f)[bb, :, :nch])
    assert torch.equal(a["out"], b["out"])


def test_budget_adapts_per_head_qwen8b_b1_16k(gpu):
    """Single-layer Qwen3-8B shape, batch 1, 16k context, per-head query
    temperature in [0.5, 4]: every head against the oracle."""
    w = S.workload("qwen8b_b1_16k")
    say(w)
    case = S.make_case(w, gpu)
    desc = desc_for(case)
    g = run_stages(case, desc)
    rep = check_case(case, g, w.p)
    say(rep)
    budgets = g["tiers"].count[0].float() / (w.T[0] - w.W)
    assert budgets.max() - budgets.min() > 0.15   # head-adaptive


def _sample_heads(w, n, seed):
    rng = np.random.default_rng(seed)
    heads = {(0, 0), (w.B - 1, w.Hkv - 1)}
    while len(heads) < n:
        heads.add((int(rng.integers(w.B)), int(rng.integers(w.Hkv))))
    return sorted(heads)


def test_headline_b32_16k_paged(gpu):
    """The headline workload at full size through hardkv_step: every one of
    the 256 (sequence, KV head) pairs against the oracle."""
    w = S.workload("qwen8b_b32_16k_paged")
    say(w.name)
    case = S.make_case(w, gpu)
    desc = desc_for(case)
    g = run_step(case, desc)
    check_all_heads_invariants(case, desc, g)
    rep = check_case(case, g, w.p, stages=False)
    say(rep)
    assert rep["heads"] == w.B * w.Hkv


def test_headline_with_sinks_and_weighted_merging(gpu):
    """The headline shape with 4 sink tokens and attention-weighted merging:
    sampled heads against the oracle, invariants on every head."""
    w = S.workload("qwen8b_b32_16k_paged", sinks=4, merge=1)
    say(w.name, "sinks", w.sinks, "merge", w.merge)
    case = S.make_case(w, gpu)
    desc = desc_for(case)
    g = run_step(case, desc)
    check_all_heads_invariants(case, desc, g)
    rep = check_case(case, g, w.p, heads=_sample_heads(w, 6, 2), stages=False)
    say(rep)


def test_headline_with_window_metric(gpu):
    """The headline shape with every KV head on the observation-window
    metric (4 queries, pooling radius 3): sampled heads against the oracle,
    invariants on every head."""
    w = S.workload("qwen8b_b32_16k_paged", metric=(S.METRIC_WINDOW,) * 8, obs_window=4,
                   pool_radius=3)
    say(w.name, "window", w.obs_window, "radius", w.pool_radius)
    case = S.make_case(w, gpu)
    desc = desc_for(case)
    g = run_step(case, desc)
    check_all_heads_invariants(case, desc, g)
    rep = check_case(case, g, w.p, heads=_sample_heads(w, 4, 3), stages=False)
    say(rep)


def test_headline_with_entropy_calibration(gpu):
    """The headline shape with every other KV head on the key norm,
    calibrated by the entropy-matched temperature: sampled heads against the
    oracle, invariants on every head."""
    w = S.workload("qwen8b_b32_16k_paged", metric=(S.METRIC_L2, S.METRIC_QK) * 4, calibration=1)
    say(w.name, "entropy calibration")
    case = S.make_case(w, gpu)
    desc = desc_for(case)
    g = run_step(case, desc)
    check_all_heads_invariants(case, desc, g)
    rep = check_case(case, g, w.p, heads=_sample_heads(w, 6, 4), stages=False)
    say(rep)


def test_headline_with_key_dissimilarity(gpu):
    """The headline shape with half the KV heads on the key-dissimilarity
    metric (spread rule) and the stage-by-stage path: sampled heads against
    the oracle, invariants on every head."""
    w = S.workload("qwen8b_b32_16k_paged", metric=(S.METRIC_QK, S.METRIC_KEYDIFF) * 4)
    say(w.name, "key dissimilarity")
    case = S.make_case(w, gpu)
    desc = desc_for(case)
    g = run_stages(case, desc)
    check_all_heads_invariants(case, desc, g)
    rep = check_case(case, g, w.p, heads=_sample_heads(w, 6, 4))
    say(rep)


def test_headline_with_redundancy(gpu):
    """The headline shape with half the KV heads on the R-KV redundancy
    metric: the product call on every head and the stage-by-stage calls on
    sampled heads against the oracle."""
    w = S.workload("qwen8b_b32_16k_paged", metric=(S.METRIC_RKV, S.METRIC_QK) * 4)
    say(w.name, "redundancy")
    case = S.make_case(w, gpu)
    desc = desc_for(case)
    g = run_step(case, desc)
    check_all_heads_invariants(case, desc, g)
    rep = check_case(case, g, w.p, stages=False)
    say("step", rep)
    assert rep["heads"] == w.B * w.Hkv
    del g
    g = run_stages(case, desc)
    rep = check_case(case, g, w.p, heads=_sample_heads(w, 6, 5))
    say("stages", rep)


def test_block_size_one_equals_token_selection(gpu):
    """Blocks of one position select exactly the token-level set."""
    w = small("blk1", T=(3000, 1500, 700), metric=(S.METRIC_QK, S.METRIC_L2))
    case = S.make_case(w, gpu)
    tok = run_step(case, desc_for(case))
    from dataclasses import replace
    case_b = S.Case(replace(w, select_block=1), case.q, case.k, case.v, case.ctx_len,
                    case.block_table, case.metric, case.ctx_cap, case.max_blocks)
    blk = run_step(case_b, desc_for(case_b))
    assert torch.equal(tok["tiers"].count, blk["tiers"].count)
    for b in range(w.B):
        for h in range(w.Hkv):
            n = int(tok["tiers"].count[b, h])
            assert torch.equal(tok["tiers"].pos[b, h, :n], blk["tiers"].pos[b, h, :n])


@pytest.mark.parametrize("name,bs", [("qwen8b_b32_16k_paged", 16), ("qwen8b_b8_64k_mixed", 16)])
def test_block_selection_full_size(gpu, name, bs):
    """Block-granular selection at full size through hardkv_step, every head
    against the oracle (the 64k heads hold 4081 blocks, near the 4096 cap)."""
    w = S.workload(name, select_block=bs)
    say(w.name, "select_block", bs)
    case = S.make_case(w, gpu)
    desc = desc_for(case)
    g = run_step(case, desc)
    check_all_heads_invariants(case, desc, g)
    rep = check_case(case, g, w.p, stages=False)
    say(rep)
    assert rep["heads"] == w.B * w.Hkv


def test_mixed_metric_64k_entropy_calibration(gpu):
    """65280 candidates per head: the standalone calibrate kernel's entropy
    bisection on flat and peaked key-norm heads."""
    w = S.workload("qwen8b_b8_64k_mixed", calibration=1)
    say(w.name, "entropy calibration")
    case = S.make_case(w, gpu)
    desc = desc_for(case, top_p=0.9)
    g = run_stages(case, desc)
    check_all_heads_invariants(case, desc, g)
    rep = check_case(case, g, 0.9, heads=[(0, 4), (2, 5), (7, 6), (1, 0)])
    say(rep)
    # the peaked key-norm head keeps far fewer tokens than the flat ones
    cnt = g["tiers"].count.float()
    assert cnt[:, 4].max() < 0.5 * cnt[:, [5, 6, 7]].min()


def test_ragged_b32_paged(gpu):
    """Ragged contexts of 8192..32768 tokens in a paged cache.  The product
    call hardkv_step (more than 16384 candidates per head: separate
    calibrate and select launches, up to 32 fused compaction tiles per head)
    is compared with the oracle on all 256 heads; the stage-by-stage calls on
    sampled heads."""
    w = S.workload("qwen8b_b32_ragged_paged")
    say(w.name, w.T[:4])
    assert max(w.T) - w.W > 16384
    case = S.make_case(w, gpu)
    desc = desc_for(case)
    g = run_step(case, desc)
    check_all_heads_invariants(case, desc, g)
    rep = check_case(case, g, w.p, stages=False)
    say("step", rep)
    assert rep["heads"] == w.B * w.Hkv
    del g
    g = run_stages(case, desc)
    check_all_heads_invariants(case, desc, g)
    rep = check_case(case, g, w.p, heads=_sample_heads(w, 8, 2))
    say("stages", rep)


@pytest.mark.parametrize("p", [0.8, 0.9, 0.99])
def test_mixed_metric_64k_step(gpu, p):
    """65280 candidates per head, logit and key-norm heads, peaked and flat:
    the product call hardkv_step (separate calibrate and select launches, 64
    fused compaction tiles per head) against the oracle on all 64 heads."""
    w = S.workload("qwen8b_b8_64k_mixed")
    say(w.name, "p", p)
    case = S.make_case(w, gpu)
    desc = desc_for(case, top_p=p)
    g = run_step(case, desc)
    check_all_heads_invariants(case, desc, g)
    rep = check_case(case, g, p, stages=False)
    say(rep)
    assert rep["heads"] == w.B * w.Hkv
    cnt = g["tiers"].count.float() / (w.T[0] - w.W)
    assert cnt[:, 0].max() < 0.01 and cnt[:, 4].max() < 0.01


def test_mixed_metric_64k_p_sweep(gpu):
    w = S.workload("qwen8b_b8_64k_mixed")
    say(w.name)
    case = S.make_case(w, gpu)
    prev = None
    heads = [(0, 0), (0, 4), (3, 1), (5, 6), (7, 0), (7, 4)]
    for p in (0.8, 0.9, 0.99):
        desc = desc_for(case, top_p=p)
        g = run_stages(case, desc)
        check_all_heads_invariants(case, desc, g)
        rep = check_case(case, g, p, heads=heads)
        say(p, rep)
        A = w.T[0] - w.W
        m = g["mask"][:, :, :A].bool()
        if prev is not None:
            assert not torch.any(prev & ~m)      # S(p1) is inside S(p2)
        prev = m
        cnt = g["tiers"].count.float() / A
        # peaked heads keep far fewer tokens than flat heads
        assert cnt[:, 0].max() < 0.01 and cnt[:, 4].max() < 0.01
        assert cnt[:, [0, 4]].max() < 0.5 * cnt[:, [1, 2, 3, 5, 6, 7]].min()
        del g
