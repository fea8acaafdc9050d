"""Pins of the oracle's attention-sink tokens and attention-weighted merging
(gist.science technical summary, section 2.A: Tier 1 keeps attention sinks,
Tier 3 evicts or merges with weights).  CPU only.

Weighted merging is pinned by a hand-worked chunk, its invariance to the
scale of the weights, the floor, and the reductions in which merging cannot
matter (nothing evicted, one token per chunk, identical tokens per chunk),
which must give full softmax attention.  Sinks are pinned by the tier
partition, the chunk alignment and the same reductions.
"""
import numpy as np
import pytest
import torch

import oracle as O


def bf16(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def sdpa_reference(q, K, V):
    G, d = q.shape
    qt = torch.tensor(np.asarray(q, np.float64))[None, :, None, :]
    kt = torch.tensor(np.asarray(K, np.float64))[None, None].expand(1, G, -1, -1).contiguous()
    vt = torch.tensor(np.asarray(V, np.float64))[None, None].expand(1, G, -1, -1).contiguous()
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, :, 0].numpy()


def _case(seed, T=300, d=32, G=2, scale=1.5):
    rng = np.random.default_rng(seed)
    return (bf16(rng.standard_normal((G, d)) * scale), bf16(rng.standard_normal((T, d))),
            bf16(rng.standard_normal((T, d))))


# ------------------------------------------------------- weighted merging --
def test_weighted_chunk_hand_example():
    # chunk 0 of size 4 holds evicted tokens 0 and 2 with weights 1 and 3:
    # representative key (1*k0 + 3*k2) / 4, stored scaled by n = 2
    K = np.array([[1.0, 0.0], [5.0, 5.0], [0.0, 1.0], [7.0, 7.0]])
    V = np.array([[2.0, 0.0], [9.0, 9.0], [0.0, 2.0], [9.0, 9.0]])
    ks, vs, cnt = O.condense(K, V, [0, 2], np.arange(4), 4, 1, weights=[1.0, 3.0])
    assert cnt.tolist() == [2]
    assert np.allclose(ks[0], [0.5, 1.5]) and np.allclose(vs[0], [1.0, 3.0])
    # mean merging: plain sums
    ks, vs, cnt = O.condense(K, V, [0, 2], np.arange(4), 4, 1)
    assert np.allclose(ks[0], [1.0, 1.0]) and np.allclose(vs[0], [2.0, 2.0])
    # the chunk grid starts at `origin`
    ks, _, cnt = O.condense(K, V, [1, 2], np.arange(4), 2, 2, origin=1)
    assert cnt.tolist() == [2, 0] and np.allclose(ks[0], K[1] + K[2])


def test_weighted_merge_scale_invariant_and_floor():
    rng = np.random.default_rng(1)
    K = rng.standard_normal((40, 8))
    V = rng.standard_normal((40, 8))
    ev = np.arange(0, 40, 3)
    w = rng.random(ev.size) + 0.1
    a = O.condense(K, V, ev, np.arange(40), 8, 5, weights=w)
    b = O.condense(K, V, ev, np.arange(40), 8, 5, weights=w * 1e-30)
    assert all(np.allclose(x, y, rtol=1e-12) for x, y in zip(a, b))
    # the floor: a far-below-maximum weight is e^-60 of the top, never 0
    ww = O.merge_weights(np.array([0.0, -1000.0, -59.0], np.float32), 0.0)
    assert ww[0] == 1.0 and ww[1] == np.exp(-60.0) and ww[2] == np.exp(-59.0)
    # one dominant token per chunk: the chunk is that token, up to e^-60
    c = np.full(40, -500.0, np.float32)
    c[ev[::2]] = 0.0
    ks, _, cnt = O.condense(K, V, ev, np.arange(40), 80, 1, weights=O.merge_weights(c[ev], 0.0))
    dom = ev[::2]
    assert np.allclose(ks[0] / cnt[0], K[dom].mean(axis=0), atol=1e-24)


@pytest.mark.parametrize("S", [0, 5])
def test_weighted_merge_reductions_to_full_attention(S):
    q, K, V = _case(2)
    # nothing evicted
    r = O.step_head(q, K, V, 300, 40, 16, 1.0, O.METRIC_QK, S, O.MERGE_WEIGHTED)
    assert r.cnt.sum() == 0
    assert np.allclose(r.out, sdpa_reference(q, K, V), rtol=1e-12, atol=1e-13)
    # one token per chunk: the weighted mean is the token itself
    for p in (0.4, 0.9):
        r = O.step_head(q, K, V, 300, 40, 1, p, O.METRIC_QK, S, O.MERGE_WEIGHTED)
        assert 0 < r.sel.k < r.A
        assert np.allclose(r.out, sdpa_reference(q, K, V), rtol=1e-12, atol=1e-13)


def test_weighted_merge_chunk_constant_is_full_attention():
    # identical evicted rows within each chunk: any weights give that row
    T, W, C, d, S = 301, 37, 8, 32, 3
    rng = np.random.default_rng(12)
    base_k = bf16(rng.standard_normal((T // C + 2, d)) * 1.3)
    base_v = bf16(rng.standard_normal((T // C + 2, d)))
    K = bf16(rng.standard_normal((T, d)))
    V = bf16(rng.standard_normal((T, d)))
    for t in range(S, T - W):
        K[t] = base_k[(t - S) // C]
        V[t] = base_v[(t - S) // C]
    q = bf16(rng.standard_normal((2, d)) * 2)
    for metric in (O.METRIC_QK, O.METRIC_L2):
        r = O.step_head(q, K, V, T, W, C, 0.6, metric, S, O.MERGE_WEIGHTED)
        assert r.cnt.sum() > 0
        assert np.allclose(r.out, sdpa_reference(q, K, V), rtol=1e-12, atol=1e-13)


def test_weighted_differs_from_mean_and_favours_heavy_tokens():
    q, K, V = _case(3, T=400)
    rm = O.step_head(q, K, V, 400, 40, 16, 0.5, O.METRIC_QK, 0, O.MERGE_MEAN)
    rw = O.step_head(q, K, V, 400, 40, 16, 0.5, O.METRIC_QK, 0, O.MERGE_WEIGHTED)
    assert np.array_equal(rm.pos, rw.pos) and np.array_equal(rm.cnt, rw.cnt)
    assert not np.allclose(rm.ksum, rw.ksum)
    # each weighted chunk key is the weighted mean of its evicted keys
    ev = np.nonzero(rw.mask == 0)[0]
    a = O.merge_weights(rw.cal.c[ev], rw.cal.m)
    for j in range(rw.cnt.size):
        m = (ev // 16) == j
        if m.any():
            want = (a[m, None] * K[ev[m]]).sum(0) / a[m].sum()
            assert np.allclose(rw.ksum[j] / rw.cnt[j], want, rtol=1e-12)


# ------------------------------------------------------------- sinks -------
def test_sinks_zero_is_the_plain_step():
    q, K, V = _case(4)
    a = O.step_head(q, K, V, 300, 40, 16, 0.8, O.METRIC_QK)
    b = O.step_head(q, K, V, 300, 40, 16, 0.8, O.METRIC_QK, 0, O.MERGE_MEAN)
    assert np.array_equal(a.out, b.out) and np.array_equal(a.pos, b.pos)


@pytest.mark.parametrize("S,merge", [(4, O.MERGE_MEAN), (37, O.MERGE_WEIGHTED)])
def test_sinks_partition_and_chunk_alignment(S, merge):
    q, K, V = _case(5, T=500)
    T, W, C = 500, 50, 16
    r = O.step_head(q, K, V, T, W, C, 0.7, O.METRIC_QK, S, merge)
    assert r.A == T - W - S
    dense = O.dense_positions(T, S, r.A)
    ev = S + np.nonzero(r.mask == 0)[0]
    allpos = np.concatenate([dense, r.pos, ev])
    assert np.array_equal(np.sort(allpos), np.arange(T))        # disjoint cover
    assert r.pos.min() >= S and ev.min() >= S                  # sinks stay dense
    assert np.array_equal(dense[:S], np.arange(S))
    # chunk j pools evicted positions [S + jC, S + (j+1)C)
    want = np.bincount((ev - S) // C, minlength=r.cnt.size)
    assert np.array_equal(r.cnt, want)


@pytest.mark.parametrize("S", [3, 64])
def test_sinks_reductions_to_full_attention(S):
    q, K, V = _case(6)
    for C, p in ((16, 1.0), (1, 0.6)):
        r = O.step_head(q, K, V, 300, 40, C, p, O.METRIC_QK, S)
        assert np.allclose(r.out, sdpa_reference(q, K, V), rtol=1e-12, atol=1e-13)
    # sinks and window cover the context: no candidates
    r = O.step_head(q, K, V, 300, 240, 16, 0.5, O.METRIC_QK, 60)
    assert r.A == 0 and r.sel.k == 0
    assert np.allclose(r.out, sdpa_reference(q, K, V), rtol=1e-12, atol=1e-13)
    # reuse after a selection with sinks: the dense tier keeps the sinks
    r = O.step_head(q, K, V, 250, 40, 1, 0.6, O.METRIC_QK, S)
    qn = bf16(np.random.default_rng(7).standard_normal((2, 32)))
    assert np.allclose(O.reuse_head(qn, K, V, 300, r), sdpa_reference(qn, K, V),
                       rtol=1e-12, atol=1e-13)
