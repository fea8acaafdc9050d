"""Pins of the oracle's rewrite-versus-sparse-loading policy and of the
attention that reuses a selection (CPU only).

The pages name a Memory-Time Integral that balances the one-off cost of a
rewrite against the per-step gain, and two budget thresholds L_lower and
L_upper (gist.science technical summary, section 2.C, "Trade-off
Management"), but no formula.  The oracle's reading is pinned here by a
worked example, a break-even closed form derived by hand from the integral,
the degenerate cases whose answer follows without the formula, and the
threshold precedence.  Reuse attention is pinned by its reductions to plain
softmax attention.
"""
import numpy as np
import pytest
import torch

import oracle as O


def bf16(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()


# ------------------------------------------------------------- MTI ---------
def test_mti_worked_example():
    # A = 10 aged rows, k = 2 kept, W = 2, horizon 3 (selection + 2 reuse steps).
    # Sparse: footprint 12 rows throughout.  The selection step moves 3*10 + 2*2
    # = 34 rows, each reuse step 2*(2 + 2) = 8: 12*34 + 12*8 + 12*8 = 600.
    # Rewrite: footprint 12 + 2 = 14 while the copy exists, for 34 + 4 = 38
    # rows of time; then 4 rows for the two reuse steps of 8: 532 + 32 + 32 = 596.
    assert O.mti_head(10, 2, 2, 3) == (596, 600)
    assert O.plan_head(10, 2, 2, O.POLICY_MTI, 3) == O.MODE_REWRITE
    # one reuse step fewer: sparse 12*34 + 96 = 504, rewrite 532 + 32 = 564
    assert O.mti_head(10, 2, 2, 2) == (564, 504)
    assert O.plan_head(10, 2, 2, O.POLICY_MTI, 2) == O.MODE_SPARSE


def _rewrite_by_breakeven(A, k, W, N):
    # Subtracting the two integrals: the rewrite pays, once,
    #   (A + W + k)(3A + 2W + 2k) - (A + W)(3A + 2W) = 2k(A + W) + k(3A + 2W + 2k)
    # and saves (A - k) rows of footprint on each of the N - 1 reuse steps of
    # 2(k + W) rows each.
    once = 2 * k * (A + W) + k * (3 * A + 2 * W + 2 * k)
    per_step = (A - k) * 2 * (k + W)
    return (N - 1) * per_step > once


def test_mti_breakeven_closed_form():
    rng = np.random.default_rng(5)
    for _ in range(3000):
        A = int(rng.integers(0, 40000))
        k = int(rng.integers(0, A + 1))
        W = int(rng.integers(0, 600))
        N = int(rng.integers(1, 80))
        want = O.MODE_REWRITE if _rewrite_by_breakeven(A, k, W, N) else O.MODE_SPARSE
        assert O.plan_head(A, k, W, O.POLICY_MTI, N, l_lower=-1) == want, (A, k, W, N)


def test_mti_degenerate_cases():
    for A, W in [(1, 0), (100, 16), (16128, 256)]:
        for k in range(1, min(A, 50) + 1):
            # no reuse: the rewrite only adds work and memory
            assert O.plan_head(A, k, W, O.POLICY_MTI, 1, l_lower=-1) == O.MODE_SPARSE
        for N in (1, 2, 10, 1000):
            # nothing evicted: a rewrite frees nothing
            assert O.plan_head(A, A, W, O.POLICY_MTI, N, l_lower=-1) == O.MODE_SPARSE
    # nothing kept, a window and at least one reuse step: the footprint drops
    # from A + W to W at no cost
    assert O.plan_head(50, 0, 8, O.POLICY_MTI, 2, l_lower=-1) == O.MODE_REWRITE
    assert O.plan_head(50, 0, 8, O.POLICY_MTI, 1, l_lower=-1) == O.MODE_SPARSE


def test_mti_monotone_in_horizon():
    # once the rewrite pays for a horizon it pays for every longer one
    for A, k, W in [(16128, 13548, 256), (16128, 60, 256), (1000, 999, 0), (5000, 2500, 64)]:
        modes = [O.plan_head(A, k, W, O.POLICY_MTI, N, l_lower=-1) for N in range(1, 400)]
        first = modes.index(O.MODE_REWRITE) if O.MODE_REWRITE in modes else len(modes)
        assert all(m == O.MODE_SPARSE for m in modes[:first])
        assert all(m == O.MODE_REWRITE for m in modes[first:])
    # a near-dense head needs a long reuse horizon, a sparse one almost none
    flat = [O.plan_head(16128, 13548, 256, O.POLICY_MTI, N) for N in range(1, 40)]
    peaked = [O.plan_head(16128, 60, 256, O.POLICY_MTI, N) for N in range(1, 40)]
    assert flat.index(O.MODE_REWRITE) > 10 and peaked.index(O.MODE_REWRITE) == 1


def test_thresholds_override_the_integral():
    A, W = 16128, 256
    # MTI alone: k = 60 rewrites at N = 4, k = 13548 stays sparse
    assert O.plan_head(A, 60, W, O.POLICY_MTI, 4) == O.MODE_REWRITE
    assert O.plan_head(A, 13548, W, O.POLICY_MTI, 4) == O.MODE_SPARSE
    # budget at or above L_upper: sparse; at or below L_lower: rewrite
    assert O.plan_head(A, 60, W, O.POLICY_MTI, 4, l_upper=60) == O.MODE_SPARSE
    assert O.plan_head(A, 13548, W, O.POLICY_MTI, 4, l_lower=13548) == O.MODE_REWRITE
    # L_lower is checked first
    assert O.plan_head(A, 100, W, O.POLICY_MTI, 1, l_lower=100, l_upper=50) == O.MODE_REWRITE
    # fixed policies ignore everything else
    assert O.plan_head(A, 60, W, O.POLICY_SPARSE, 1000) == O.MODE_SPARSE
    assert O.plan_head(A, 13548, W, O.POLICY_REWRITE, 1) == O.MODE_REWRITE
    with pytest.raises(ValueError):
        O.mti_head(10, 11, 0, 1)
    with pytest.raises(ValueError):
        O.mti_head(10, 1, 0, 0)


# ------------------------------------------------------- reuse steps --------
def sdpa_reference(q, K, V):
    G, d = q.shape
    qt = torch.tensor(np.asarray(q, np.float64))[None, :, None, :]
    kt = torch.tensor(np.asarray(K, np.float64))[None, None].expand(1, G, -1, -1).contiguous()
    vt = torch.tensor(np.asarray(V, np.float64))[None, None].expand(1, G, -1, -1).contiguous()
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, :, 0].numpy()


def _seq(seed, T, d=32, G=2):
    rng = np.random.default_rng(seed)
    return (bf16(rng.standard_normal((G, d)) * 1.5), bf16(rng.standard_normal((T, d))),
            bf16(rng.standard_normal((T, d))), bf16(rng.standard_normal((6, G, d)) * 1.5))


def test_reuse_at_selection_length_is_the_step():
    q, K, V, _ = _seq(1, 400)
    r = O.step_head(q, K, V, 300, 40, 16, 0.8, O.METRIC_QK)
    assert np.array_equal(O.reuse_head(q, K, V, 300, r), r.out)


@pytest.mark.parametrize("C,p", [(16, 1.0), (1, 0.7), (1, 0.95)])
def test_reuse_reduces_to_full_attention(C, p):
    # p = 1 keeps every aged token; C = 1 pools each evicted token alone
    # (count 1, bias 0).  Either way every later step attends to the whole
    # context [0, T_now), whatever was selected.
    q, K, V, later = _seq(2, 400)
    r = O.step_head(q, K, V, 300, 40, C, p, O.METRIC_QK)
    if p < 1:
        assert 0 < r.sel.k < r.A
    for i, T_now in enumerate([300, 301, 317, 400]):
        qn = later[i]
        assert np.allclose(O.reuse_head(qn, K, V, T_now, r), sdpa_reference(qn, K[:T_now], V[:T_now]),
                           rtol=1e-12, atol=1e-13)


def test_reuse_dense_tier_grows():
    # The tokens that aged after the selection are attended exactly: with
    # chunk-constant aged rows the pooled tier is exact too, so reuse equals
    # full attention although most aged tokens were evicted.
    T, W, C, d = 260, 20, 8, 32
    rng = np.random.default_rng(3)
    A = T - W
    K = bf16(rng.standard_normal((T + 30, d)))
    V = bf16(rng.standard_normal((T + 30, d)))
    bk = bf16(rng.standard_normal((A // C + 1, d)))
    bv = bf16(rng.standard_normal((A // C + 1, d)))
    for t in range(A):
        K[t], V[t] = bk[t // C], bv[t // C]
    q = bf16(rng.standard_normal((2, d)) * 2)
    r = O.step_head(q, K, V, T, W, C, 0.6, O.METRIC_QK)
    assert r.cnt.sum() > A // 4
    for T_now in (T, T + 1, T + 30):
        qn = bf16(rng.standard_normal((2, d)) * 2)
        assert np.allclose(O.reuse_head(qn, K, V, T_now, r), sdpa_reference(qn, K[:T_now], V[:T_now]),
                           rtol=1e-12, atol=1e-13)
    with pytest.raises(ValueError):
        O.reuse_head(q, K, V, A - 1, r)


# ------------------------------------------------------ packed region -------
def test_pack_heads_worked_example():
    # four heads, budgets 3, 5, 2, 4; the second is sparse-loaded
    counts = np.array([[3, 5], [2, 4]])
    modes = np.array([[0, 1], [0, 0]], np.uint8)
    off, m = O.pack_heads(counts, modes, 100)
    assert off.tolist() == [[0, 3], [3, 5]] and m.tolist() == modes.tolist()
    # a region of 8 rows: heads 0 and 2 fit (rows 0-2, 3-4), head 3 (rows 5-8) does not
    off, m = O.pack_heads(counts, modes, 8)
    assert off.tolist() == [[0, 3], [3, 5]] and m.tolist() == [[0, 1], [0, 1]]
    # exactly full
    off, m = O.pack_heads(counts, modes, 9)
    assert m.tolist() == [[0, 1], [0, 0]]


def test_pack_heads_brute_force():
    # against a direct enumeration of which prefix of rewritten heads fits
    rng = np.random.default_rng(9)
    for _ in range(300):
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        counts = rng.integers(0, 20, (B, H))
        modes = (rng.random((B, H)) < 0.3).astype(np.uint8)
        cap = int(rng.integers(0, 60))
        off, m = O.pack_heads(counts, modes, cap)
        k, md = counts.ravel(), modes.ravel()
        for i in range(k.size):
            before = sum(int(k[j]) for j in range(i) if md[j] == 0)
            assert off.ravel()[i] == before
            fits = md[i] == 0 and before + int(k[i]) <= cap
            assert m.ravel()[i] == (0 if fits else 1)
        # rewritten heads never overlap and stay inside the region
        used = [(int(off.ravel()[i]), int(k[i])) for i in range(k.size) if m.ravel()[i] == 0]
        for a, (o, n) in enumerate(used):
            assert o + n <= cap
            for o2, n2 in used[a + 1:]:
                assert o + n <= o2 or o2 + n2 <= o


# ------------------------------------------- rewritten tier's block manager --
def test_tier_alloc_worked_example():
    # four heads (B=2, Hkv=2), blocks of 4 rows, a pool of 6 blocks, all free
    table = np.full((2, 2, 3), -1)
    held = np.zeros((2, 2), np.int64)
    ids = np.arange(6)
    counts = np.array([[5, 3], [9, 0]])      # needs 2, 1, 3, 0 blocks
    modes = np.zeros((2, 2), np.uint8)
    t, hd, ids2, top, m = O.tier_alloc(table, held, ids, 6, counts, modes, 4, 100)
    # pops from the top: head 0 takes 5, 4; head 1 takes 3; head 2 takes 2, 1, 0
    assert t[0, 0, :2].tolist() == [5, 4] and t[0, 1, :1].tolist() == [3]
    assert t[1, 0, :3].tolist() == [2, 1, 0]
    assert hd.tolist() == [[2, 1], [3, 0]] and top == 0 and m.tolist() == modes.tolist()
    # next selection: budgets 1, 8, 2, 4 (needs 1, 2, 1, 1); everything is
    # pushed back in head order (5 4 | 3 | 2 1 0), then popped from the top
    t3, hd3, ids3, top3, m3 = O.tier_alloc(t, hd, ids2, top, np.array([[1, 8], [2, 4]]),
                                           modes, 4, 100)
    assert t3[0, 0, 0] == 0 and t3[0, 1, :2].tolist() == [1, 2] and t3[1, 0, 0] == 3
    assert t3[1, 1, 0] == 4 and top3 == 1 and ids3[0] == 5
    assert hd3.tolist() == [[1, 2], [1, 1]]
    # a pool that runs out: needs 2, 1, 3 with 4 free blocks -> head 2 and
    # every rewritten head after it is sparse-loaded
    t4, hd4, _, top4, m4 = O.tier_alloc(table, held, np.arange(6), 4, counts, modes, 4, 100)
    assert m4.tolist() == [[0, 0], [1, 1]] and hd4.tolist() == [[2, 1], [0, 0]] and top4 == 1
    # sparse-loaded heads by policy need nothing; counts clamp to the cap
    m_in = np.array([[1, 0], [0, 0]], np.uint8)
    _, hd5, _, top5, m5 = O.tier_alloc(table, held, np.arange(6), 6, counts, m_in, 4, 6)
    assert hd5.tolist() == [[0, 1], [2, 0]] and top5 == 3 and m5.tolist() == m_in.tolist()


def test_tier_alloc_invariants_and_pack_rule():
    """Over random histories: blocks are conserved and never shared, each
    head holds ceil(k / tb) blocks when rewritten, and which heads fit is
    pack_heads' rule applied to block needs over the blocks free after the
    pushes."""
    rng = np.random.default_rng(12)
    for trial in range(60):
        B, Hkv, tb = int(rng.integers(1, 4)), int(rng.integers(1, 4)), int(rng.choice([4, 8]))
        cap, nblk = 40, int(rng.integers(1, 30))
        maxb = -(-cap // tb)
        table = np.full((B, Hkv, maxb), -1)
        held = np.zeros((B, Hkv), np.int64)
        ids, top = np.arange(nblk), nblk
        for step in range(5):
            counts = rng.integers(-3, cap + 10, (B, Hkv))
            modes = (rng.random((B, Hkv)) < 0.25).astype(np.uint8)
            table, held2, ids, top2, m = O.tier_alloc(table, held, ids, top, counts, modes, tb,
                                                      cap)
            need = -(-np.clip(counts, 0, cap) // tb)
            _, want = O.pack_heads(need, modes, top + int(held.sum()))
            assert np.array_equal(m, want)
            live = [int(table[b, h, j]) for b in range(B) for h in range(Hkv)
                    for j in range(int(held2[b, h]))]
            stack = ids[:top2].tolist()
            assert sorted(live + stack) == list(range(nblk))       # conserved, distinct
            for b in range(B):
                for h in range(Hkv):
                    want_h = need[b, h] if m[b, h] == O.MODE_REWRITE else 0
                    assert held2[b, h] == want_h
            held, top = held2, top2
