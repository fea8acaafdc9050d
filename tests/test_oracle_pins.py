"""Pins of the CPU oracle to things other than itself.

Each test checks the oracle against a closed form, a hand-derived value,
brute force on tiny inputs, a library routine for a special case that
reduces to plain attention, or an invariant the pages state (HARD-KV,
gist.science technical summary, sections 2.A-2.C).  None of these retypes
the oracle's own formula.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O


def sylvester(n):
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def bf16(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()


# ----------------------------------------------------------------- score ----
def test_score_hadamard_closed_form():
    # Rows of a Hadamard matrix are orthogonal with squared norm d, so
    # (a H_i) . (b H_j) = a b d [i == j].  With G = 3 scaled query rows the
    # max-pooled logit of key b_t H_j is max over the g with i_g == j of
    # a_g b_t sqrt(d), and 0 when no query row matches (other rows give 0).
    d = 64
    H = sylvester(d)
    qi = [5, 9, 5]
    qa = [0.5, -2.0, 3.0]
    q = np.stack([a * H[i] for a, i in zip(qa, qi)])
    kj = [5, 9, 7, 5, 9]
    kb = [1.0, 1.0, 2.0, -1.0, -0.25]
    K = np.stack([b * H[j] for b, j in zip(kb, kj)])
    ell, s = O.score_head(q, K)
    want = []
    for b, j in zip(kb, kj):
        vals = [a * b * math.sqrt(d) for a, i in zip(qa, qi) if i == j]
        want.append(max(vals + [0.0]) if len(vals) < 3 else max(vals))
    # key 0: matches q0 (0.5*8=4) and q2 (3*8=24) -> 24; key 1: only q1 -> -16,
    # the other rows give 0, so max = 0; key 2: no match -> 0; key 3: -4, -24
    # and 0 -> 0; key 4: q1 gives 0.5*8 = 4 -> 4.
    assert list(ell) == [24.0, 0.0, 0.0, 0.0, 4.0]
    assert np.allclose(ell, want)
    assert np.allclose(s, np.abs(kb) * math.sqrt(d))


def test_score_group_mapping_uses_only_own_queries():
    # Each KV head h sees only query rows h*G .. h*G+G-1.  A query row of the
    # other group aligned with a key must not change that key's score.
    d = 16
    H = sylvester(d)
    q = np.stack([H[1], H[2], 10 * H[3], 10 * H[4]])   # G = 2, two groups
    cache = np.stack([H[3], H[1]])
    res = O.step(q[None], lambda b, h: cache, lambda b, h: cache, [2], 0, 1, 1.0,
                 [O.METRIC_QK, O.METRIC_QK])
    assert list(res[(0, 0)].ell) == [0.0, 4.0]          # H[1] . H[1] / 4
    assert list(res[(0, 1)].ell) == [40.0, 0.0]         # 10 H[3] . H[3] / 4


def test_key_norm_integer_triples():
    # Pythagorean quadruples have integer norms.
    rows = [(3, 4, 0, 0), (1, 2, 2, 0), (2, 3, 6, 0), (1, 4, 8, 0), (2, 4, 4, 0), (0, 0, 0, 0)]
    K = np.array(rows, float)
    _, s = O.score_head(np.ones((1, 4)), K)
    assert list(s) == [5.0, 3.0, 7.0, 9.0, 6.0, 0.0]


def test_score_brute_force_exact_rationals():
    # Brute force in exact rational arithmetic on bf16 data.
    rng = np.random.default_rng(1)
    d, G, n = 8, 2, 6
    q = bf16(rng.standard_normal((G, d)))
    K = bf16(rng.standard_normal((n, d)))
    ell, _ = O.score_head(q, K)
    inv = 1.0 / math.sqrt(d)
    for t in range(n):
        dots = [sum(Fraction(float(q[g, i])) * Fraction(float(K[t, i])) for i in range(d))
                for g in range(G)]
        exact = float(max(dots)) * inv
        assert abs(float(ell[t]) - exact) <= abs(exact) * 2 ** -23


# ------------------------------------------------------------- calibrate ----
def test_calibrate_qk_is_raw_softmax():
    rng = np.random.default_rng(2)
    ell = rng.standard_normal(50).astype(np.float32) * 3
    cal = O.calibrate_head(ell, np.zeros(50, np.float32), O.METRIC_QK)
    assert np.array_equal(cal.c, ell)
    ref = torch.softmax(torch.tensor(ell, dtype=torch.float64), 0).numpy()
    assert np.allclose(cal.w / cal.Z, ref, rtol=1e-14, atol=0)


def test_calibrate_l2_hand_example():
    # s = (1, 2, 3): mean 2, population std sqrt(2/3); ell = (0, 2, 4): std
    # sqrt(8/3).  Temperature ratio sqrt(8/3)/sqrt(2/3) = 2, so c = (-2, 0, 2);
    # permuting the tokens permutes c.
    cal = O.calibrate_head(np.array([0, 2, 4], np.float32), np.array([1, 2, 3], np.float32),
                           O.METRIC_L2)
    assert np.allclose(cal.c, [-2, 0, 2], atol=1e-6)
    cal = O.calibrate_head(np.array([4, 0, 2], np.float32), np.array([3, 1, 2], np.float32),
                           O.METRIC_L2)
    assert np.allclose(cal.c, [2, -2, 0], atol=1e-6)
    # softmax of (-2, 0, 2) by hand
    e = np.exp([-4.0, -2.0, 0.0])
    assert np.allclose(np.sort(cal.w / cal.Z), np.sort(e / e.sum()), rtol=1e-12)


def test_calibrate_l2_invariants():
    # Order preserved (the pages: calibration keeps the order of the original
    # strategy), zero mean, spread equal to the raw-logit spread, and
    # invariance under an exact positive affine change of the metric.
    rng = np.random.default_rng(3)
    s = rng.integers(0, 1000, 400).astype(np.float32)
    ell = (rng.standard_normal(400) * 1.7).astype(np.float32)
    cal = O.calibrate_head(ell, s, O.METRIC_L2)
    o = np.argsort(s, kind="stable")
    assert np.all(np.diff(cal.c[o].astype(np.float64)) >= 0)
    assert abs(np.mean(cal.c.astype(np.float64))) < 1e-5
    assert abs(np.std(cal.c.astype(np.float64)) - np.std(ell.astype(np.float64))) < 1e-5
    cal2 = O.calibrate_head(ell, (4 * s + 8).astype(np.float32), O.METRIC_L2)
    ulp = np.spacing(np.abs(cal.c).astype(np.float32))
    assert np.all(np.abs(cal2.c.astype(np.float64) - cal.c) <= ulp)
    flat = O.calibrate_head(ell, np.full(400, 7.0, np.float32), O.METRIC_L2)
    assert np.all(flat.c == 0) and np.allclose(flat.w, 1.0)


# --------------------------------------------------------------- top-p ------
def brute_force_topp(c, p):
    """Minimum cardinality, then maximum mass, then lexicographically smallest
    positions, over all subsets, with exactly rounded sums."""
    n = len(c)
    w = [math.exp(float(x) - float(max(c))) for x in c]
    Z = math.fsum(w)
    target = float(np.float32(p)) * Z
    for k in range(1, n + 1):
        best = None
        for sub in itertools.combinations(range(n), k):
            m = math.fsum(w[i] for i in sub)
            key = (-m, sub)
            if best is None or key < best:
                best = key
        if -best[0] >= target:
            return list(best[1]), w, Z
    return list(range(n)), w, Z


def oracle_topp(c, p):
    cal = O.calibrate_head(np.asarray(c, np.float32), np.zeros(len(c), np.float32), O.METRIC_QK)
    return O.topp_head(cal.c, cal.w, cal.Z, p)


@pytest.mark.parametrize("seed", range(40))
def test_topp_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 11))
    if seed % 3 == 0:
        c = rng.integers(-2, 3, n).astype(np.float32)     # many exact ties
    else:
        c = (rng.standard_normal(n) * 2).astype(np.float32)
    p = np.float32(rng.uniform(0.05, 0.999))
    sel = oracle_topp(c, p)
    want, w, Z = brute_force_topp(c, p)
    # keep the draw away from mass boundaries, where rounding order matters
    pref = np.cumsum(np.sort(w)[::-1]) / Z
    if np.min(np.abs(pref - float(p))) < 1e-12:
        pytest.skip("draw lands on a mass boundary")
    assert list(sel.selected) == sorted(want)


def test_topp_uniform_closed_form():
    # All-equal scores: every weight is 1, so k = ceil(p n) and the tie rule
    # keeps the k lowest positions.
    for n in (1, 7, 10, 1000, 4097):
        for p in (0.05, 0.25, 0.5, 0.9, 0.95, 0.999):
            p32 = np.float32(p)
            k = math.ceil(Fraction(float(p32)) * n)
            sel = oracle_topp(np.full(n, 1.5, np.float32), p32)
            assert sel.k == k
            assert list(sel.selected) == list(range(k))


def test_topp_two_level_closed_form():
    # M tokens at logit L, n - M at 0: weights 1 and r = e^-L, Z = M + (n-M) r.
    # If p Z <= M, k = ceil(p Z); else k = M + ceil((p Z - M) / r).
    n, M, L = 500, 20, 3.0
    r = math.exp(-L)
    Z = M + (n - M) * r
    c = np.zeros(n, np.float32)
    rng = np.random.default_rng(5)
    hot = np.sort(rng.choice(n, M, replace=False))
    c[hot] = L
    for p in (0.1, 0.5, 0.7, 0.8, 0.95):
        pZ = float(np.float32(p)) * Z
        if pZ <= M:
            k = math.ceil(pZ)
            want = list(hot[:k])
        else:
            extra = math.ceil((pZ - M) / r)
            cold = [i for i in range(n) if i not in set(hot)]
            want = sorted(list(hot) + cold[:extra])
            k = M + extra
        sel = oracle_topp(c, p)
        assert sel.k == k, p
        assert list(sel.selected) == want


def test_topp_minimal_mass_and_nesting():
    rng = np.random.default_rng(6)
    for _ in range(30):
        n = int(rng.integers(1, 3000))
        c = (rng.standard_normal(n) * rng.uniform(0.2, 5)).astype(np.float32)
        prev = set()
        for p in (0.3, 0.8, 0.9, 0.99):
            sel = oracle_topp(c, p)
            cal = O.calibrate_head(c, np.zeros(n, np.float32), O.METRIC_QK)
            w = cal.w
            mass = math.fsum(w[sel.selected])
            assert mass >= float(np.float32(p)) * cal.Z * (1 - 1e-12)
            last = sel.order[sel.k - 1]
            assert mass - w[last] < float(np.float32(p)) * cal.Z * (1 + 1e-12)
            # every unselected candidate ranks no higher than the last selected
            unsel = np.setdiff1d(np.arange(n), sel.selected)
            if unsel.size:
                assert c[unsel].max() <= c[last]
            s = set(sel.selected.tolist())
            assert prev <= s
            prev = s


def test_topp_budget_grows_with_temperature():
    # A softmax flattened by a higher temperature needs at least as many
    # tokens to reach the same mass (head-adaptive budgets follow the
    # attention pattern, section 2.A / 2.B).
    rng = np.random.default_rng(7)
    z = rng.standard_normal(5000)
    ks = [oracle_topp((z / tau).astype(np.float32), 0.9).k for tau in (0.25, 0.5, 1, 2, 4)]
    assert ks == sorted(ks) and ks[0] < ks[-1]


def test_topp_edge_cases():
    assert oracle_topp(np.zeros(0, np.float32), 0.9).k == 0
    assert oracle_topp(np.array([3.0, -1.0], np.float32), 1.0).k == 2
    assert oracle_topp(np.array([3.0, -1.0], np.float32), 1e-9).k == 1
    with pytest.raises(ValueError):
        oracle_topp(np.array([1.0], np.float32), 0.0)
    with pytest.raises(ValueError):
        O.score_head(np.ones((1, 4)), np.array([[np.nan, 0, 0, 0]]))


# --------------------------------------------------------- full pipeline ----
def sdpa_reference(q, K, V):
    """Full decode attention through torch's library routine (float64, CPU)."""
    G, d = q.shape
    qt = torch.tensor(np.asarray(q, np.float64))[None, :, None, :]
    kt = torch.tensor(np.asarray(K, np.float64))[None, None].expand(1, G, -1, -1).contiguous()
    vt = torch.tensor(np.asarray(V, np.float64))[None, None].expand(1, G, -1, -1).contiguous()
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, :, 0].numpy()


def _case(seed, T=300, d=32, G=3):
    rng = np.random.default_rng(seed)
    q = bf16(rng.standard_normal((G, d)) * 1.5)
    K = bf16(rng.standard_normal((T, d)))
    V = bf16(rng.standard_normal((T, d)))
    return q, K, V


@pytest.mark.parametrize("metric", [O.METRIC_QK, O.METRIC_L2])
def test_p_one_is_full_attention(metric):
    q, K, V = _case(10)
    r = O.step_head(q, K, V, 300, 40, 16, 1.0, metric)
    assert r.sel.k == r.A == 260 and r.cnt.sum() == 0
    assert np.allclose(r.out, sdpa_reference(q, K, V), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("p", [0.3, 0.8, 0.95])
def test_chunk_size_one_is_full_attention(p):
    # Each evicted token is its own chunk: count 1, bias ln 1 = 0, pooled key
    # and value equal to the token's own.
    q, K, V = _case(11)
    r = O.step_head(q, K, V, 300, 40, 1, p, O.METRIC_QK)
    assert 0 < r.sel.k < r.A
    assert np.allclose(r.out, sdpa_reference(q, K, V), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("metric,p,C", [(O.METRIC_QK, 0.5, 8), (O.METRIC_L2, 0.8, 16),
                                        (O.METRIC_QK, 0.9, 7)])
def test_chunk_constant_rows_are_full_attention(metric, p, C):
    # Identical rows within each chunk: n pooled copies of a token weigh
    # exp(q.k/sqrt(d) + ln n) = n exp(q.k/sqrt(d)), exactly what the n tokens
    # contribute to full attention.  Pins the ln n bias and the mean pooling.
    T, W, d = 301, 37, 32
    rng = np.random.default_rng(12)
    A = T - W
    nch = -(-A // C)
    base_k = bf16(rng.standard_normal((nch, d)) * 1.3)
    base_v = bf16(rng.standard_normal((nch, d)))
    K = bf16(rng.standard_normal((T, d)))
    V = bf16(rng.standard_normal((T, d)))
    for t in range(A):
        K[t] = base_k[t // C]
        V[t] = base_v[t // C]
    q = bf16(rng.standard_normal((2, d)) * 2)
    r = O.step_head(q, K, V, T, W, C, p, metric)
    assert r.cnt.sum() > 0
    assert np.allclose(r.out, sdpa_reference(q, K, V), rtol=1e-12, atol=1e-13)


def test_window_covering_context_is_full_attention():
    q, K, V = _case(13, T=50)
    r = O.step_head(q, K, V, 50, 64, 8, 0.5, O.METRIC_QK)
    assert r.A == 0 and r.sel.k == 0 and r.cnt.size == 0
    assert np.allclose(r.out, sdpa_reference(q, K, V), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("metric", [O.METRIC_QK, O.METRIC_L2])
def test_tiers_disjoint_cover_and_bit_copies(metric):
    # Dense, sparse and condensed tiers are disjoint and cover the context;
    # the rewritten rows are bit copies in ascending position order.
    q, K, V = _case(14, T=700)
    W, C = 64, 32
    r = O.step_head(q, K, V, 700, W, C, 0.85, metric)
    sel = set(r.pos.tolist())
    ev = set(range(r.A)) - sel
    dense = set(range(r.A, 700))
    assert not (sel & dense) and not (ev & dense) and len(sel) + len(ev) + len(dense) == 700
    assert np.all(np.diff(r.pos) > 0)
    assert np.array_equal(r.Kc.view(np.uint32), K[r.pos].view(np.uint32))
    assert np.array_equal(r.Vc.view(np.uint32), V[r.pos].view(np.uint32))
    assert r.cnt.sum() == len(ev)
    for j in range(len(r.cnt)):
        members = [t for t in ev if t // C == j]
        assert r.cnt[j] == len(members)
    assert np.array_equal(r.mask, np.isin(np.arange(r.A), r.pos).astype(np.uint8))


# -------------------------------------------------------- lifecycle ---------
def _lifecycle(seed, T0, W, C, p, steps, d=16, G=2):
    rng = np.random.default_rng(seed)
    Tmax = T0 + steps
    K = bf16(rng.standard_normal((Tmax, d)))
    V = bf16(rng.standard_normal((Tmax, d)))
    Q = bf16(rng.standard_normal((steps, G, d)) * 1.5)
    st = O.init_state(K, V, T0, W, C, -(-(Tmax - W) // C))
    return K, V, Q, st


def test_lifecycle_invariants():
    T0, W, C, steps = 200, 32, 8, 25
    K, V, Q, st = _lifecycle(20, T0, W, C, 0.9, steps)
    pool_prev = set(st.pool_pos.tolist())
    for s in range(steps):
        P = T0 + s
        out, info = O.lifecycle_step(st, Q[s], K[P], V[P], 0.9, O.METRIC_QK)
        ring_pos = set(range(P - W + 1, P + 1))
        pool = set(st.pool_pos.tolist())
        assert np.all(np.diff(st.pool_pos) > 0)
        assert pool <= pool_prev | {P - W}             # nothing comes back
        assert not (pool & ring_pos)
        assert len(pool) + int(st.cnt.sum()) + W == P + 1
        for t in range(P - W + 1, P + 1):
            assert np.array_equal(st.ring_K[t % W], K[t])
        pool_prev = pool
    # the running chunk scale sum|x| is, chunk by chunk, the brute-force sum
    # of |k| and |v| over the positions merged into it (every aged position
    # outside the pool)
    merged = sorted(set(range(T0 + steps - W)) - set(st.pool_pos.tolist()))
    ka = np.zeros_like(st.kabs)
    va = np.zeros_like(st.vabs)
    for t in merged:
        ka[t // C] += np.abs(K[t].astype(np.float64))
        va[t // C] += np.abs(V[t].astype(np.float64))
    assert np.allclose(st.kabs, ka, rtol=1e-13, atol=0) and np.allclose(st.vabs, va, rtol=1e-13, atol=0)
    assert np.all(np.abs(st.ksum) <= st.kabs * (1 + 1e-12))


@pytest.mark.parametrize("p,C", [(1.0, 8), (0.7, 1)])
def test_lifecycle_reduces_to_full_attention(p, C):
    # p = 1 never evicts; C = 1 pools every evicted token alone.  Both give
    # full attention over all tokens seen so far at every step.
    T0, W, steps = 120, 16, 12
    K, V, Q, st = _lifecycle(21, T0, W, C, p, steps)
    for s in range(steps):
        P = T0 + s
        out, _ = O.lifecycle_step(st, Q[s], K[P], V[P], p, O.METRIC_QK)
        assert np.allclose(out, sdpa_reference(Q[s], K[:P + 1], V[:P + 1]),
                           rtol=1e-12, atol=1e-13)


def test_lifecycle_first_step_equals_single_step():
    T0, W, C = 300, 32, 16
    K, V, Q, st = _lifecycle(22, T0, W, C, 0.9, 1)
    out, info = O.lifecycle_step(st, Q[0], K[T0], V[T0], 0.9, O.METRIC_QK)
    r = O.step_head(Q[0], K, V, T0 + 1, W, C, 0.9, O.METRIC_QK)
    assert info["k"] == r.sel.k
    assert np.array_equal(st.pool_pos, r.pos)
    assert np.allclose(out, r.out, rtol=1e-13, atol=1e-14)
