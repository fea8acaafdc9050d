"""Pins of the oracle's entropy-matched calibration (CPU only).

The pages calibrate non-logit metrics by adjusting a temperature so that
they map onto the raw attention distribution, and tie Tier-2 budgets to
attention entropy (gist.science technical summary, sections 2.A and 2.B).
The entropy rule picks the inverse temperature beta at which the metric's
softmax has the entropy of the head's raw attention.  Pinned here against a
proportional-logit closed form (logits = kappa * metric gives beta = kappa),
an independent root of the same equation (scipy's brentq over scipy's
softmax and entr), exact invariance under power-of-two rescaling, and the
limits the bisection reaches without a root (uniform attention, tied maxima,
a constant metric).
"""
import math

import numpy as np
import pytest
from scipy.optimize import brentq
from scipy.special import entr, softmax

import oracle as O


def _entropy_scipy(x):
    return float(entr(softmax(np.asarray(x, np.float64))).sum())


def _f32(x):
    return np.asarray(x, np.float32)


def _rel(a, b):
    return abs(a - b) / abs(b)


@pytest.mark.parametrize("kappa", [0.3, 1.0, 2.5])
def test_proportional_logits_give_their_factor(kappa):
    rng = np.random.default_rng(1)
    s = _f32(rng.standard_normal(3000) * 1.7 + 5.0)
    ell = _f32(kappa * s.astype(np.float64))
    beta = O.entropy_temperature(ell, s)
    assert _rel(beta, kappa) < 1e-5, (beta, kappa)


def test_matches_an_independent_root():
    rng = np.random.default_rng(2)
    for trial in range(6):
        n = int(rng.integers(50, 4000))
        ell = _f32(rng.standard_normal(n) * rng.uniform(0.5, 3.0))
        s = _f32(np.abs(rng.standard_normal(n)) * rng.uniform(0.1, 10.0))
        target = _entropy_scipy(ell)
        f = lambda beta: _entropy_scipy(beta * s.astype(np.float64)) - target  # noqa: E731
        hi = O.ENTROPY_SPAN / float(s.max() - s.min())
        ref = brentq(f, 1e-12, hi, xtol=1e-15, rtol=1e-13)
        beta = O.entropy_temperature(ell, s)
        assert _rel(beta, ref) < 2e-6, (trial, beta, ref)


def test_calibrated_values_carry_the_attention_entropy():
    rng = np.random.default_rng(3)
    ell = _f32(rng.standard_normal(2000) * 2.0)
    s = _f32(rng.gamma(2.0, 1.0, 2000))
    cal = O.calibrate_head(ell, s, O.METRIC_L2, O.CALIB_ENTROPY)
    assert cal.shift == float(s.max()) and cal.m == 0.0
    assert abs(_entropy_scipy(cal.c) - _entropy_scipy(ell)) < 1e-5
    # order preserved: the calibrated value is an increasing map of s
    order_s = np.lexsort((np.arange(s.size), -s.astype(np.float64)))
    assert np.all(np.diff(cal.c[order_s].astype(np.float64)) <= 0)


@pytest.mark.parametrize("a", [2.0, 0.25, 8.0])
def test_power_of_two_rescaling_is_exact(a):
    # s -> a s with a a power of two: every bisection midpoint scales by 1/a
    # exactly, so beta scales by 1/a and the calibrated values are bit-equal
    rng = np.random.default_rng(4)
    ell = _f32(rng.standard_normal(1500))
    s = _f32(rng.standard_normal(1500))
    c1 = O.calibrate_head(ell, s, O.METRIC_L2, O.CALIB_ENTROPY)
    c2 = O.calibrate_head(ell, _f32(a * s.astype(np.float64)), O.METRIC_L2, O.CALIB_ENTROPY)
    assert c2.scale == c1.scale / a
    assert np.array_equal(c1.c, c2.c)
    t1 = O.topp_head(c1.c, c1.w, c1.Z, 0.9)
    t2 = O.topp_head(c2.c, c2.w, c2.Z, 0.9)
    assert np.array_equal(np.sort(t1.selected), np.sort(t2.selected))


def test_affine_metric_same_temperature_per_unit():
    rng = np.random.default_rng(5)
    ell = _f32(rng.standard_normal(1000) * 1.5)
    s = _f32(rng.standard_normal(1000))
    b1 = O.entropy_temperature(ell, s)
    b2 = O.entropy_temperature(ell, _f32(3.0 * s.astype(np.float64) + 7.0))
    assert _rel(b2, b1 / 3.0) < 1e-5


def test_sharper_attention_gives_a_smaller_budget():
    rng = np.random.default_rng(6)
    base = rng.standard_normal(4000)
    s = _f32(np.abs(rng.standard_normal(4000)))
    ks = []
    for scale in (0.25, 0.5, 1.0, 2.0, 4.0):
        cal = O.calibrate_head(_f32(scale * base), s, O.METRIC_L2, O.CALIB_ENTROPY)
        ks.append(O.topp_head(cal.c, cal.w, cal.Z, 0.9).k)
    assert all(x >= y for x, y in zip(ks, ks[1:])) and ks[0] > ks[-1]


def test_uniform_attention_keeps_the_top_ceil_pn_by_metric():
    # constant logits: target ln n, every midpoint falls short, beta -> 0;
    # weights are 1 - O(1e-7) and the budget is ceil(p n), by metric order
    rng = np.random.default_rng(7)
    n, p = 1000, 0.8037
    s = _f32(rng.standard_normal(n))
    cal = O.calibrate_head(np.zeros(n, np.float32), s, O.METRIC_L2, O.CALIB_ENTROPY)
    hi = O.ENTROPY_SPAN / float(s.max() - s.min())
    assert 0 < cal.scale <= hi * 2.0 ** -O.ENTROPY_STEPS
    sel = O.topp_head(cal.c, cal.w, cal.Z, p)
    assert sel.k == math.ceil(p * n)
    top = np.lexsort((np.arange(n), -s.astype(np.float64)))[:sel.k]
    assert np.array_equal(np.sort(sel.selected), np.sort(top))


def test_tied_maxima_clamp_at_the_bracket_end():
    # one dominant logit (target entropy ~0) but three tied metric maxima:
    # no temperature reaches the target, beta ends at the top of the bracket,
    # the ties carry all the mass and are taken lowest position first
    n = 200
    ell = np.zeros(n, np.float32)
    ell[17] = 60.0
    s = _f32(np.linspace(0.0, 1.0, n))
    s[[5, 90, 150]] = 2.0
    cal = O.calibrate_head(ell, s, O.METRIC_L2, O.CALIB_ENTROPY)
    hi = O.ENTROPY_SPAN / 2.0
    assert cal.scale == pytest.approx(hi, rel=1e-9)
    sel = O.topp_head(cal.c, cal.w, cal.Z, 0.5)
    assert sel.k == 2 and sorted(sel.selected.tolist()) == [5, 90]


def test_constant_metric_and_empty_head():
    s = np.full(50, 3.5, np.float32)
    ell = _f32(np.random.default_rng(8).standard_normal(50))
    cal = O.calibrate_head(ell, s, O.METRIC_L2, O.CALIB_ENTROPY)
    assert cal.scale == 0.0 and np.all(cal.c == 0)
    sel = O.topp_head(cal.c, cal.w, cal.Z, 0.7)
    assert sel.k == 35 and np.array_equal(np.sort(sel.selected), np.arange(35))
    cal0 = O.calibrate_head(np.zeros(0, np.float32), np.zeros(0, np.float32), O.METRIC_L2,
                            O.CALIB_ENTROPY)
    assert cal0.c.size == 0 and cal0.Z == 0.0


def test_qk_heads_ignore_the_rule():
    rng = np.random.default_rng(9)
    ell = _f32(rng.standard_normal(300))
    a = O.calibrate_head(ell, ell, O.METRIC_QK, O.CALIB_SPREAD)
    b = O.calibrate_head(ell, ell, O.METRIC_QK, O.CALIB_ENTROPY)
    assert np.array_equal(a.c, b.c) and a.scale == b.scale == 1.0


def test_step_with_entropy_rule_reduces_to_full_attention():
    import torch
    rng = np.random.default_rng(10)
    G, d, T = 2, 32, 300
    bf = lambda x: torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()  # noqa: E731
    q = bf(rng.standard_normal((G, d)) * 1.5)
    K = bf(rng.standard_normal((T, d)))
    V = bf(rng.standard_normal((T, d)))
    qt = torch.tensor(q, dtype=torch.float64)[None, :, None, :]
    kt = torch.tensor(K, dtype=torch.float64)[None, None].expand(1, G, -1, -1).contiguous()
    vt = torch.tensor(V, dtype=torch.float64)[None, None].expand(1, G, -1, -1).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, :, 0].numpy()
    for metric in (O.METRIC_L2, O.METRIC_WINDOW):
        for C, p in ((16, 1.0), (1, 0.6)):
            r = O.step_head(q, K, V, T, 40, C, p, metric, calib=O.CALIB_ENTROPY)
            assert np.allclose(r.out, ref, rtol=1e-12, atol=1e-13)
    with pytest.raises(ValueError):
        O.calibrate_head(ell := _f32(rng.standard_normal(10)), ell, O.METRIC_L2, 7)
