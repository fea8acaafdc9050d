"""Pins of the oracle's observation-window metric (gist.science technical
summary, section 2.B: calibration maps selection strategies such as SnapKV
onto one probability space; "Goal": max-pooled logits).  CPU only.

Pinned by a Hadamard closed form over several window queries, the pooling
against scipy's maximum filter, the reduction of a one-query unpooled window
to the raw logits, and the uniform closed form a pooling radius covering the
candidates produces.
"""
import math

import numpy as np
import pytest
import torch
from scipy.ndimage import maximum_filter1d

import oracle as O


def sylvester(n):
    h = np.array([[1.0]])
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def bf16(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def test_window_hadamard_closed_form():
    # keys: the 8 rows of a Hadamard matrix; window of 3 queries x 2 group
    # heads, each a multiple of one Hadamard row: k_t . q = 8 c when the rows
    # match, 0 otherwise
    H = sylvester(8)
    q = np.zeros((3, 2, 8))
    q[0, 0], q[0, 1] = 2 * H[1], -1 * H[3]
    q[1, 0], q[1, 1] = 3 * H[5], 0.5 * H[1]
    q[2, 0], q[2, 1] = 1 * H[6], 4 * H[6]
    want = np.zeros(8)
    want[1] = 16.0                  # max(2 * 8, 0.5 * 8)
    want[3] = 0.0                   # -1 * 8 < 0 from the other queries
    want[5] = 24.0
    want[6] = 32.0
    want /= math.sqrt(8)
    got = O.window_score_head(q, H, 0)
    assert np.array_equal(got, want.astype(np.float32))
    # pooling over one neighbour on each side
    pooled = O.window_score_head(q, H, 1)
    assert np.array_equal(pooled, maximum_filter1d(want.astype(np.float32), 3, mode="nearest"))


@pytest.mark.parametrize("r", [0, 1, 3, 17])
def test_window_pooling_is_a_clamped_maximum_filter(r):
    rng = np.random.default_rng(r)
    q = bf16(rng.standard_normal((4, 2, 32)))
    K = bf16(rng.standard_normal((200, 32)))
    raw = O.window_score_head(q, K, 0)
    want = maximum_filter1d(raw, size=2 * r + 1, mode="constant", cval=-np.inf)
    assert np.array_equal(O.window_score_head(q, K, r), want)
    # the window contains the current query: never below its own logits
    ell, _ = O.score_head(q[0], K)
    assert np.all(raw >= ell)


def test_window_of_one_query_is_the_raw_logit():
    rng = np.random.default_rng(3)
    q = bf16(rng.standard_normal((1, 4, 64)))
    K = bf16(rng.standard_normal((300, 64)))
    ell, _ = O.score_head(q[0], K)
    x = O.window_score_head(q, K, 0)
    assert np.array_equal(x, ell)
    cal = O.calibrate_head(ell, x, O.METRIC_WINDOW)
    # equal spreads: the temperature is exactly 1, c = fl32(ell - mean(ell))
    assert cal.scale == 1.0
    assert np.array_equal(cal.c, (ell.astype(np.float64) - np.mean(ell.astype(np.float64))).astype(np.float32))


def test_window_radius_covering_candidates_is_uniform():
    # every token pooled to the global maximum: equal calibrated values, so
    # top-p keeps the first ceil(p n) positions (zero spread -> c = 0)
    rng = np.random.default_rng(4)
    T, W, d = 120, 20, 16
    q = bf16(rng.standard_normal((2, d)))
    hist = bf16(rng.standard_normal((2, 2, d)))
    K = bf16(rng.standard_normal((T, d)))
    V = bf16(rng.standard_normal((T, d)))
    for p in (0.3, 0.77):
        r = O.step_head(q, K, V, T, W, 16, p, O.METRIC_WINDOW, q_hist=hist, radius=T)
        n = T - W
        assert np.all(r.cal.c == 0)
        k = math.ceil(np.float32(p) * n)
        assert r.sel.k == k and np.array_equal(r.pos, np.arange(k))


def test_window_step_uses_the_history():
    # a token aligned with an old query only is kept by the window metric
    rng = np.random.default_rng(5)
    T, W, d = 400, 40, 32
    q = bf16(rng.standard_normal((2, d)))
    hist = bf16(rng.standard_normal((3, 2, d)))
    K = bf16(rng.standard_normal((T, d)))
    V = bf16(rng.standard_normal((T, d)))
    target = 123
    K[target] = bf16(6.0 * hist[2, 1] / np.linalg.norm(hist[2, 1]) * math.sqrt(d) ** 0.5)
    rq = O.step_head(q, K, V, T, W, 16, 0.5, O.METRIC_QK)
    rw = O.step_head(q, K, V, T, W, 16, 0.5, O.METRIC_WINDOW, q_hist=hist, radius=2)
    assert target not in rq.pos[:1] and target in rw.pos
    # pooling ties its neighbours to it at the top; equal values go by position
    top = np.argsort(-rw.cal.c, kind="stable")[:5]
    assert sorted(top.tolist()) == list(range(target - 2, target + 3))
    assert rw.pos[:3].tolist() == [target - 2, target - 1, target]
    rw9 = O.step_head(q, K, V, T, W, 16, 0.95, O.METRIC_WINDOW, q_hist=hist, radius=2)
    assert set(range(target - 2, target + 3)) <= set(rw9.pos.tolist())
