"""Pins of the oracle's key-dissimilarity metric (CPU only).

The pages count similarity scores among the importance metrics that
calibration brings into one probability space (gist.science technical
summary, section 2.B "Goal") and list key-similarity-based eviction among
related work.  The metric s_t = -cos(k_t, sum of the candidate keys) is
pinned here against scipy's cosine distance, closed forms (two antipodal
key groups, an orthonormal key set), exact invariance under power-of-two
scaling and permutation, the zero-vector convention, the ranking of a
planted off-direction key, and reductions of the whole step to full
softmax attention (p = 1 and C = 1).
"""
import math

import numpy as np
import pytest
import torch
from scipy.spatial.distance import cosine

import oracle as O


def _f32(x):
    return np.asarray(x, np.float32)


def _ulps(a, b):
    ia = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


def test_matches_scipy_cosine_distance():
    rng = np.random.default_rng(1)
    for trial in range(4):
        n, d = int(rng.integers(20, 400)), int(rng.choice([64, 128]))
        K = _f32(rng.standard_normal((n, d)) + rng.uniform(-1, 1, d))
        mu = K.astype(np.float64).sum(0)
        ref = _f32([cosine(k.astype(np.float64), mu) - 1.0 for k in K])
        s = O.keydiff_head(K)
        assert _ulps(s, ref).max() <= 1, trial


def test_antipodal_groups():
    # n1 keys along +a e1, n2 along -b e1: the sum points along the larger
    # group, whose keys score -1; the other group scores +1
    d = 16
    K = np.zeros((7, d), np.float32)
    K[:4, 0] = 0.5    # 4 x 0.5 = 2
    K[4:, 0] = -0.25  # 3 x -0.25 = -0.75
    s = O.keydiff_head(K)
    assert np.array_equal(s, _f32([-1, -1, -1, -1, 1, 1, 1]))


def test_orthonormal_keys():
    d = 64
    s = O.keydiff_head(np.eye(d, dtype=np.float32))
    assert np.array_equal(s, np.full(d, np.float32(-1.0 / math.sqrt(d))))


@pytest.mark.parametrize("a", [0.5, 4.0])
def test_power_of_two_scale_and_permutation(a):
    rng = np.random.default_rng(2)
    K = _f32(rng.standard_normal((300, 128)))
    s = O.keydiff_head(K)
    assert np.array_equal(O.keydiff_head(_f32(a * K.astype(np.float64))), s)
    perm = rng.permutation(300)
    assert np.array_equal(O.keydiff_head(K[perm]), s[perm])


def test_zero_vectors():
    rng = np.random.default_rng(3)
    K = _f32(rng.standard_normal((50, 32)))
    K[7] = 0
    s = O.keydiff_head(K)
    assert s[7] == 0 and np.count_nonzero(s) == 49
    # keys that sum to zero: every score is 0, the metric is constant, c = 0
    K2 = np.concatenate([K, -K])
    s2 = O.keydiff_head(K2)
    assert np.all(s2 == 0)
    ell = _f32(rng.standard_normal(100))
    cal = O.calibrate_head(ell, s2, O.METRIC_KEYDIFF)
    assert np.all(cal.c == 0)
    sel = O.topp_head(cal.c, cal.w, cal.Z, 0.625)  # p exact in float32
    assert sel.k == math.ceil(0.625 * 100) and np.array_equal(np.sort(sel.selected), np.arange(sel.k))
    assert O.keydiff_head(np.zeros((0, 8), np.float32)).size == 0


def test_off_direction_key_ranks_first():
    rng = np.random.default_rng(4)
    d = 128
    common = rng.standard_normal(d)
    K = _f32(common + 0.3 * rng.standard_normal((500, d)))
    K[123] = _f32(-common + 0.3 * rng.standard_normal(d))  # opposite direction
    s = O.keydiff_head(K)
    assert int(np.argmax(s)) == 123 and s[123] > 0.9
    # calibrated onto a head's logits it is the heaviest candidate
    ell = _f32(rng.standard_normal(500))
    for calib in (O.CALIB_SPREAD, O.CALIB_ENTROPY):
        cal = O.calibrate_head(ell, s, O.METRIC_KEYDIFF, calib)
        assert int(np.argmax(cal.c)) == 123


def test_step_reduces_to_full_attention():
    rng = np.random.default_rng(5)
    G, d, T = 4, 64, 400
    bf = lambda x: torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()  # noqa: E731
    q = bf(rng.standard_normal((G, d)))
    K = bf(rng.standard_normal((T, d)))
    V = bf(rng.standard_normal((T, d)))
    # full softmax attention from torch's library routine (float64, CPU)
    qt = torch.tensor(np.asarray(q, np.float64))[None, :, None, :]
    kt = torch.tensor(np.asarray(K, np.float64))[None, None].expand(1, G, -1, -1).contiguous()
    vt = torch.tensor(np.asarray(V, np.float64))[None, None].expand(1, G, -1, -1).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, :, 0].numpy()
    for calib in (O.CALIB_SPREAD, O.CALIB_ENTROPY):
        for C, p in ((32, 1.0), (1, 0.4)):
            r = O.step_head(q, K, V, T, 50, C, p, O.METRIC_KEYDIFF, calib=calib)
            assert np.allclose(r.out, ref, rtol=1e-12, atol=1e-13), (calib, C, p)
