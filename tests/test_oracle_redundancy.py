"""Pins of the oracle's R-KV redundancy metric (redundancy_head).

The metric is a reading (the pages name R-KV among the strategies the
calibration maps, with no formula): s_t = -mean_{j != t} cos(k_t, k_j).
These tests hold the oracle's implementation to that definition through
routes that share none of its arithmetic: an explicit double loop over all
pairs with scipy's cosine distance, closed forms, exact invariances, and
reductions of the whole step to torch's scaled_dot_product_attention.
"""
import numpy as np
import pytest
import torch
from scipy.spatial.distance import cosine

import oracle as O


def _f32(x):
    return np.asarray(x, np.float32)


def _bf16(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def _brute(K):
    """-(1 / (n - 1)) sum over j != t of cos(k_t, k_j), pair by pair."""
    K = np.asarray(K, np.float64)
    n = len(K)
    out = np.zeros(n)
    for t in range(n):
        acc = 0.0
        for j in range(n):
            if j == t:
                continue
            if not K[t].any() or not K[j].any():
                continue  # cosine with a zero key is 0
            acc += 1.0 - cosine(K[t], K[j])
        out[t] = -acc / (n - 1) if n > 1 else 0.0
    return out


@pytest.mark.parametrize("seed,n,d", [(1, 7, 16), (2, 30, 64), (3, 41, 128), (4, 2, 8)])
def test_matches_pairwise_brute_force(seed, n, d):
    rng = np.random.default_rng(seed)
    K = _bf16(rng.standard_normal((n, d)) + 0.4 * rng.standard_normal(d))
    s = O.redundancy_head(K)
    ref = _brute(K)
    assert s.dtype == np.float32
    # one float32 rounding of the same float64 quantity: equal or 1 ulp apart
    ulp = np.abs(s.view(np.int32).astype(np.int64) - _f32(ref).view(np.int32).astype(np.int64))
    assert ulp.max() <= 1, ulp.max()
    assert np.allclose(s, ref, rtol=0, atol=1e-6)


def test_identical_directions_are_fully_redundant():
    rng = np.random.default_rng(5)
    v = _f32(rng.standard_normal(32))
    K = np.stack([v * 2.0 ** e for e in (-3, 0, 1, 4, 7)])   # exact positive multiples
    assert np.array_equal(O.redundancy_head(K), np.full(5, -1.0, np.float32))


def test_orthonormal_keys_are_not_redundant():
    K = np.eye(16, dtype=np.float32)[:9] * 3.0
    s = O.redundancy_head(K)
    assert np.all(s == 0.0)


@pytest.mark.parametrize("a,b", [(3, 1), (5, 4), (1, 6)])
def test_two_antipodal_groups(a, b):
    v = np.zeros(8, np.float32)
    v[2] = 1.0
    K = np.concatenate([np.tile(v, (a, 1)), np.tile(-v, (b, 1))])
    s = O.redundancy_head(K)
    n = a + b
    assert np.all(s[:a] == np.float32(-(a - 1 - b) / (n - 1)))
    assert np.all(s[a:] == np.float32(-(b - 1 - a) / (n - 1)))


def test_power_of_two_scaling_and_permutation():
    rng = np.random.default_rng(6)
    K = _bf16(rng.standard_normal((50, 64)))
    s = O.redundancy_head(K)
    scale = 2.0 ** rng.integers(-6, 7, size=50)
    assert np.array_equal(O.redundancy_head(K * scale[:, None]), s)
    perm = rng.permutation(50)
    assert np.array_equal(O.redundancy_head(K[perm]), s[perm])


def test_zero_key_and_single_candidate():
    rng = np.random.default_rng(7)
    K = _bf16(rng.standard_normal((6, 16)))
    K0 = np.concatenate([K, np.zeros((1, 16), np.float32)])
    s0 = O.redundancy_head(K0)
    assert s0[-1] == 0.0
    # the zero key adds no similarity but counts among the others
    assert np.allclose(s0[:-1], O.redundancy_head(K).astype(np.float64) * 5 / 6, atol=1e-7)
    assert np.array_equal(O.redundancy_head(K[:1]), np.zeros(1, np.float32))
    assert O.redundancy_head(K[:0]).shape == (0,)


def test_unique_key_ranks_first_after_calibration():
    rng = np.random.default_rng(8)
    common = rng.standard_normal(64)
    K = _f32(common + 0.2 * rng.standard_normal((200, 64)))
    K[77] = _f32(rng.standard_normal(64))      # a key unlike the others
    s = O.redundancy_head(K)
    assert int(np.argmax(s)) == 77
    ell = _f32(rng.standard_normal(200))
    for calib in (O.CALIB_SPREAD, O.CALIB_ENTROPY):
        cal = O.calibrate_head(ell, s, O.METRIC_RKV, calib)
        assert int(np.argmax(cal.c)) == 77
        # calibration keeps the metric's order (a temperature)
        assert np.all(np.diff(cal.c[np.argsort(s, kind="stable")]) >= 0)


def _sdpa(q, K, V):
    G = q.shape[0]
    qt = torch.tensor(np.asarray(q, np.float64))[None, :, None, :]
    kt = torch.tensor(np.asarray(K, np.float64))[None, None].expand(1, G, -1, -1).contiguous()
    vt = torch.tensor(np.asarray(V, np.float64))[None, None].expand(1, G, -1, -1).contiguous()
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, :, 0].numpy()


def test_step_reduces_to_full_attention():
    rng = np.random.default_rng(9)
    G, d, T = 4, 64, 400
    q = _bf16(rng.standard_normal((G, d)))
    K = _bf16(rng.standard_normal((T, d)))
    V = _bf16(rng.standard_normal((T, d)))
    ref = _sdpa(q, K, V)
    for calib in (O.CALIB_SPREAD, O.CALIB_ENTROPY):
        for C, p in ((32, 1.0), (1, 0.4)):
            r = O.step_head(q, K, V, T, 50, C, p, O.METRIC_RKV, calib=calib)
            assert np.allclose(r.out, ref, rtol=1e-12, atol=1e-13), (calib, C, p)
            assert r.s.shape == (T - 50,)
