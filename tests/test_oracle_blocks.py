"""Pins of the oracle's block-granular top-p (block_topp_head).

Block-granular selection is a reading (section 2.C: selected blocks are
moved into contiguous ranges): position-aligned blocks ranked by their
calibrated mass, the shortest prefix reaching p.  These tests hold the
oracle to that definition by routes that share none of its arithmetic:
token-level top-p at block size 1, brute force over every subset of blocks
(math.fsum masses), a uniform closed form, invariants, and reductions of the
whole step to torch's scaled_dot_product_attention.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle as O


def _bf16(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()


@pytest.mark.parametrize("seed", range(6))
def test_block_size_one_is_token_topp(seed):
    rng = np.random.default_rng(seed)
    n = 300
    c = np.float32(rng.standard_normal(n) * (1 + seed))
    c[::7] = c[3]                       # ties, broken by position either way
    w = np.exp(c.astype(np.float64) - c.max())
    Z = w.sum()
    for p in (0.3, 0.8, 0.95):
        tok = O.topp_head(c, w, Z, p)
        blk = O.block_topp_head(w, Z, p, np.arange(n), 1)
        assert np.array_equal(blk.selected, tok.selected)
        assert blk.k == tok.k


def _brute_blocks(bmass, p):
    """Minimal number of blocks reaching p * total, then the largest mass."""
    nb = len(bmass)
    total = math.fsum(bmass)
    target = float(np.float32(p)) * total
    for k in range(1, nb + 1):
        best = None
        for sub in itertools.combinations(range(nb), k):
            m = math.fsum(bmass[i] for i in sub)
            if m >= target and (best is None or m > best[0]):
                best = (m, sub)
        if best is not None:
            return set(best[1])
    return set(range(nb))


@pytest.mark.parametrize("seed,bs,start", [(1, 4, 0), (2, 8, 3), (3, 16, 5), (4, 2, 1)])
def test_brute_force_over_block_subsets(seed, bs, start):
    rng = np.random.default_rng(seed)
    pos = start + np.arange(bs * 9 + 3)       # partial blocks at both ends when start > 0
    w = np.exp(rng.standard_normal(len(pos)) * 2.0)
    Z = w.sum()
    for p in (0.25, 0.6, 0.9):
        blk = O.block_topp_head(w, Z, p, pos, bs)
        ids = pos // bs
        uniq = np.unique(ids)
        bmass = [math.fsum(w[ids == b]) for b in uniq]
        want = _brute_blocks(bmass, p)
        got = set(np.searchsorted(uniq, np.unique(ids[blk.selected])).tolist())
        assert got == want, (p, got, want)


def test_uniform_weights_closed_form():
    bs, nb = 16, 40
    pos = np.arange(bs * nb)
    w = np.ones(len(pos))
    for p in (0.1, 0.5, 0.77, 0.95):
        blk = O.block_topp_head(w, w.sum(), p, pos, bs)
        k = math.ceil(float(np.float32(p)) * nb)
        assert blk.k == k
        assert np.array_equal(blk.selected, np.arange(k * bs))     # lowest block ids first
    # a partial first block (candidates start mid-block) has less mass: last in rank
    pos2 = np.arange(5, bs * nb)
    blk = O.block_topp_head(np.ones(len(pos2)), len(pos2), 0.999, pos2, bs)
    assert blk.blocks[blk.order[-1]] == 0


def test_invariants_and_nesting():
    rng = np.random.default_rng(9)
    pos = 37 + np.arange(2000)
    c = np.float32(rng.standard_normal(len(pos)) * 2)
    w = np.exp(c.astype(np.float64) - c.max())
    Z = w.sum()
    prev = set()
    for p in (0.2, 0.5, 0.8, 0.95, 0.999):
        blk = O.block_topp_head(w, Z, p, pos, 16)
        sel = set(blk.selected.tolist())
        ids = pos // 16
        kept_blocks = set(ids[blk.selected].tolist())
        # whole blocks only
        assert sel == set(np.nonzero(np.isin(ids, list(kept_blocks)))[0].tolist())
        mass = w[blk.selected].sum()
        assert mass >= float(np.float32(p)) * Z * (1 - 1e-12)
        last = blk.blocks[blk.order[blk.k - 1]]
        assert mass - w[ids == last].sum() < float(np.float32(p)) * Z
        assert prev <= sel
        prev = sel
    assert O.block_topp_head(w, Z, 1.0, pos, 16).selected.size == len(pos)


def _sdpa(q, K, V):
    G = q.shape[0]
    qt = torch.tensor(np.asarray(q, np.float64))[None, :, None, :]
    kt = torch.tensor(np.asarray(K, np.float64))[None, None].expand(1, G, -1, -1).contiguous()
    vt = torch.tensor(np.asarray(V, np.float64))[None, None].expand(1, G, -1, -1).contiguous()
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, :, 0].numpy()


@pytest.mark.parametrize("metric", [O.METRIC_QK, O.METRIC_L2, O.METRIC_RKV])
def test_step_reduces_to_full_attention(metric):
    rng = np.random.default_rng(10)
    G, d, T = 4, 64, 500
    q = _bf16(rng.standard_normal((G, d)))
    K = _bf16(rng.standard_normal((T, d)))
    V = _bf16(rng.standard_normal((T, d)))
    ref = _sdpa(q, K, V)
    for C, p, S in ((32, 1.0, 0), (1, 0.4, 0), (1, 0.6, 3)):
        r = O.step_head(q, K, V, T, 60, C, p, metric, sinks=S, select_block=16)
        assert np.allclose(r.out, ref, rtol=1e-12, atol=1e-13), (C, p, S)
        # whole blocks of absolute positions kept
        ids = r.pos // 16
        cand = S + np.arange(r.A)
        kept = np.isin(cand // 16, ids)
        assert np.array_equal(np.nonzero(kept)[0] + S, r.pos)
