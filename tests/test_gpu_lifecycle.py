"""GPU parity of the multi-step token lifecycle (hardkv_step_inplace):
dense ring -> sparse pool (re-selected every step, compacted in place) ->
condensed running chunk sums, against the oracle's lifecycle step by step.

Per step and head: pool positions equal (borderline tokens allowed, counted,
and the oracle then re-synchronised from the GPU state, as a staged check),
pool rows bit copies of the source tokens, chunk counts exact, chunk sums
within 1e-5 * sum|x| over the chunk's tokens, ring contents exact,
attention within 2e-3.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from decode_kv_cache_head_amd import hardkv as H

from parity import ATTN_TOL, borderline_tokens

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


class Run:
    """Seeded lifecycle inputs and the GPU state for one layer."""

    def __init__(self, dev, seed, B, Hq, Hkv, d, T0, W, C, p, steps, dtype=torch.bfloat16,
                 pool_block=0, pool_blocks=None, metric=None):
        g = torch.Generator(device=dev).manual_seed(seed)
        self.B, self.Hq, self.Hkv, self.d, self.T0, self.W, self.C, self.p = B, Hq, Hkv, d, T0, W, C, p
        self.G = Hq // Hkv
        self.dt = dtype
        self.metrics = tuple(metric) if metric else (O.METRIC_QK,) * Hkv
        self.metric = (torch.tensor(self.metrics, dtype=torch.int8, device=dev)
                       if metric else None)
        Tmax = T0 + steps
        self.K = torch.randn((B, Hkv, T0, d), generator=g, device=dev).to(dtype)
        self.V = torch.randn((B, Hkv, T0, d), generator=g, device=dev).to(dtype)
        self.knew = torch.randn((steps, B, Hkv, d), generator=g, device=dev).to(dtype)
        self.vnew = torch.randn((steps, B, Hkv, d), generator=g, device=dev).to(dtype)
        self.q = (torch.randn((steps, B, Hq, d), generator=g, device=dev) * 1.5).to(dtype)
        self.desc = H.make_desc(B, Hq, Hkv, d, H.BF16 if dtype == torch.bfloat16 else H.F32,
                                W, C, p, Tmax)
        A = T0 - W
        tiers = H.alloc_tiers(self.desc, dev, zero=True)
        tiers.k[:, :, :A] = self.K[:, :, :A]
        tiers.v[:, :, :A] = self.V[:, :, :A]
        tiers.pos[:, :, :A] = torch.arange(A, dtype=torch.int32, device=dev)
        tiers.count.fill_(A)
        ring_k = torch.empty((B, Hkv, W, d), dtype=dtype, device=dev)
        ring_v = torch.empty_like(ring_k)
        for t in range(T0 - W, T0):
            ring_k[:, :, t % W] = self.K[:, :, t]
            ring_v[:, :, t % W] = self.V[:, :, t]
        seq = torch.full((B,), T0, dtype=torch.int32, device=dev)
        if pool_block:
            maxb = -(-self.desc.sparse_cap // pool_block)
            nblk = pool_blocks if pool_blocks is not None else B * Hkv * maxb
            self.state = H.paged_state(self.desc, self.K[:, :, :A], self.V[:, :, :A], ring_k,
                                       ring_v, seq, pool_block, nblk)
        else:
            self.state = H.State(ring_k, ring_v, tiers, seq)
        self.ws = H.alloc_workspace(self.desc, dev)
        self.out = torch.empty((B, Hq, d), device=dev)

    def oracle_state(self, b, h):
        K = self.K[b, h].float().cpu().numpy()
        V = self.V[b, h].float().cpu().numpy()
        return O.init_state(K, V, self.T0, self.W, self.C, self.desc.chunk_cap)

    def gpu_step(self, s):
        H.step_inplace(self.desc, self.q[s], self.knew[s], self.vnew[s], self.metric, self.state,
                       self.out, self.ws)
        torch.cuda.synchronize()


def add_abs(st, rows, positions):
    """Adds |x| of the given tokens to their chunks' sum|x| scale: after a
    borderline difference the GPU's chunks may hold a token the oracle kept,
    so the scale covers the differing tokens on both sides."""
    for r, t in zip(np.abs(np.asarray(rows, np.float64)), positions):
        j = int(t) // st.C
        st.kabs[j] += r[0]
        st.vabs[j] += r[1]


def resync(st, run, b, h, diff_rows=None, diff_pos=()):
    """Oracle state of (b, h) from the GPU tiers (staged comparison)."""
    t = run.state.tiers
    n = int(t.count[b, h])
    if diff_rows is not None:
        add_abs(st, diff_rows, diff_pos)
    st.pool_K = run.state.pool_rows(b, h, "k").float().cpu().numpy()
    st.pool_V = run.state.pool_rows(b, h, "v").float().cpu().numpy()
    st.pool_pos = t.pos[b, h, :n].cpu().numpy().astype(np.int64)
    st.ksum = t.ksum[b, h].double().cpu().numpy()
    st.vsum = t.vsum[b, h].double().cpu().numpy()
    st.cnt = t.ccount[b, h].cpu().numpy().astype(np.int64)


def check_blocks(state):
    """Block manager invariants: each head holds exactly ceil(count / bs)
    blocks (its first table entries), ids are distinct, and the held and the
    free blocks together are the whole pool."""
    if not state.pool_block:
        return
    bs = state.pool_block
    tab = state.pool_table.cpu().numpy()
    cnt = state.tiers.count.cpu().numpy()
    held = []
    for b in range(tab.shape[0]):
        for h in range(tab.shape[1]):
            need = -(-int(cnt[b, h]) // bs)
            assert (tab[b, h, :need] >= 0).all() and (tab[b, h, need:] == -1).all(), (b, h)
            held += tab[b, h, :need].tolist()
    top = int(state.free_top.item())
    free = state.free_ids[:top].cpu().numpy().tolist()
    nblk = state.free_ids.numel()
    assert len(set(held)) == len(held) and len(set(free)) == len(free)
    assert not set(held) & set(free)
    assert len(held) + top == nblk
    assert all(0 <= x < nblk for x in held + free)


def check_step(run, states, s, rep):
    t = run.state.tiers
    G, W = run.G, run.W
    P = run.T0 + s
    assert torch.all(run.state.seq_len == P + 1)
    for (b, h), st in states.items():
        pool_before = st.pool_pos.copy()
        q = run.q[s, b, h * G:(h + 1) * G].float().cpu().numpy().astype(np.float64)
        kn = run.knew[s, b, h].float().cpu().numpy()
        vn = run.vnew[s, b, h].float().cpu().numpy()
        out_ref, info = O.lifecycle_step(st, q, kn, vn, run.p, run.metrics[h])
        n = int(t.count[b, h])
        pos = t.pos[b, h, :n].cpu().numpy().astype(np.int64)
        diff = np.setxor1d(pos, st.pool_pos)
        rep["selected"] += n
        rep["candidates"] += info["n_candidates"]
        if diff.size:
            # rank the differing tokens in the oracle's own selection
            cand_pos = np.concatenate([pool_before, [P - W]])
            idx = np.searchsorted(cand_pos, diff)
            ref = O.HeadResult(len(cand_pos), None, None, info["cal"], info["sel"], None, None,
                               None, None, None, None, None, None)
            assert borderline_tokens(ref, run.p, idx).all(), (s, b, h, diff[:8])
            rep["borderline"] += int(diff.size)
            rows = np.stack([np.concatenate([run.K[b, h].float().cpu().numpy(),
                                             run.knew[:s + 1, b, h].float().cpu().numpy()]),
                             np.concatenate([run.V[b, h].float().cpu().numpy(),
                                             run.vnew[:s + 1, b, h].float().cpu().numpy()])],
                            axis=1)[diff]
            resync(st, run, b, h, rows, diff)
            rep["resyncs"] += 1
        # pool rows are bit copies of the tokens at their positions
        src_k = np.concatenate([run.K[b, h].float().cpu().numpy(),
                                run.knew[:s + 1, b, h].float().cpu().numpy()])
        assert np.array_equal(run.state.pool_rows(b, h, "k").float().cpu().numpy(), src_k[pos])
        assert np.array_equal(t.pos[b, h, :n].cpu().numpy(), st.pool_pos)
        cc = t.ccount[b, h].cpu().numpy()
        assert np.array_equal(cc, st.cnt)
        assert np.all(np.abs(t.ksum[b, h].double().cpu().numpy() - st.ksum) <=
                      1e-5 * st.kabs + 1e-30)
        assert np.all(np.abs(t.vsum[b, h].double().cpu().numpy() - st.vsum) <=
                      1e-5 * st.vabs + 1e-30)
        rk = run.state.ring_k[b, h].float().cpu().numpy()
        assert np.array_equal(rk, st.ring_K)
        o = run.out[b, h * G:(h + 1) * G].double().cpu().numpy()
        if diff.size:
            out_ref = O.attend_head(q, st.ring_K, st.ring_V, st.pool_K, st.pool_V, st.ksum,
                                    st.vsum, st.cnt)
        err = np.abs(o - out_ref).max(axis=1) / np.abs(out_ref).max(axis=1)
        assert np.all(err <= ATTN_TOL), (s, b, h, err.max())
        rep["max_attn_err"] = max(rep["max_attn_err"], float(err.max()))
    check_blocks(run.state)


@pytest.mark.parametrize("cfg", [
    dict(B=2, Hq=16, Hkv=2, d=128, T0=1500, W=512, C=64, p=0.95, steps=12),
    dict(B=3, Hq=8, Hkv=4, d=64, T0=700, W=100, C=7, p=0.8, steps=9),
    dict(B=1, Hq=4, Hkv=4, d=128, T0=300, W=64, C=1, p=0.5, steps=6, dtype=torch.float32),
    # chunks wider than a compaction sub-tile (128 bf16 rows): running sums
    # carried across sub-tiles
    dict(B=2, Hq=8, Hkv=2, d=128, T0=1400, W=64, C=300, p=0.9, steps=5),
    # the pool under the head-wise block manager
    dict(B=2, Hq=16, Hkv=2, d=128, T0=1500, W=512, C=64, p=0.95, steps=12, pool_block=64),
    dict(B=3, Hq=8, Hkv=4, d=64, T0=700, W=100, C=7, p=0.8, steps=9, pool_block=16),
    dict(B=1, Hq=4, Hkv=4, d=128, T0=300, W=64, C=1, p=0.5, steps=6, dtype=torch.float32,
         pool_block=32),
    dict(B=2, Hq=8, Hkv=2, d=128, T0=1400, W=64, C=300, p=0.9, steps=5, pool_block=128),
    # key-norm heads beside QK heads, calibrated onto the logit spread
    dict(B=2, Hq=16, Hkv=4, d=128, T0=1200, W=128, C=64, p=0.9, steps=8,
         metric=(O.METRIC_QK, O.METRIC_L2, O.METRIC_L2, O.METRIC_QK)),
    dict(B=3, Hq=8, Hkv=2, d=64, T0=600, W=64, C=16, p=0.85, steps=8, pool_block=32,
         metric=(O.METRIC_L2, O.METRIC_QK)),
    # key-dissimilarity heads: the key sum of each step's pool formed first
    dict(B=2, Hq=16, Hkv=4, d=128, T0=2600, W=128, C=64, p=0.9, steps=6,
         metric=(O.METRIC_KEYDIFF, O.METRIC_QK, O.METRIC_L2, O.METRIC_KEYDIFF)),
    dict(B=2, Hq=8, Hkv=2, d=64, T0=900, W=64, C=16, p=0.85, steps=6, pool_block=32,
         metric=(O.METRIC_QK, O.METRIC_KEYDIFF)),
    # R-KV redundancy heads: the unit-key sum of each step's pool formed first
    dict(B=2, Hq=16, Hkv=4, d=128, T0=2000, W=128, C=64, p=0.9, steps=6,
         metric=(O.METRIC_RKV, O.METRIC_QK, O.METRIC_RKV, O.METRIC_KEYDIFF)),
    dict(B=2, Hq=8, Hkv=2, d=64, T0=900, W=64, C=16, p=0.85, steps=6, pool_block=32,
         metric=(O.METRIC_RKV, O.METRIC_L2)),
])
def test_lifecycle_matches_oracle(gpu, cfg):
    steps = cfg.pop("steps")
    run = Run(gpu, 11, steps=steps, **cfg)
    say("lifecycle", cfg, "steps", steps)
    states = {(b, h): run.oracle_state(b, h) for b in range(run.B) for h in range(run.Hkv)}
    rep = dict(selected=0, candidates=0, borderline=0, resyncs=0, max_attn_err=0.0)
    for s in range(steps):
        run.gpu_step(s)
        check_step(run, states, s, rep)
    say(rep)
    # tokens keep flowing dense -> sparse -> condensed
    assert int(run.state.tiers.ccount.sum()) > 0


def test_block_manager_returns_blocks_and_runs_out_gracefully(gpu):
    """p = 1 keeps every token, so the pools only grow; with one spare block
    the first requester in (b, h) order takes it and the other heads' aged
    tokens go straight into their chunks.  Nothing is lost, the run is
    deterministic, and with fresh random queries (p = 0.9) the blocks the
    compaction empties return to the stack."""
    cfg = dict(B=2, Hq=8, Hkv=2, d=128, T0=700, W=64, C=32, steps=12, pool_block=16)
    A = 700 - 64                      # 636 rows: 40 blocks per head, 4 rows free in the last
    runs = [Run(gpu, 31, p=1.0, pool_blocks=4 * 40 + 1, **cfg) for _ in range(2)]
    for s in range(12):
        for r in runs:
            r.gpu_step(s)
        a, b_ = runs[0].state, runs[1].state
        assert torch.equal(a.tiers.count, b_.tiers.count) and torch.equal(a.pool_table, b_.pool_table)
        assert torch.equal(a.tiers.ccount, b_.tiers.ccount) and torch.equal(a.tiers.ksum, b_.tiers.ksum)
        aged = 700 + s + 1 - 64
        total = a.tiers.count + a.tiers.ccount.sum(-1)
        assert torch.all(total == aged), (s, total.tolist())
        check_blocks(a)
    cnt = runs[0].state.tiers.count.cpu().tolist()
    # head (0, 0) got the spare block at step 5 (row 640) and keeps growing
    assert cnt[0][0] == A + 12 and cnt[0][1] == cnt[1][0] == cnt[1][1] == 640
    assert int(runs[0].state.free_top.item()) == 0
    # compaction under fresh random queries empties blocks, which return
    run = Run(gpu, 32, p=0.9, **cfg)
    before = run.state.blocks_held()
    for s in range(12):
        run.gpu_step(s)
        check_blocks(run.state)
    assert run.state.blocks_held() < before // 2
    assert int(run.state.free_top.item()) == run.state.free_ids.numel() - run.state.blocks_held()


def test_lifecycle_p_one_keeps_everything(gpu):
    run = Run(gpu, 12, B=2, Hq=8, Hkv=2, d=128, T0=600, W=128, C=32, p=1.0, steps=5)
    for s in range(5):
        run.gpu_step(s)
    assert torch.all(run.state.tiers.count == 600 - 128 + 5)
    assert int(run.state.tiers.ccount.sum()) == 0


def test_first_lifecycle_step_equals_single_step(gpu):
    """Step 1 on the raw prefill equals hardkv_step on the cache that holds
    the new token: same kept set, same compacted rows, same attention."""
    run = Run(gpu, 13, B=2, Hq=16, Hkv=2, d=128, T0=2000, W=256, C=64, p=0.9, steps=1)
    run.gpu_step(0)
    T = run.T0 + 1
    k = torch.cat([run.K, run.knew[0][:, :, None]], dim=2).contiguous()
    v = torch.cat([run.V, run.vnew[0][:, :, None]], dim=2).contiguous()
    ctx = torch.full((run.B,), T, dtype=torch.int32, device=gpu)
    desc = H.make_desc(run.B, run.Hq, run.Hkv, run.d, H.BF16, run.W, run.C, run.p, T)
    tiers = H.alloc_tiers(desc, gpu)
    out = torch.empty_like(run.out)
    H.step(desc, run.q[0], H.cache_struct(k, v, ctx), None, tiers, out, H.alloc_workspace(desc, gpu))
    torch.cuda.synchronize()
    st = run.state.tiers
    assert torch.equal(st.count, tiers.count)
    for b in range(run.B):
        for h in range(run.Hkv):
            n = int(tiers.count[b, h])
            assert torch.equal(st.pos[b, h, :n], tiers.pos[b, h, :n])
            assert torch.equal(st.k[b, h, :n], tiers.k[b, h, :n])
            nch = -(-(T - run.W) // run.C)
            assert torch.equal(st.ccount[b, h, :nch], tiers.ccount[b, h, :nch])
    err = ((out - run.out).abs().amax(-1) / out.abs().amax(-1)).max().item()
    assert err < 1e-5


def snapshot(state):
    """Device copies of everything a lifecycle step reads from one layer."""
    t = state.tiers
    return dict(rk=state.ring_k.clone(), rv=state.ring_v.clone(), k=t.k.clone(), v=t.v.clone(),
                pos=t.pos.clone(), count=t.count.clone(), ksum=t.ksum.clone(),
                vsum=t.vsum.clone(), ccount=t.ccount.clone(), T=state.seq_len.clone())


def check_every_head(snap, state, q, kn, vn, out, W, C, p, rep):
    """Every (b, h) of one layer after one step, against the oracle's step
    from the state the GPU started from (snap): the kept positions (borderline
    tokens counted), the pool rows as bit copies, the chunk counts, the chunk
    sums within 1e-5 * (|old sum| + sum|x| of the tokens merged this step), the
    ring, and attention within the bf16 tolerance."""
    t = state.tiers
    B, Hkv = snap["count"].shape
    G = q.shape[1] // Hkv
    cnt0, cnt1 = snap["count"].cpu().numpy(), t.count.cpu().numpy()
    T = snap["T"].cpu().numpy()
    ks0, vs0 = snap["ksum"].double().cpu().numpy(), snap["vsum"].double().cpu().numpy()
    cc0 = snap["ccount"].cpu().numpy().astype(np.int64)
    ks1, vs1 = t.ksum.double().cpu().numpy(), t.vsum.double().cpu().numpy()
    cc1 = t.ccount.cpu().numpy().astype(np.int64)
    pos0, pos1 = snap["pos"].cpu().numpy(), t.pos.cpu().numpy()
    rk0, rv0 = snap["rk"].float().cpu().numpy(), snap["rv"].float().cpu().numpy()
    rk1 = state.ring_k.float().cpu().numpy()
    qa = q.float().cpu().numpy().astype(np.float64)
    kna, vna = kn.float().cpu().numpy(), vn.float().cpu().numpy()
    oa = out.double().cpu().numpy()
    for b in range(B):
        m0, m1 = int(cnt0[b].max()), int(cnt1[b].max())
        k0 = snap["k"][b, :, :m0].float().cpu().numpy()
        v0 = snap["v"][b, :, :m0].float().cpu().numpy()
        k1 = t.k[b, :, :m1].float().cpu().numpy()
        v1 = t.v[b, :, :m1].float().cpu().numpy()
        for h in range(Hkv):
            n0, n1 = int(cnt0[b, h]), int(cnt1[b, h])
            st = O.HeadState(W, C, rk0[b, h].copy(), rv0[b, h].copy(), k0[h, :n0], v0[h, :n0],
                             pos0[b, h, :n0].astype(np.int64), ks0[b, h].copy(),
                             vs0[b, h].copy(), cc0[b, h].copy(), int(T[b]),
                             np.abs(ks0[b, h]), np.abs(vs0[b, h]))
            pool_before = st.pool_pos.copy()
            qh = qa[b, h * G:(h + 1) * G]
            out_ref, info = O.lifecycle_step(st, qh, kna[b, h], vna[b, h], p, O.METRIC_QK)
            pos = pos1[b, h, :n1].astype(np.int64)
            diff = np.setxor1d(pos, st.pool_pos)
            rep["heads"] += 1
            assert np.array_equal(rk1[b, h], st.ring_K), (b, h)
            if diff.size:
                cand = np.concatenate([pool_before, [int(T[b]) - W]])
                ref = O.HeadResult(len(cand), None, None, info["cal"], info["sel"], None, None,
                                   None, None, None, None, None, None)
                assert borderline_tokens(ref, p, np.searchsorted(cand, diff)).all(), (b, h)
                rep["borderline"] += int(diff.size)
                # attention over the GPU's own tiers (the oracle's attention)
                out_ref = O.attend_head(qh, st.ring_K, st.ring_V, k1[h, :n1], v1[h, :n1],
                                        ks1[b, h], vs1[b, h], cc1[b, h])
            else:
                assert np.array_equal(k1[h, :n1], st.pool_K), (b, h)
                assert np.array_equal(v1[h, :n1], st.pool_V), (b, h)
                assert np.array_equal(cc1[b, h], st.cnt), (b, h)
                assert np.all(np.abs(ks1[b, h] - st.ksum) <= 1e-5 * st.kabs + 1e-30), (b, h)
                assert np.all(np.abs(vs1[b, h] - st.vsum) <= 1e-5 * st.vabs + 1e-30), (b, h)
            o = oa[b, h * G:(h + 1) * G]
            err = np.abs(o - out_ref).max(axis=1) / np.abs(out_ref).max(axis=1)
            assert np.all(err <= ATTN_TOL), (b, h, err.max())
            rep["max_attn_err"] = max(rep["max_attn_err"], float(err.max()))


def test_lifecycle_qwen32b_64_layers_256_steps(gpu):
    """Full-size lifecycle: Qwen3-32B attention shape (64 query heads, 8 KV
    heads, d=128), 64 layers with their own caches, 64 sequences starting at
    12288 tokens, 256 decode steps, window 512, chunk 64, p = 0.95.  Sampled
    (layer, sequence, head) triples follow the oracle step by step; at steps
    1, 50 and 256 every head of layers 0, 31 and 63 is checked against the
    oracle's step from the state the GPU started that step with; every head
    is checked for the token-count invariant at several steps."""
    L, B, Hq, Hkv, d, T0, W, C, p, steps = 64, 64, 64, 8, 128, 12288, 512, 64, 0.95, 256
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    need = (L + 1) * B * Hkv * ((T0 + steps - W) * d * 4 + W * d * 4 + 188 * d * 8) * 1.02
    if free < need:
        pytest.skip(f"needs {need / 2**30:.0f} GiB of device memory, {free / 2**30:.0f} free")
    desc = H.make_desc(B, Hq, Hkv, d, H.BF16, W, C, p, T0 + steps)
    A = T0 - W
    ws = H.alloc_workspace(desc, gpu)
    out = torch.empty((B, Hq, d), device=gpu)
    layers = []
    for layer in range(L):
        g = torch.Generator(device=gpu).manual_seed(1000 + layer)
        t = H.alloc_tiers(desc, gpu)
        for i in range(0, B, 8):   # draw in slices to bound the float32 temporaries
            t.k[i:i + 8, :, :A] = torch.randn((8, Hkv, A, d), generator=g, device=gpu).to(torch.bfloat16)
            t.v[i:i + 8, :, :A] = torch.randn((8, Hkv, A, d), generator=g, device=gpu).to(torch.bfloat16)
        t.pos[:, :, :A] = torch.arange(A, dtype=torch.int32, device=gpu)
        t.count.fill_(A)
        t.ksum.zero_()
        t.vsum.zero_()
        t.ccount.zero_()
        rk = torch.randn((B, Hkv, W, d), generator=g, device=gpu).to(torch.bfloat16)
        rv = torch.randn((B, Hkv, W, d), generator=g, device=gpu).to(torch.bfloat16)
        layers.append(H.State(rk, rv, t, torch.full((B,), T0, dtype=torch.int32, device=gpu)))
    say("allocated", L, "layers")
    samples = [(0, 0, 0), (17, 33, 5), (63, 63, 7)]
    states = {}
    for (layer, b, h) in samples:
        st = layers[layer]
        pk = st.tiers.k[b, h, :A].float().cpu().numpy()
        pv = st.tiers.v[b, h, :A].float().cpu().numpy()
        o = O.HeadState(W, C, st.ring_k[b, h].float().cpu().numpy(), st.ring_v[b, h].float().cpu().numpy(),
                        pk, pv, np.arange(A), np.zeros((desc.chunk_cap, d)), np.zeros((desc.chunk_cap, d)),
                        np.zeros(desc.chunk_cap, np.int64), T0, np.zeros((desc.chunk_cap, d)),
                        np.zeros((desc.chunk_cap, d)))
        states[(layer, b, h)] = o
    rep = dict(borderline=0, resyncs=0, max_attn_err=0.0)
    gq = torch.Generator(device=gpu).manual_seed(7)
    G = Hq // Hkv
    for s in range(steps):
        for layer in range(L):
            q = (torch.randn((B, Hq, d), generator=gq, device=gpu)).to(torch.bfloat16)
            kn = torch.randn((B, Hkv, d), generator=gq, device=gpu).to(torch.bfloat16)
            vn = torch.randn((B, Hkv, d), generator=gq, device=gpu).to(torch.bfloat16)
            full = layer in (0, 31, 63) and s in (0, 49, steps - 1)
            snap = snapshot(layers[layer]) if full else None
            H.step_inplace(desc, q, kn, vn, None, layers[layer], out, ws)
            if snap is not None:
                torch.cuda.synchronize()
                every = dict(heads=0, borderline=0, max_attn_err=0.0)
                check_every_head(snap, layers[layer], q, kn, vn, out, W, C, p, every)
                say(f"step {s + 1}: every head of layer {layer}", every)
                rep["borderline"] += every["borderline"]
                rep["max_attn_err"] = max(rep["max_attn_err"], every["max_attn_err"])
                del snap
            for (ly, b, h), st in states.items():
                if ly != layer:
                    continue
                torch.cuda.synchronize()
                qh = q[b, h * G:(h + 1) * G].float().cpu().numpy().astype(np.float64)
                pool_before = st.pool_pos.copy()
                o_ref, info = O.lifecycle_step(st, qh, kn[b, h].float().cpu().numpy(),
                                               vn[b, h].float().cpu().numpy(), p, O.METRIC_QK)
                t = layers[layer].tiers
                n = int(t.count[b, h])
                pos = t.pos[b, h, :n].cpu().numpy().astype(np.int64)
                diff = np.setxor1d(pos, st.pool_pos)
                if diff.size:
                    P = T0 + s
                    cand = np.concatenate([pool_before, [P - W]])
                    ref = O.HeadResult(len(cand), None, None, info["cal"], info["sel"], None, None,
                                       None, None, None, None, None, None)
                    assert borderline_tokens(ref, p, np.searchsorted(cand, diff)).all()
                    rep["borderline"] += int(diff.size)
                    # |x| of the differing tokens: kept by the GPU (its pool
                    # rows) or by the oracle (its pool rows before the resync)
                    for tpos in diff:
                        if tpos in pos:
                            i = int(np.searchsorted(pos, tpos))
                            rk, rv = t.k[b, h, i], t.v[b, h, i]
                            rk, rv = rk.float().cpu().numpy(), rv.float().cpu().numpy()
                        else:
                            i = int(np.searchsorted(st.pool_pos, tpos))
                            rk, rv = st.pool_K[i], st.pool_V[i]
                        add_abs(st, [np.stack([rk, rv])], [tpos])
                    st.pool_K = t.k[b, h, :n].float().cpu().numpy()
                    st.pool_V = t.v[b, h, :n].float().cpu().numpy()
                    st.pool_pos = pos
                    st.ksum = t.ksum[b, h].double().cpu().numpy()
                    st.vsum = t.vsum[b, h].double().cpu().numpy()
                    st.cnt = t.ccount[b, h].cpu().numpy().astype(np.int64)
                    o_ref = O.attend_head(qh, st.ring_K, st.ring_V, st.pool_K, st.pool_V, st.ksum,
                                          st.vsum, st.cnt)
                    rep["resyncs"] += 1
                assert np.array_equal(t.ccount[b, h].cpu().numpy(), st.cnt)
                if s % 32 == 0 or s == steps - 1:
                    assert np.array_equal(t.k[b, h, :n].float().cpu().numpy(), st.pool_K)
                    assert np.all(np.abs(t.ksum[b, h].double().cpu().numpy() - st.ksum) <=
                                  1e-5 * st.kabs + 1e-30)
                    assert np.all(np.abs(t.vsum[b, h].double().cpu().numpy() - st.vsum) <=
                                  1e-5 * st.vabs + 1e-30)
                og = out[b, h * G:(h + 1) * G].double().cpu().numpy()
                err = np.abs(og - o_ref).max(axis=1) / np.abs(o_ref).max(axis=1)
                assert np.all(err <= ATTN_TOL), (s, layer, b, h, err.max())
                rep["max_attn_err"] = max(rep["max_attn_err"], float(err.max()))
        if s in (0, 1, 9, 19, 49, steps - 1):
            torch.cuda.synchronize()
            P1 = T0 + s + 1
            for layer in (0, 31, 63):
                t = layers[layer].tiers
                tot = t.count.long() + t.ccount.long().sum(-1) + W
                assert torch.all(tot == P1), (s, layer)
                assert torch.all(layers[layer].seq_len == P1)
            pool = layers[0].tiers.count.float().mean().item()
            say(f"step {s + 1}: mean pool size {pool:.0f} (layer 0)", rep)
    say(rep)
    del layers, ws
    torch.cuda.empty_cache()
