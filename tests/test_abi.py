"""C ABI checks that need no GPU: the library loads, exports every entry
point include/hardkv.h declares, and rejects bad arguments with the
documented codes before launching anything."""
import ctypes
import os
import re

import pytest

from decode_kv_cache_head_amd import hardkv as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "hardkv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hardkv_\w+)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = H.load()
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(H.EXPORTS)


def test_version_and_strerror():
    lib = H.load()
    assert lib.hardkv_version() == 10900
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.hardkv_strerror(code)
    assert lib.hardkv_strerror(99) == b"unknown error"


def base_desc(**kw):
    d = dict(B=2, Hq=8, Hkv=2, d=128, dtype=H.BF16, W=64, C=32, top_p=0.9, ctx_cap=1000)
    d.update(kw)
    return H.make_desc(d["B"], d["Hq"], d["Hkv"], d["d"], d["dtype"], d["W"], d["C"], d["top_p"],
                       d["ctx_cap"], d.get("block_size", 0), d.get("max_blocks", 0),
                       d.get("sparse_cap"), d.get("chunk_cap"), d.get("sinks", 0),
                       d.get("merge", 0), d.get("packed_rows", 0), d.get("obs_window", 1),
                       d.get("pool_radius", 0), d.get("calibration", 0),
                       d.get("select_block", 0), d.get("tier_block", 0),
                       d.get("tier_blocks", 0))


@pytest.mark.parametrize("kw,code", [
    ({}, H.OK),
    (dict(Hq=7), H.ERR_INVALID_ARG),
    (dict(Hq=6, Hkv=2), H.ERR_UNSUPPORTED),      # G = 3
    (dict(Hq=32, Hkv=2), H.ERR_UNSUPPORTED),     # G = 16
    (dict(d=96), H.ERR_UNSUPPORTED),
    (dict(dtype=7), H.ERR_UNSUPPORTED),
    (dict(W=-1), H.ERR_INVALID_ARG),
    (dict(C=0), H.ERR_INVALID_ARG),
    (dict(top_p=0.0), H.ERR_INVALID_ARG),
    (dict(top_p=1.5), H.ERR_INVALID_ARG),
    (dict(top_p=float("nan")), H.ERR_INVALID_ARG),
    (dict(top_p=1.0), H.OK),
    (dict(sparse_cap=935), H.ERR_CAPACITY),
    (dict(chunk_cap=29), H.ERR_CAPACITY),
    (dict(chunk_cap=30), H.OK),
    (dict(block_size=16, max_blocks=63), H.OK),
    (dict(block_size=16, max_blocks=62), H.ERR_INVALID_ARG),
    (dict(block_size=12, max_blocks=100), H.ERR_UNSUPPORTED),
    (dict(B=0), H.ERR_INVALID_ARG),
    (dict(ctx_cap=0), H.ERR_INVALID_ARG),
    (dict(W=2000), H.OK),                          # everything dense
    (dict(sinks=4), H.OK),
    (dict(sinks=-1), H.ERR_INVALID_ARG),
    (dict(sinks=100, sparse_cap=835), H.ERR_CAPACITY),  # 1000 - 64 - 100 = 836 candidates
    (dict(sinks=100, sparse_cap=836), H.OK),
    (dict(sinks=2000), H.OK),                      # sinks and window cover everything
    (dict(merge=1), H.OK),
    (dict(merge=2), H.ERR_INVALID_ARG),
    (dict(packed_rows=100), H.OK),
    (dict(packed_rows=-1), H.ERR_INVALID_ARG),
    (dict(B=1 << 18, Hkv=16, Hq=16, packed_rows=1), H.ERR_INVALID_ARG),  # offsets past int32
    (dict(obs_window=0), H.OK),
    (dict(obs_window=64, pool_radius=512), H.OK),
    (dict(obs_window=65), H.ERR_INVALID_ARG),
    (dict(pool_radius=513), H.ERR_INVALID_ARG),
    (dict(pool_radius=-1), H.ERR_INVALID_ARG),
    (dict(calibration=H.CALIB_ENTROPY), H.OK),
    (dict(calibration=2), H.ERR_INVALID_ARG),
    (dict(calibration=-1), H.ERR_INVALID_ARG),
    (dict(select_block=16), H.OK),
    (dict(select_block=1), H.OK),
    (dict(select_block=1024), H.OK),
    (dict(select_block=12), H.ERR_INVALID_ARG),
    (dict(select_block=-16), H.ERR_INVALID_ARG),
    (dict(select_block=2048), H.ERR_INVALID_ARG),
    # at most 4096 blocks per head: ceil(A / bs) + 1
    (dict(ctx_cap=4095 + 64, select_block=1), H.OK),
    (dict(ctx_cap=4096 + 64, select_block=1), H.ERR_UNSUPPORTED),
    (dict(ctx_cap=65520 + 256, W=256, select_block=16), H.OK),
    (dict(ctx_cap=65536 + 256, W=256, select_block=16), H.ERR_UNSUPPORTED),
    (dict(tier_block=16, tier_blocks=100), H.OK),
    (dict(tier_block=1024, tier_blocks=1), H.OK),
    (dict(tier_block=8, tier_blocks=100), H.ERR_INVALID_ARG),
    (dict(tier_block=48, tier_blocks=100), H.ERR_INVALID_ARG),
    (dict(tier_block=2048, tier_blocks=100), H.ERR_INVALID_ARG),
    (dict(tier_block=16, tier_blocks=0), H.ERR_INVALID_ARG),
    (dict(tier_block=16, tier_blocks=1 << 27), H.ERR_INVALID_ARG),
    (dict(tier_block=16, tier_blocks=100, packed_rows=500), H.ERR_INVALID_ARG),
    (dict(B=2049, Hkv=8, Hq=8, tier_block=16, tier_blocks=100), H.ERR_UNSUPPORTED),
    (dict(B=2048, Hkv=8, Hq=8, tier_block=16, tier_blocks=100), H.OK),
    (dict(B=2048, Hkv=8, Hq=8), H.OK),
])
def test_validate_codes(kw, code):
    assert H.validate(base_desc(**kw)) == code


def test_workspace_size():
    d = base_desc()
    n = H.workspace_size(d)
    assert n > 0 and n % 256 == 0
    assert H.workspace_size(base_desc(Hq=7)) == 0
    big = base_desc(ctx_cap=4000)
    assert H.workspace_size(big) > n


ENTRY_POINTS = ("score", "calibrate", "topp_select", "compact", "decode_attn", "step",
                "step_inplace", "step_policy")
# the entry points that take a query pointer
TAKES_Q = ("score", "decode_attn", "step", "step_inplace", "step_policy")


def _call_all(desc, ws_bytes, null_q=False, only=ENTRY_POINTS):
    """Calls the named entry points with fake (never dereferenced) device
    pointers and returns their codes in ENTRY_POINTS order.  Every call made
    here must fail validation: a call whose arguments all pass would enqueue
    kernels on the fake pointers, so callers pass only the entry points that
    the argument under test makes invalid (with null_q, those taking q)."""
    lib = H.load()
    fake = ctypes.c_void_p(0x1000)
    cache = H.Cache(fake, fake, None, fake)
    tiers = H.TiersC(*([fake] * 9))
    state = H.StateC(fake, fake, H.TiersC(*([fake] * 7)), fake)
    pol = H.policy(H.POLICY_MTI, 4)
    q = None if null_q else fake
    d = ctypes.byref(desc)
    st = ctypes.c_void_p(0)
    calls = {
        "score": lambda: lib.hardkv_score(d, q, ctypes.byref(cache), None, fake, None, fake,
                                          ws_bytes, st),
        "calibrate": lambda: lib.hardkv_calibrate(d, fake, None, fake, None, fake, fake,
                                                  ws_bytes, st),
        "topp_select": lambda: lib.hardkv_topp_select(d, fake, None, fake, None, fake, fake,
                                                      fake, fake, ws_bytes, st),
        "compact": lambda: lib.hardkv_compact(d, ctypes.byref(cache), fake, ctypes.byref(tiers),
                                              fake, ws_bytes, st),
        "decode_attn": lambda: lib.hardkv_decode_attn(d, q, ctypes.byref(cache),
                                                      ctypes.byref(tiers), fake, fake, ws_bytes,
                                                      st),
        "step": lambda: lib.hardkv_step(d, q, ctypes.byref(cache), None, ctypes.byref(tiers),
                                        fake, fake, ws_bytes, st),
        "step_inplace": lambda: lib.hardkv_step_inplace(d, q, fake, fake, None,
                                                        ctypes.byref(state), fake, fake,
                                                        ws_bytes, st),
        "step_policy": lambda: lib.hardkv_step_policy(d, ctypes.byref(pol), q,
                                                      ctypes.byref(cache), None,
                                                      ctypes.byref(tiers), fake, fake, ws_bytes,
                                                      st),
    }
    assert set(only) <= set(ENTRY_POINTS)
    return [calls[n]() for n in ENTRY_POINTS if n in only]


def test_errors_before_launch():
    desc = base_desc()
    need = H.workspace_size(desc)
    assert _call_all(desc, need - 1) == [H.ERR_WORKSPACE] * 8
    assert _call_all(base_desc(d=96), need) == [H.ERR_UNSUPPORTED] * 8
    assert _call_all(base_desc(top_p=2.0), need) == [H.ERR_INVALID_ARG] * 8
    assert _call_all(base_desc(sparse_cap=10), need) == [H.ERR_CAPACITY] * 8
    # a null query: only the entry points that take one are called, and every
    # one of them must refuse
    assert _call_all(desc, need, null_q=True, only=TAKES_Q) == [H.ERR_INVALID_ARG] * len(TAKES_Q)
    # the lifecycle needs a contiguous layout and a window (the single-step
    # calls accept a paged descriptor, so they are not called here)
    paged = base_desc(block_size=16, max_blocks=63)
    assert _call_all(paged, H.workspace_size(paged), only=("step_inplace",)) == \
        [H.ERR_INVALID_ARG]
    lib = H.load()
    assert lib.hardkv_validate(None) == H.ERR_INVALID_ARG
    assert lib.hardkv_workspace_size(None) == 0


def test_noalloc_step_errors_before_launch():
    """hardkv_step_noalloc refuses, before touching any device, a descriptor
    whose workspace exceeds the library-held array and every missing
    argument."""
    lib = H.load()
    fake = ctypes.c_void_p(0x1000)
    cache = H.Cache(fake, fake, None, fake)
    tiers = H.TiersC(*([fake] * 9))
    st = ctypes.c_void_p(0)
    # 32 sequences x 8 heads x 32k tokens: 106 MiB of workspace
    big = base_desc(B=32, Hq=32, Hkv=8, W=256, C=64, ctx_cap=32768)
    assert H.workspace_size(big) > H.SCRATCH_BYTES
    assert lib.hardkv_step_noalloc(ctypes.byref(big), fake, ctypes.byref(cache), None,
                                   ctypes.byref(tiers), fake, st) == H.ERR_WORKSPACE
    # the headline shape fits
    head = base_desc(B=32, Hq=32, Hkv=8, W=256, C=64, ctx_cap=16384, block_size=16,
                     max_blocks=1024)
    assert H.workspace_size(head) <= H.SCRATCH_BYTES
    d = ctypes.byref(base_desc())
    no_ccount = H.TiersC(*([fake] * 6), None)
    for args in ((None, cache, tiers, fake), (fake, H.Cache(fake, None, None, fake), tiers, fake),
                 (fake, cache, no_ccount, fake), (fake, cache, tiers, None)):
        q, c, t, out = args
        assert lib.hardkv_step_noalloc(d, q, ctypes.byref(c), None, ctypes.byref(t), out,
                                       st) == H.ERR_INVALID_ARG
    assert lib.hardkv_step_noalloc(ctypes.byref(base_desc(d=96)), fake, ctypes.byref(cache), None,
                                   ctypes.byref(tiers), fake, st) == H.ERR_UNSUPPORTED


def test_l2_buffer_required_with_metric():
    desc = base_desc()
    lib = H.load()
    fake = ctypes.c_void_p(0x1000)
    cache = H.Cache(fake, fake, None, fake)
    rc = lib.hardkv_score(ctypes.byref(desc), fake, ctypes.byref(cache), fake, fake, None, fake,
                          H.workspace_size(desc), ctypes.c_void_p(0))
    assert rc == H.ERR_INVALID_ARG


def test_policy_errors_before_launch():
    lib = H.load()
    desc = base_desc()
    ws_bytes = H.workspace_size(desc)
    fake = ctypes.c_void_p(0x1000)
    cache = H.Cache(fake, fake, None, fake)
    st = ctypes.c_void_p(0)
    d = ctypes.byref(desc)
    with_mode = H.TiersC(*([fake] * 8))
    no_mode = H.TiersC(*([fake] * 7))

    def step_policy(pol, tiers):
        return lib.hardkv_step_policy(d, pol, fake, ctypes.byref(cache), None,
                                      ctypes.byref(tiers), fake, fake, ws_bytes, st)

    for bad in (H.policy(3), H.policy(-1), H.policy(H.POLICY_MTI, 0)):
        assert step_policy(ctypes.byref(bad), with_mode) == H.ERR_INVALID_ARG
        assert lib.hardkv_plan(d, ctypes.byref(bad), fake, fake, fake, st) == H.ERR_INVALID_ARG
    assert step_policy(None, with_mode) == H.ERR_INVALID_ARG
    # the policy's choice needs somewhere to go
    assert step_policy(ctypes.byref(H.policy()), no_mode) == H.ERR_INVALID_ARG
    good = ctypes.byref(H.policy(H.POLICY_MTI, 8, 16, 1 << 20))
    for args in ((None, fake, fake), (fake, None, fake), (fake, fake, None)):
        assert lib.hardkv_plan(d, good, *args, st) == H.ERR_INVALID_ARG
    assert lib.hardkv_plan(ctypes.byref(base_desc(d=96)), good, fake, fake, fake, st) == \
        H.ERR_UNSUPPORTED
    # the lifecycle compacts in place: no per-head mode
    state = H.StateC(fake, fake, with_mode, fake)
    assert lib.hardkv_step_inplace(d, fake, fake, fake, None, ctypes.byref(state), fake, fake,
                                   ws_bytes, st) == H.ERR_INVALID_ARG


def test_host_plan_matches_oracle_reading():
    """The memory-time integrals documented with hardkv_policy in
    include/hardkv.h, evaluated in Python integers, agree with the oracle's."""
    import oracle as O
    for A, k, W, N in [(10, 2, 2, 3), (10, 2, 2, 2), (16128, 13548, 256, 22),
                       (16128, 13548, 256, 23), (16128, 60, 256, 2), (0, 0, 256, 5)]:
        sparse = (A + W) * (3 * A + 2 * W) + (N - 1) * (A + W) * 2 * (k + W)
        rewrite = (A + W + k) * (3 * A + 2 * W + 2 * k) + (N - 1) * (k + W) * 2 * (k + W)
        assert (rewrite, sparse) == O.mti_head(A, k, W, N)


def test_sinks_and_merge_errors_before_launch():
    lib = H.load()
    fake = ctypes.c_void_p(0x1000)
    cache = H.Cache(fake, fake, None, fake)
    tiers = H.TiersC(*([fake] * 7))
    st = ctypes.c_void_p(0)
    weighted = base_desc(merge=H.MERGE_WEIGHTED)
    need = H.workspace_size(weighted)
    d = ctypes.byref(weighted)
    # weighted merging needs the scores: plain hardkv_compact refuses it
    assert lib.hardkv_compact(d, ctypes.byref(cache), fake, ctypes.byref(tiers), fake, need,
                              st) == H.ERR_INVALID_ARG
    for args in ((None, None, fake, fake), (None, fake, fake, None), (fake, fake, None, fake)):
        metric, logit, l2, stats = args
        assert lib.hardkv_compact_scored(d, ctypes.byref(cache), metric, logit, l2, stats, fake,
                                         ctypes.byref(tiers), fake, need, st) == H.ERR_INVALID_ARG
    assert lib.hardkv_compact_scored(d, ctypes.byref(cache), None, fake, None, fake, fake,
                                     ctypes.byref(tiers), fake, need - 1, st) == H.ERR_WORKSPACE
    # the lifecycle has neither sinks nor weighted merging
    for desc in (base_desc(sinks=8), weighted):
        state = H.StateC(fake, fake, tiers, fake)
        assert lib.hardkv_step_inplace(ctypes.byref(desc), fake, fake, fake, None,
                                       ctypes.byref(state), fake, fake, H.workspace_size(desc),
                                       st) == H.ERR_INVALID_ARG
    # sinks add dense tiles (64 + 500 rows: two 512-entry tiles instead of
    # one): at equal capacities the workspace grows with them
    assert H.workspace_size(base_desc(sinks=500, sparse_cap=936, chunk_cap=30)) > \
        H.workspace_size(base_desc())


def test_packed_tier_errors_before_launch():
    lib = H.load()
    fake = ctypes.c_void_p(0x1000)
    cache = H.Cache(fake, fake, None, fake)
    st = ctypes.c_void_p(0)
    packed = base_desc(packed_rows=500)
    need = H.workspace_size(packed)
    d = ctypes.byref(packed)
    full = H.TiersC(*([fake] * 9))
    no_offset = H.TiersC(*([fake] * 8))
    no_mode = H.TiersC(*([fake] * 7), None, fake)
    for t in (no_offset, no_mode):
        tb = ctypes.byref(t)
        assert lib.hardkv_step(d, fake, ctypes.byref(cache), None, tb, fake, fake, need, st) == \
            H.ERR_INVALID_ARG
        assert lib.hardkv_compact(d, ctypes.byref(cache), fake, tb, fake, need, st) == \
            H.ERR_INVALID_ARG
        assert lib.hardkv_decode_attn(d, fake, ctypes.byref(cache), tb, fake, fake, need, st) == \
            H.ERR_INVALID_ARG
        assert lib.hardkv_pack(d, fake, tb, st) == H.ERR_INVALID_ARG
    assert lib.hardkv_pack(d, None, ctypes.byref(full), st) == H.ERR_INVALID_ARG
    # hardkv_pack needs a packed descriptor
    assert lib.hardkv_pack(ctypes.byref(base_desc()), fake, ctypes.byref(full), st) == \
        H.ERR_INVALID_ARG
    # the lifecycle keeps per-head pools
    state = H.StateC(fake, fake, H.TiersC(*([fake] * 7)), fake)
    assert lib.hardkv_step_inplace(d, fake, fake, fake, None, ctypes.byref(state), fake, fake,
                                   need, st) == H.ERR_INVALID_ARG


def test_tier_block_manager_errors_before_launch():
    """Every call with a block-managed rewritten tier needs the manager's
    state and the per-head modes; init and alloc need a block-managed
    descriptor.  No call here passes validation."""
    lib = H.load()
    fake = ctypes.c_void_p(0x1000)
    cache = H.Cache(fake, fake, None, fake)
    st = ctypes.c_void_p(0)
    bm = base_desc(tier_block=16, tier_blocks=200)
    need = H.workspace_size(bm)
    d = ctypes.byref(bm)
    full = H.TiersC(*([fake] * 8), None, *([fake] * 4))
    partial = [H.TiersC(*([fake] * 7), None, None, *([fake] * 4)),     # no mode
               H.TiersC(*([fake] * 8), None, None, *([fake] * 3)),     # no table
               H.TiersC(*([fake] * 8), None, fake, None, fake, fake),  # no held
               H.TiersC(*([fake] * 8), None, fake, fake, None, fake),  # no free ids
               H.TiersC(*([fake] * 8), None, fake, fake, fake, None)]  # no top
    pol = H.policy()
    for t in partial:
        tb = ctypes.byref(t)
        assert lib.hardkv_step(d, fake, ctypes.byref(cache), None, tb, fake, fake, need, st) == \
            H.ERR_INVALID_ARG
        assert lib.hardkv_step_policy(d, ctypes.byref(pol), fake, ctypes.byref(cache), None, tb,
                                      fake, fake, need, st) == H.ERR_INVALID_ARG
        assert lib.hardkv_compact(d, ctypes.byref(cache), fake, tb, fake, need, st) == \
            H.ERR_INVALID_ARG
        assert lib.hardkv_decode_attn(d, fake, ctypes.byref(cache), tb, fake, fake, need, st) == \
            H.ERR_INVALID_ARG
        assert lib.hardkv_tier_alloc(d, fake, tb, st) == H.ERR_INVALID_ARG
    for t in partial[1:]:
        assert lib.hardkv_tier_init(d, ctypes.byref(t), st) == H.ERR_INVALID_ARG
    assert lib.hardkv_tier_alloc(d, None, ctypes.byref(full), st) == H.ERR_INVALID_ARG
    assert lib.hardkv_tier_init(d, None, st) == H.ERR_INVALID_ARG
    # both need a block-managed descriptor
    plain = ctypes.byref(base_desc())
    assert lib.hardkv_tier_init(plain, ctypes.byref(full), st) == H.ERR_INVALID_ARG
    assert lib.hardkv_tier_alloc(plain, fake, ctypes.byref(full), st) == H.ERR_INVALID_ARG
    assert lib.hardkv_tier_init(ctypes.byref(base_desc(tier_block=12, tier_blocks=9)),
                                ctypes.byref(full), st) == H.ERR_INVALID_ARG
    # the lifecycle keeps its own pool manager
    state = H.StateC(fake, fake, H.TiersC(*([fake] * 7)), fake)
    assert lib.hardkv_step_inplace(d, fake, fake, fake, None, ctypes.byref(state), fake, fake,
                                   need, st) == H.ERR_INVALID_ARG


def test_window_metric_needs_the_query_history():
    lib = H.load()
    fake = ctypes.c_void_p(0x1000)
    no_hist = H.Cache(fake, fake, None, fake, None)
    with_hist = H.Cache(fake, fake, None, fake, fake)
    tiers = H.TiersC(*([fake] * 7))
    st = ctypes.c_void_p(0)
    win = base_desc(obs_window=4, pool_radius=3)
    need = H.workspace_size(win)
    assert need > H.workspace_size(base_desc())   # float64 window queries + pre-pool metric
    d = ctypes.byref(win)
    assert lib.hardkv_score(d, fake, ctypes.byref(no_hist), fake, fake, fake, fake, need, st) == \
        H.ERR_INVALID_ARG
    assert lib.hardkv_step(d, fake, ctypes.byref(no_hist), fake, ctypes.byref(tiers), fake, fake,
                           need, st) == H.ERR_INVALID_ARG
    assert lib.hardkv_score(d, fake, ctypes.byref(with_hist), fake, fake, fake, fake, need - 1,
                            st) == H.ERR_WORKSPACE
    # the lifecycle has no window metric
    state = H.StateC(fake, fake, tiers, fake)
    assert lib.hardkv_step_inplace(d, fake, fake, fake, None, ctypes.byref(state), fake, fake,
                                   need, st) == H.ERR_INVALID_ARG


def test_lifecycle_has_no_block_selection():
    lib = H.load()
    fake = ctypes.c_void_p(0x1000)
    st = ctypes.c_void_p(0)
    d = base_desc(select_block=16)
    state = H.StateC(fake, fake, H.TiersC(*([fake] * 7)), fake)
    assert lib.hardkv_step_inplace(ctypes.byref(d), fake, fake, fake, None, ctypes.byref(state),
                                   fake, fake, H.workspace_size(d), st) == H.ERR_INVALID_ARG


def test_lifecycle_keeps_the_spread_rule():
    # the running chunk sums of the lifecycle are built under one rule
    lib = H.load()
    fake = ctypes.c_void_p(0x1000)
    st = ctypes.c_void_p(0)
    ent = base_desc(calibration=H.CALIB_ENTROPY)
    need = H.workspace_size(ent)
    assert need == H.workspace_size(base_desc())  # no extra workspace
    state = H.StateC(fake, fake, H.TiersC(*([fake] * 7)), fake)
    assert lib.hardkv_step_inplace(ctypes.byref(ent), fake, fake, fake, None, ctypes.byref(state),
                                   fake, fake, need, st) == H.ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(pool_block=48), dict(pool_block=8192), dict(pool_block=-16),
                                dict(pool_block=16, pool_blocks=0),
                                dict(pool_block=16, table=False), dict(pool_block=16, stack=False)])
def test_block_manager_arguments(kw):
    lib = H.load()
    fake = ctypes.c_void_p(0x1000)
    st = ctypes.c_void_p(0)
    d = base_desc()
    need = H.workspace_size(d)
    state = H.StateC(fake, fake, H.TiersC(*([fake] * 7)), fake,
                     None if kw.get("table") is False else fake,
                     None if kw.get("stack") is False else fake, fake,
                     kw.get("pool_block", 0), kw.get("pool_blocks", 64))
    assert lib.hardkv_step_inplace(ctypes.byref(d), fake, fake, fake, None, ctypes.byref(state),
                                   fake, fake, need, st) == H.ERR_INVALID_ARG
