"""ctypes binding of libhardkv.so (the HIP library).

Argument marshalling only: every step of the decode path runs in the HIP
kernels behind the C ABI declared in include/hardkv.h.  Tensors are torch
tensors on the GPU; their data pointers and the current HIP stream are passed
through.  A missing library raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhardkv.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_CAPACITY, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4, -5
F32, BF16 = 0, 1
METRIC_QK, METRIC_L2, METRIC_WINDOW, METRIC_KEYDIFF, METRIC_RKV = 0, 1, 2, 3, 4
MODE_REWRITE, MODE_SPARSE = 0, 1
MERGE_MEAN, MERGE_WEIGHTED = 0, 1
CALIB_SPREAD, CALIB_ENTROPY = 0, 1
POLICY_REWRITE, POLICY_SPARSE, POLICY_MTI = 0, 1, 2
INT32_MAX = 2 ** 31 - 1

_lib = None


class HardKVError(RuntimeError):
    def __init__(self, code, fn):
        self.code = code
        msg = _lib.hardkv_strerror(code).decode() if _lib else str(code)
        super().__init__(f"{fn}: {msg} ({code})")


class Desc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("dense_window", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("ctx_cap", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
                ("sparse_cap", ctypes.c_int32), ("chunk_cap", ctypes.c_int32),
                ("top_p", ctypes.c_float), ("sinks", ctypes.c_int32), ("merge", ctypes.c_int32),
                ("packed_rows", ctypes.c_int32), ("obs_window", ctypes.c_int32),
                ("pool_radius", ctypes.c_int32), ("calibration", ctypes.c_int32),
                ("select_block", ctypes.c_int32), ("tier_block", ctypes.c_int32),
                ("tier_blocks", ctypes.c_int32)]


class Cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("ctx_len", ctypes.c_void_p),
                ("q_hist", ctypes.c_void_p)]


class TiersC(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("pos", ctypes.c_void_p),
                ("count", ctypes.c_void_p), ("ksum", ctypes.c_void_p),
                ("vsum", ctypes.c_void_p), ("ccount", ctypes.c_void_p),
                ("mode", ctypes.c_void_p), ("offset", ctypes.c_void_p),
                ("table", ctypes.c_void_p), ("held", ctypes.c_void_p),
                ("free_ids", ctypes.c_void_p), ("free_top", ctypes.c_void_p)]


class Policy(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("horizon", ctypes.c_int32),
                ("l_lower", ctypes.c_int32), ("l_upper", ctypes.c_int32)]


class StateC(ctypes.Structure):
    _fields_ = [("ring_k", ctypes.c_void_p), ("ring_v", ctypes.c_void_p),
                ("tiers", TiersC), ("seq_len", ctypes.c_void_p),
                ("pool_table", ctypes.c_void_p), ("free_ids", ctypes.c_void_p),
                ("free_top", ctypes.c_void_p), ("pool_block", ctypes.c_int32),
                ("pool_blocks", ctypes.c_int32)]


_P = ctypes.c_void_p
OBSERVER = ctypes.CFUNCTYPE(None, ctypes.c_char_p, ctypes.c_void_p, ctypes.c_void_p)
_SIGS = {
    "hardkv_set_launch_observer": ([OBSERVER, _P], None),
    "hardkv_version": ([], ctypes.c_int),
    "hardkv_strerror": ([ctypes.c_int], ctypes.c_char_p),
    "hardkv_validate": ([ctypes.POINTER(Desc)], ctypes.c_int),
    "hardkv_workspace_size": ([ctypes.POINTER(Desc)], ctypes.c_size_t),
    "hardkv_score": ([ctypes.POINTER(Desc), _P, ctypes.POINTER(Cache), _P, _P, _P, _P,
                      ctypes.c_size_t, _P], ctypes.c_int),
    "hardkv_calibrate": ([ctypes.POINTER(Desc), _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
                         ctypes.c_int),
    "hardkv_topp_select": ([ctypes.POINTER(Desc), _P, _P, _P, _P, _P, _P, _P, _P,
                            ctypes.c_size_t, _P], ctypes.c_int),
    "hardkv_compact": ([ctypes.POINTER(Desc), ctypes.POINTER(Cache), _P, ctypes.POINTER(TiersC),
                        _P, ctypes.c_size_t, _P], ctypes.c_int),
    "hardkv_compact_scored": ([ctypes.POINTER(Desc), ctypes.POINTER(Cache), _P, _P, _P, _P, _P,
                               ctypes.POINTER(TiersC), _P, ctypes.c_size_t, _P], ctypes.c_int),
    "hardkv_decode_attn": ([ctypes.POINTER(Desc), _P, ctypes.POINTER(Cache),
                            ctypes.POINTER(TiersC), _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "hardkv_step": ([ctypes.POINTER(Desc), _P, ctypes.POINTER(Cache), _P,
                     ctypes.POINTER(TiersC), _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "hardkv_step_noalloc": ([ctypes.POINTER(Desc), _P, ctypes.POINTER(Cache), _P,
                             ctypes.POINTER(TiersC), _P, _P], ctypes.c_int),
    "hardkv_plan": ([ctypes.POINTER(Desc), ctypes.POINTER(Policy), _P, _P, _P, _P],
                    ctypes.c_int),
    "hardkv_pack": ([ctypes.POINTER(Desc), _P, ctypes.POINTER(TiersC), _P], ctypes.c_int),
    "hardkv_tier_init": ([ctypes.POINTER(Desc), ctypes.POINTER(TiersC), _P], ctypes.c_int),
    "hardkv_tier_alloc": ([ctypes.POINTER(Desc), _P, ctypes.POINTER(TiersC), _P], ctypes.c_int),
    "hardkv_step_policy": ([ctypes.POINTER(Desc), ctypes.POINTER(Policy), _P,
                            ctypes.POINTER(Cache), _P, ctypes.POINTER(TiersC), _P, _P,
                            ctypes.c_size_t, _P], ctypes.c_int),
    "hardkv_step_inplace": ([ctypes.POINTER(Desc), _P, _P, _P, _P, ctypes.POINTER(StateC), _P,
                             _P, ctypes.c_size_t, _P], ctypes.c_int),
}
EXPORTS = tuple(_SIGS)


def load(path: str = LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with python -m decode_kv_cache_head_amd.build")
    lib = ctypes.CDLL(path)
    for name, (args, res) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(rc, fn):
    if rc != OK:
        raise HardKVError(rc, fn)


def make_desc(B, Hq, Hkv, d, dtype, W, C, top_p, ctx_cap, block_size=0, max_blocks=0,
              sparse_cap=None, chunk_cap=None, sinks=0, merge=MERGE_MEAN,
              packed_rows=0, obs_window=1, pool_radius=0, calibration=CALIB_SPREAD,
              select_block=0, tier_block=0, tier_blocks=0) -> Desc:
    A = max(ctx_cap - W - sinks, 0)
    if sparse_cap is None:
        sparse_cap = A
    if chunk_cap is None:
        chunk_cap = -(-A // C) if C > 0 else 0
    return Desc(B, Hq, Hkv, d, dtype, W, C, block_size, ctx_cap, max_blocks, sparse_cap,
                chunk_cap, float(top_p), sinks, merge, packed_rows, obs_window, pool_radius,
                calibration, select_block, tier_block, tier_blocks)


def validate(desc: Desc) -> int:
    return load().hardkv_validate(ctypes.byref(desc))


def workspace_size(desc: Desc) -> int:
    return load().hardkv_workspace_size(ctypes.byref(desc))


def alloc_workspace(desc: Desc, device="cuda"):
    n = workspace_size(desc)
    if n == 0:
        _check(validate(desc), "workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)


@dataclass
class Tiers:
    k: torch.Tensor
    v: torch.Tensor
    pos: torch.Tensor
    count: torch.Tensor
    ksum: torch.Tensor
    vsum: torch.Tensor
    ccount: torch.Tensor
    mode: torch.Tensor | None = None   # [B][Hkv] uint8, None = every head rewritten
    offset: torch.Tensor | None = None  # [B][Hkv] int32, packed tier only
    # block manager of the rewritten tier (tier_block > 0): k, v = [blocks][tb][d]
    table: torch.Tensor | None = None     # [B][Hkv][ceil(sparse_cap / tb)] int32
    held: torch.Tensor | None = None      # [B][Hkv] int32
    free_ids: torch.Tensor | None = None  # [blocks] int32
    free_top: torch.Tensor | None = None  # [1] int32

    def c(self) -> TiersC:
        return TiersC(*(ctypes.c_void_p(t.data_ptr()) for t in
                        (self.k, self.v, self.pos, self.count, self.ksum, self.vsum, self.ccount)),
                      _p(self.mode), _p(self.offset), _p(self.table), _p(self.held),
                      _p(self.free_ids), _p(self.free_top))

    def slots(self, b, h, which="k"):
        """Head (b, h)'s rewritten slots 0..count-1 (any layout)."""
        src = self.k if which == "k" else self.v
        n = int(self.count[b, h])
        if self.table is not None:
            tb = src.shape[1]
            ids = self.table[b, h, :-(-n // tb)].long()
            return src[ids].reshape(-1, src.shape[-1])[:n]
        if self.offset is None:
            return src[b, h, :n]
        o = int(self.offset[b, h])
        return src[o:o + n]


def alloc_tiers(desc: Desc, device="cuda", zero=False, mode=False, blocks=None) -> Tiers:
    """Tiers for `desc`; a packed desc (packed_rows > 0) gets one [packed_rows][d]
    region for K and for V plus the offsets and modes it needs; a block-managed
    desc (tier_block > 0) a pool of [tier_blocks][tier_block][d] and the
    manager's state (set up with tier_init before the first selection), or
    the given `blocks` = (k, v, free_ids, free_top) of a pool shared with
    other tiers."""
    B, Hkv, d = desc.batch, desc.num_kv_heads, desc.head_dim
    dt = torch.float32 if desc.dtype == F32 else torch.bfloat16
    mk = torch.zeros if zero else torch.empty
    cap, ccap = desc.sparse_cap, desc.chunk_cap
    packed = desc.packed_rows > 0
    if desc.tier_block > 0:
        tb = desc.tier_block
        if blocks is None:
            blocks = (mk((desc.tier_blocks, tb, d), dtype=dt, device=device),
                      mk((desc.tier_blocks, tb, d), dtype=dt, device=device),
                      torch.empty(desc.tier_blocks, dtype=torch.int32, device=device),
                      torch.empty(1, dtype=torch.int32, device=device))
        return Tiers(blocks[0], blocks[1],
                     mk((B, Hkv, cap), dtype=torch.int32, device=device),
                     mk((B, Hkv), dtype=torch.int32, device=device),
                     mk((B, Hkv, ccap, d), dtype=torch.float32, device=device),
                     mk((B, Hkv, ccap, d), dtype=torch.float32, device=device),
                     mk((B, Hkv, ccap), dtype=torch.int32, device=device),
                     torch.zeros((B, Hkv), dtype=torch.uint8, device=device), None,
                     torch.empty((B, Hkv, -(-cap // tb)), dtype=torch.int32, device=device),
                     torch.empty((B, Hkv), dtype=torch.int32, device=device),
                     blocks[2], blocks[3])
    rows = (desc.packed_rows, d) if packed else (B, Hkv, cap, d)
    return Tiers(mk(rows, dtype=dt, device=device),
                 mk(rows, dtype=dt, device=device),
                 mk((B, Hkv, cap), dtype=torch.int32, device=device),
                 mk((B, Hkv), dtype=torch.int32, device=device),
                 mk((B, Hkv, ccap, d), dtype=torch.float32, device=device),
                 mk((B, Hkv, ccap, d), dtype=torch.float32, device=device),
                 mk((B, Hkv, ccap), dtype=torch.int32, device=device),
                 torch.zeros((B, Hkv), dtype=torch.uint8, device=device)
                 if (mode or packed) else None,
                 torch.zeros((B, Hkv), dtype=torch.int32, device=device) if packed else None)


def policy(kind=POLICY_MTI, horizon=1, l_lower=0, l_upper=INT32_MAX) -> Policy:
    return Policy(kind, horizon, l_lower, l_upper)


def cache_struct(k, v, ctx_len, block_table=None, q_hist=None) -> Cache:
    return Cache(_p(k), _p(v), _p(block_table), _p(ctx_len), _p(q_hist))


def score(desc, q, cache: Cache, metric, logit, l2, ws, stream=None):
    rc = load().hardkv_score(ctypes.byref(desc), _p(q), ctypes.byref(cache), _p(metric),
                             _p(logit), _p(l2), _p(ws), ws.numel(), _stream(stream))
    _check(rc, "hardkv_score")


def calibrate(desc, ctx_len, metric, logit, l2, stats, ws, stream=None):
    rc = load().hardkv_calibrate(ctypes.byref(desc), _p(ctx_len), _p(metric), _p(logit), _p(l2),
                                 _p(stats), _p(ws), ws.numel(), _stream(stream))
    _check(rc, "hardkv_calibrate")


def topp_select(desc, ctx_len, metric, logit, l2, stats, mask, count, ws, stream=None):
    rc = load().hardkv_topp_select(ctypes.byref(desc), _p(ctx_len), _p(metric), _p(logit),
                                   _p(l2), _p(stats), _p(mask), _p(count), _p(ws), ws.numel(),
                                   _stream(stream))
    _check(rc, "hardkv_topp_select")


def compact(desc, cache: Cache, mask, tiers: Tiers, ws, stream=None):
    tc = tiers.c()
    rc = load().hardkv_compact(ctypes.byref(desc), ctypes.byref(cache), _p(mask), ctypes.byref(tc),
                               _p(ws), ws.numel(), _stream(stream))
    _check(rc, "hardkv_compact")


def compact_scored(desc, cache: Cache, metric, logit, l2, stats, mask, tiers: Tiers, ws,
                   stream=None):
    tc = tiers.c()
    rc = load().hardkv_compact_scored(ctypes.byref(desc), ctypes.byref(cache), _p(metric),
                                      _p(logit), _p(l2), _p(stats), _p(mask), ctypes.byref(tc),
                                      _p(ws), ws.numel(), _stream(stream))
    _check(rc, "hardkv_compact_scored")


def decode_attn(desc, q, cache: Cache, tiers: Tiers, out, ws, stream=None):
    tc = tiers.c()
    rc = load().hardkv_decode_attn(ctypes.byref(desc), _p(q), ctypes.byref(cache),
                                   ctypes.byref(tc), _p(out), _p(ws), ws.numel(), _stream(stream))
    _check(rc, "hardkv_decode_attn")


def step(desc, q, cache: Cache, metric, tiers: Tiers, out, ws, stream=None):
    tc = tiers.c()
    rc = load().hardkv_step(ctypes.byref(desc), _p(q), ctypes.byref(cache), _p(metric),
                            ctypes.byref(tc), _p(out), _p(ws), ws.numel(), _stream(stream))
    _check(rc, "hardkv_step")


SCRATCH_BYTES = 64 << 20  # HARDKV_SCRATCH_BYTES


def step_noalloc(desc, q, cache: Cache, metric, tiers: Tiers, out, stream=None):
    """hardkv_step with the library-held workspace of the current device."""
    tc = tiers.c()
    rc = load().hardkv_step_noalloc(ctypes.byref(desc), _p(q), ctypes.byref(cache), _p(metric),
                                    ctypes.byref(tc), _p(out), _stream(stream))
    _check(rc, "hardkv_step_noalloc")


def plan(desc, pol: Policy, ctx_len, count, mode, stream=None):
    rc = load().hardkv_plan(ctypes.byref(desc), ctypes.byref(pol), _p(ctx_len), _p(count),
                            _p(mode), _stream(stream))
    _check(rc, "hardkv_plan")


def pack(desc, count, tiers: Tiers, stream=None):
    tc = tiers.c()
    rc = load().hardkv_pack(ctypes.byref(desc), _p(count), ctypes.byref(tc), _stream(stream))
    _check(rc, "hardkv_pack")


def tier_init(desc, tiers: Tiers, stream=None):
    tc = tiers.c()
    rc = load().hardkv_tier_init(ctypes.byref(desc), ctypes.byref(tc), _stream(stream))
    _check(rc, "hardkv_tier_init")


def tier_alloc(desc, count, tiers: Tiers, stream=None):
    tc = tiers.c()
    rc = load().hardkv_tier_alloc(ctypes.byref(desc), _p(count), ctypes.byref(tc),
                                  _stream(stream))
    _check(rc, "hardkv_tier_alloc")


def step_policy(desc, pol: Policy, q, cache: Cache, metric, tiers: Tiers, out, ws, stream=None):
    tc = tiers.c()
    rc = load().hardkv_step_policy(ctypes.byref(desc), ctypes.byref(pol), _p(q),
                                   ctypes.byref(cache), _p(metric), ctypes.byref(tc), _p(out),
                                   _p(ws), ws.numel(), _stream(stream))
    _check(rc, "hardkv_step_policy")


@dataclass
class State:
    ring_k: torch.Tensor
    ring_v: torch.Tensor
    tiers: Tiers
    seq_len: torch.Tensor
    # head-wise block manager of the pool (None: per-head regions)
    pool_table: torch.Tensor | None = None  # [B][Hkv][ceil(sparse_cap / pool_block)] int32
    free_ids: torch.Tensor | None = None    # [pool_blocks] int32 stack
    free_top: torch.Tensor | None = None    # [1] int32
    pool_block: int = 0

    def c(self) -> StateC:
        nblk = self.free_ids.numel() if self.free_ids is not None else 0
        return StateC(_p(self.ring_k), _p(self.ring_v), self.tiers.c(), _p(self.seq_len),
                      _p(self.pool_table), _p(self.free_ids), _p(self.free_top),
                      self.pool_block, nblk)

    def pool_rows(self, b, h, which="k"):
        """Head (b, h)'s pool rows 0..count-1 in order (either layout)."""
        src = self.tiers.k if which == "k" else self.tiers.v
        n = int(self.tiers.count[b, h])
        if self.pool_block == 0:
            return src[b, h, :n]
        nb = -(-n // self.pool_block)
        ids = self.pool_table[b, h, :nb].long()
        return src[ids].reshape(-1, src.shape[-1])[:n]

    def blocks_held(self) -> int:
        return int((self.pool_table >= 0).sum()) if self.pool_table is not None else 0


def paged_state(desc: Desc, K_aged, V_aged, ring_k, ring_v, seq_len, pool_block: int,
                pool_blocks: int) -> State:
    """Lifecycle state with the pool under the block manager, holding the
    aged rows K_aged / V_aged ([B][Hkv][A][d], position order 0..A-1): head
    (b, h) gets blocks (b * Hkv + h) * nb .. + nb - 1, nb = ceil(A / pool_block);
    the other blocks go on the free stack, lowest id on top."""
    B, Hkv, A, d = K_aged.shape
    dev = K_aged.device
    bs = pool_block
    nb = -(-A // bs)
    maxb = -(-desc.sparse_cap // bs)
    used = B * Hkv * nb
    if used > pool_blocks or nb > maxb:
        raise ValueError("the prefill does not fit the block pool")
    tiers = alloc_tiers(desc, dev, zero=True)
    tiers.k = torch.zeros((pool_blocks, bs, d), dtype=K_aged.dtype, device=dev)
    tiers.v = torch.zeros_like(tiers.k)
    pad = nb * bs - A
    kk = torch.nn.functional.pad(K_aged, (0, 0, 0, pad)) if pad else K_aged
    vv = torch.nn.functional.pad(V_aged, (0, 0, 0, pad)) if pad else V_aged
    tiers.k[:used] = kk.reshape(used, bs, d)
    tiers.v[:used] = vv.reshape(used, bs, d)
    tiers.pos[:, :, :A] = torch.arange(A, dtype=torch.int32, device=dev)
    tiers.count.fill_(A)
    table = torch.full((B, Hkv, maxb), -1, dtype=torch.int32, device=dev)
    table[:, :, :nb] = torch.arange(used, dtype=torch.int32, device=dev).reshape(B, Hkv, nb)
    free = torch.arange(pool_blocks - 1, used - 1, -1, dtype=torch.int32, device=dev)
    free_ids = torch.full((pool_blocks,), -1, dtype=torch.int32, device=dev)
    free_ids[:free.numel()] = free
    top = torch.tensor([free.numel()], dtype=torch.int32, device=dev)
    return State(ring_k, ring_v, tiers, seq_len, table, free_ids, top, bs)


def step_inplace(desc, q, k_new, v_new, metric, state: State, out, ws, stream=None):
    sc = state.c()
    rc = load().hardkv_step_inplace(ctypes.byref(desc), _p(q), _p(k_new), _p(v_new), _p(metric),
                                    ctypes.byref(sc), _p(out), _p(ws), ws.numel(),
                                    _stream(stream))
    _check(rc, "hardkv_step_inplace")


class KernelTimer:
    """Records a CUDA event on the launch stream before every kernel the
    library enqueues (through the launch observer), so the duration of each
    kernel is the gap between consecutive events.  Use as a context manager;
    call mark() after the last library call to close the last kernel."""

    def __init__(self):
        self.events = []   # (kernel name or None, event)
        self._cb = OBSERVER(self._on_launch)

    def _on_launch(self, name, stream, user):
        ev = torch.cuda.Event(enable_timing=True)
        ev.record(torch.cuda.ExternalStream(stream) if stream else torch.cuda.default_stream())
        self.events.append((name.decode(), ev))

    def mark(self, stream=None):
        ev = torch.cuda.Event(enable_timing=True)
        ev.record(stream or torch.cuda.current_stream())
        self.events.append((None, ev))

    def __enter__(self):
        load().hardkv_set_launch_observer(self._cb, None)
        return self

    def __exit__(self, *exc):
        load().hardkv_set_launch_observer(OBSERVER(), None)
        return False

    def durations(self):
        """[(kernel, ms)] for every launch followed by an event."""
        out = []
        for (name, e0), (_, e1) in zip(self.events, self.events[1:]):
            if name is not None:
                out.append((name, e0.elapsed_time(e1)))
        return out


def scale(d: int) -> float:
    return 1.0 / math.sqrt(d)
