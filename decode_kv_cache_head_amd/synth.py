"""Seeded synthetic inputs for the decode-step workloads.

This module only draws random tensors and lays them out (contiguous or
paged caches, block tables, context lengths).  It holds none of the method's
arithmetic, so both the HIP path and the CPU oracle may take their inputs
from it.

The pages evaluate on math-reasoning generations of Qwen3 models; those
datasets and weights are not available, so these tensors stand in for them
at the Qwen3 attention shapes (32 or 64 query heads, 8 KV heads, head_dim
128).  Values are N(0, 1) unless a workload plants structure.
"""
from __future__ import annotations

import math
import zlib
from dataclasses import dataclass, field, replace

import torch

DT_F32 = 0
DT_BF16 = 1
METRIC_QK = 0
METRIC_L2 = 1
METRIC_WINDOW = 2
METRIC_KEYDIFF = 3
METRIC_RKV = 4


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    T: tuple            # context length per sequence (current token included)
    dtype: int          # DT_F32 or DT_BF16 for q, K and V
    W: int              # dense window
    C: int              # condensed chunk size
    p: float            # top-p
    block_size: int = 0  # 0 = contiguous cache [B][Hkv][ctx_cap][d]
    metric: tuple = ()  # per KV head; empty = all QK
    planted: int = 0    # planted heavy keys per KV head (tiny workload)
    temp_range: tuple = ()  # per-KV-head query temperature range
    peaked_heads: tuple = ()  # heads with Zipf-planted keys
    peaked_m: int = 64
    peaked_zipf: float = 1.2
    peaked_top: float = 24.0
    seed: int = 20260627
    sinks: int = 0       # leading positions kept in the dense tier
    merge: int = 0       # 0 mean, 1 attention-weighted merging of evicted tokens
    obs_window: int = 1  # queries in the observation window (window-metric heads)
    pool_radius: int = 0  # max-pooling radius of the window metric
    calibration: int = 0  # temperature rule of non-logit heads: 0 spread, 1 entropy
    select_block: int = 0  # 0 token-level top-p; > 0 whole blocks of this many positions

    @property
    def G(self):
        return self.Hq // self.Hkv

    @property
    def metrics(self):
        return self.metric if self.metric else (METRIC_QK,) * self.Hkv


def _ragged(B, lo, hi, seed):
    g = torch.Generator().manual_seed(seed)
    return tuple(int(x) for x in torch.randint(lo, hi + 1, (B,), generator=g))


def workload(name: str, **over) -> Workload:
    """The named workloads (tiny fp32 check, Qwen3-8B-shaped single layer,
    batched paged 16k headline and its all-peaked variant, ragged paged
    batch, mixed-metric 64k)."""
    if name == "tiny":
        w = Workload("tiny", 1, 4, 2, 64, (512,), DT_F32, 64, 32, 0.9, planted=8)
    elif name == "qwen8b_b1_16k":
        w = Workload("qwen8b_b1_16k", 1, 32, 8, 128, (16384,), DT_BF16, 256, 64, 0.95,
                     temp_range=(0.5, 4.0))
    elif name == "qwen8b_b32_16k_paged":
        w = Workload("qwen8b_b32_16k_paged", 32, 32, 8, 128, (16384,) * 32, DT_BF16,
                     256, 64, 0.95, block_size=16)
    elif name == "qwen8b_b32_16k_paged_peaked":
        # the headline shape with every KV head peaked (Zipf-planted keys),
        # the concentrated attention for which a selection keeps few tokens
        w = Workload("qwen8b_b32_16k_paged_peaked", 32, 32, 8, 128, (16384,) * 32, DT_BF16,
                     256, 64, 0.95, block_size=16, peaked_heads=tuple(range(8)))
    elif name == "qwen8b_b32_ragged_paged":
        w = Workload("qwen8b_b32_ragged_paged", 32, 32, 8, 128,
                     _ragged(32, 8192, 32768, 20260627 + 3), DT_BF16, 256, 64, 0.95,
                     block_size=16)
    elif name == "qwen8b_b8_64k_mixed":
        w = Workload("qwen8b_b8_64k_mixed", 8, 32, 8, 128, (65536,) * 8, DT_BF16, 256, 64,
                     0.9, metric=(METRIC_QK,) * 4 + (METRIC_L2,) * 4, peaked_heads=(0, 4))
    else:
        raise KeyError(name)
    if "T" in over and isinstance(over["T"], int):
        over["T"] = (over["T"],) * over.get("B", w.B)
    if "B" in over and "T" not in over:
        over["T"] = tuple((list(w.T) * over["B"])[:over["B"]])
    return replace(w, **over)


def _seed(w: Workload, *tags) -> int:
    key = "/".join([w.name, str(w.seed)] + [str(t) for t in tags])
    return zlib.crc32(key.encode()) & 0x7FFFFFFF


def _gen(w, device, *tags):
    return torch.Generator(device=device).manual_seed(_seed(w, *tags))


def _randn(shape, w, device, *tags):
    return torch.randn(shape, generator=_gen(w, device, *tags), device=device,
                       dtype=torch.float32)


def _tdtype(w):
    return torch.float32 if w.dtype == DT_F32 else torch.bfloat16


@dataclass
class Case:
    """Device-resident (or CPU) inputs of one decode step."""
    w: Workload
    q: torch.Tensor            # [B][Hq][d]
    k: torch.Tensor            # contiguous [B][Hkv][ctx_cap][d] or pool [nblk][Hkv][bs][d]
    v: torch.Tensor
    ctx_len: torch.Tensor      # [B] int32
    block_table: torch.Tensor | None  # [B][max_blocks] int32
    metric: torch.Tensor | None  # [Hkv] int8, or None when every head is QK
    ctx_cap: int
    max_blocks: int
    extra: dict = field(default_factory=dict)
    q_hist: torch.Tensor | None = None  # [B][obs_window - 1][Hq][d] earlier queries


def make_case(w: Workload, device="cpu") -> Case:
    """Draw one decode step's q, K, V with the workload's structure."""
    B, Hq, Hkv, d, G = w.B, w.Hq, w.Hkv, w.d, w.G
    dt = _tdtype(w)
    q = _randn((B, Hq, d), w, device, "q")
    if w.temp_range:
        lo, hi = w.temp_range
        tau = torch.rand((Hkv,), generator=_gen(w, "cpu", "tau")) * (hi - lo) + lo
        q = q / tau.repeat_interleave(G).to(device)[None, :, None]
    q = q.to(dt)
    Tmax = max(w.T)
    bs = w.block_size
    if bs:
        nb = [-(-t // bs) for t in w.T]
        max_blocks = max(nb)
        ctx_cap = max_blocks * bs
        nblk = sum(nb)
        perm = torch.randperm(nblk, generator=_gen(w, "cpu", "perm")).to(torch.int32)
        table = torch.full((B, max_blocks), -1, dtype=torch.int32)
        o = 0
        for b in range(B):
            table[b, :nb[b]] = perm[o:o + nb[b]]
            o += nb[b]
        k = torch.empty((nblk, Hkv, bs, d), dtype=dt, device=device)
        v = torch.empty_like(k)
    else:
        ctx_cap = Tmax
        max_blocks = 0
        table = None
        k = torch.empty((B, Hkv, ctx_cap, d), dtype=dt, device=device)
        v = torch.empty_like(k)
    extra = {}
    for b in range(B):
        T = w.T[b]
        L = -(-T // bs) * bs if bs else ctx_cap
        kb = _randn((Hkv, L, d), w, device, "k", b)
        vb = _randn((Hkv, L, d), w, device, "v", b)
        qb = q[b].float()
        if w.planted:
            A = max(T - w.W, 0)
            for h in range(Hkv):
                g0 = h * G
                qh = qb[g0]
                heavy = 4.0 * qh / qh.norm()
                pos = torch.randperm(A, generator=_gen(w, "cpu", "plant", b, h))[:w.planted]
                kb[h, pos.to(device)] = heavy
                extra[("planted", b, h)] = sorted(int(x) for x in pos)
        for h in w.peaked_heads:
            A = max(T - w.W, 0)
            g0 = h * G
            qh = qb[g0]
            r = torch.arange(1, w.peaked_m + 1, dtype=torch.float32, device=device)
            L_r = w.peaked_top - w.peaked_zipf * torch.log(r)
            if w.metrics[h] == METRIC_L2:
                # a key-norm head ranks by |k|: the planted keys' norms stand
                # L_r standard deviations of a flat key's norm (1/sqrt(2) for
                # N(0, 1) entries) above the typical norm sqrt(d)
                norm = math.sqrt(d) + L_r / math.sqrt(2.0)
            else:
                # a logit head: the planted keys' logit with q_g0 is L_r
                norm = L_r * math.sqrt(d) / qh.norm()
            keys = norm[:, None] * (qh / qh.norm())[None, :]
            pos = torch.randperm(A, generator=_gen(w, "cpu", "peak", b, h))[:w.peaked_m]
            kb[h, pos.to(device)] = keys[:len(pos)]
            extra[("peaked", b, h)] = [int(x) for x in pos]
        kb = kb.to(dt)
        vb = vb.to(dt)
        if bs:
            ids = table[b, :nb[b]].long().to(device)
            k[ids] = kb.view(Hkv, nb[b], bs, d).permute(1, 0, 2, 3)
            v[ids] = vb.view(Hkv, nb[b], bs, d).permute(1, 0, 2, 3)
        else:
            k[b] = kb
            v[b] = vb
    ctx_len = torch.tensor(w.T, dtype=torch.int32, device=device)
    # no metric array when every head scores with the logit (NULL = all QK)
    metric = torch.tensor(w.metric, dtype=torch.int8, device=device) if w.metric else None
    if table is not None:
        table = table.to(device)
    q_hist = None
    if w.obs_window > 1:
        # earlier decode queries of the observation window, most recent first
        q_hist = _randn((B, w.obs_window - 1, Hq, d), w, device, "q_hist").to(dt)
    return Case(w, q, k, v, ctx_len, table, metric, ctx_cap, max_blocks, extra, q_hist)


def head_rows(case: Case, b: int, h: int, which: str = "k", upto: int | None = None):
    """Position-ordered rows [T_b][d] of KV head h of sequence b (a view or a
    gather through the block table; data layout only)."""
    src = case.k if which == "k" else case.v
    T = case.w.T[b] if upto is None else upto
    bs = case.w.block_size
    if not bs:
        return src[b, h, :T]
    nb = -(-T // bs)
    ids = case.block_table[b, :nb].long()
    return src[ids, h].reshape(nb * bs, -1)[:T]
