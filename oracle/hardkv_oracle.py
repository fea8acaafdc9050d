"""Plain CPU oracle for the HARD-KV decode step (test infrastructure only).

This module is test infrastructure.  Only the test-suite, the package's
``smoke()`` self-check and the ``cpu_baseline`` leg of the benchmark may
import it.  The product path (the HIP library and its Python binding) never
calls it, and it shares no code with that path.

What it computes follows "HARD-KV: Head-Adaptive Regularization for
Decoding-time KV Compression" (gist.science technical summary, section 2,
"Methodology"; arXiv abstract on the mlsanity.com page).  The pages give no
formulas, so the readings taken where they are silent are written next to
each function.  Every step is the plain definition: float64 arithmetic from
the exact input values, a full sort, a cumulative sum, direct gathers and a
direct softmax.  No blocking, fusion or reordering.

Precision of decisions.  The token ranking is an integer decision taken from
floating point, so it is taken in the precision the GPU kernels keep their
ranking keys in: the score of every candidate (and the calibrated value) is
rounded once to float32, and the probability masses built from those float32
keys are float64.  Attention runs entirely in float64.

Parity pins (tests/test_oracle_pins.py): closed forms for the score
(Hadamard keys) and the key norm (integer triples), a hand-derived
calibration example, brute force over all subsets for the top-p set, uniform
and two-level closed forms, reductions to full softmax attention (p = 1,
chunk size 1, chunk-constant keys and values, window covering the context),
and the lifecycle invariants of the Cascade Cache.  The rule chosen for
calibrating a non-logit metric (moment matching, see ``calibrate_head``) is a
reading of the pages; its implementation is pinned by a hand-worked example
and invariants, the rule itself is not fixed by the pages.

The rewrite-versus-sparse-loading policy (``mti_head``, ``plan_head``) and
the reuse of a selection over later steps (``reuse_head``) are readings of
section 2.C, "Techniques" and "Trade-off Management", which name the
Memory-Time Integral and the thresholds L_lower / L_upper without a formula
(tests/test_oracle_policy.py: a worked example, a break-even closed form
derived from the integral, degenerate cases, threshold precedence, and
reductions of reuse attention to full softmax attention).  The integral's
cost model itself is this reading, not the pages'.

Attention-sink tokens in the dense tier and attention-weighted merging in
the condensed tier (``candidate_range``, ``merge_weights``, ``condense``)
read section 2.A, Tier 1 and Tier 3 (tests/test_oracle_merge.py: a
hand-worked weighted chunk, scale invariance and the weight floor, the tier
partition and chunk alignment with sinks, and reductions to full softmax
attention).

The observation-window metric (``window_score_head``; section 2.B) is pinned
in tests/test_oracle_window.py by a Hadamard closed form over several window
queries, scipy's maximum filter for the pooling, the one-query reduction to
the raw logits and the uniform closed form of a pooling radius that covers
the candidates.

The entropy-matched calibration rule (``entropy_temperature``; sections 2.A
and 2.B: a temperature, the raw attention distribution, budgets from
attention entropy) is pinned in tests/test_oracle_entropy.py by the
proportional-logit closed form, an independent root of the same equation
(scipy's brentq), exact power-of-two rescaling and the bisection's limits.

The R-KV redundancy metric (``redundancy_head``; section 2.B, "Mechanism":
strategies such as R-KV) is pinned in tests/test_oracle_redundancy.py by a
brute-force mean over all pairs of scipy's cosine distance, closed forms
(identical directions, an orthonormal set, two antipodal groups), exact
invariance under positive power-of-two scaling of single keys and under
permutation, the zero-key and single-candidate conventions, and reductions
of the whole step to full softmax attention.

The key-dissimilarity metric (``keydiff_head``; section 2.B: similarity
scores) is pinned in tests/test_oracle_keydiff.py by scipy's cosine distance,
closed forms (antipodal key groups, an orthonormal key set), exact
power-of-two scale invariance, the zero-vector convention and reductions of
the whole step to full softmax attention.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

METRIC_QK = 0      # max-over-GQA-group q.k logit
METRIC_L2 = 1      # key L2 norm
METRIC_WINDOW = 2  # observation-window, position-pooled max logit
METRIC_KEYDIFF = 3  # key dissimilarity: minus the cosine to the candidates' key sum
METRIC_RKV = 4      # R-KV redundancy: minus the mean cosine to the other candidates
AUX_METRICS = (METRIC_L2, METRIC_WINDOW, METRIC_KEYDIFF, METRIC_RKV)  # calibrated by a temperature

# Calibration rule for heads whose metric is not the raw logit
CALIB_SPREAD = 0   # temperature that matches the raw-logit spread (moments)
CALIB_ENTROPY = 1  # temperature that matches the raw-attention entropy
ENTROPY_STEPS = 32      # bisection halvings of the inverse-temperature bracket
ENTROPY_SPAN = 1024.0   # bracket [0, ENTROPY_SPAN / (max s - min s)]


def _f64(x) -> np.ndarray:
    """Exact widening of float32 / bfloat16-valued inputs to float64."""
    return np.asarray(x, dtype=np.float64)


def _check_finite(*arrays):
    # Inputs must be finite: NaN or Inf in q, K or V has no defined ranking.
    for a in arrays:
        if a is not None and not np.all(np.isfinite(a)):
            raise ValueError("oracle inputs must be finite")


# ---------------------------------------------------------------------------
# Tiers of the Cascade Cache (technical summary, section 2.A: Tier 1 dense,
# Tier 2 sparse, Tier 3 condensed).
# ---------------------------------------------------------------------------
def aged_count(T: int, W: int) -> int:
    """Number of tokens that have left the dense window.

    Tier 1 buffers the most recent tokens; a token that ages out of that
    window becomes a candidate for Tier 2 (section 2.A).  Reading: the dense
    window is the last W tokens, the current token included, so the aged
    candidates are positions [0, T - W).
    """
    if T < 1:
        raise ValueError("context length must be >= 1")
    if W < 0:
        raise ValueError("dense window must be >= 0")
    return max(T - W, 0)


# ---------------------------------------------------------------------------
# Importance scores (section 2.B, "Goal": max-pooled logits are one of the
# importance metrics the calibration normalises).
# ---------------------------------------------------------------------------
def score_head(q_group, K):
    """Importance scores of the candidate keys of one KV head.

    q_group: [G, d] query rows of the heads sharing this KV head.
    K:       [n, d] candidate key rows.
    Returns (ell, s) as float32 arrays of length n:
      ell_t = max_g (q_g . k_t) / sqrt(d)   -- the "max-pooled logits"
              (section 2.B); pooling is read as the max over the GQA group,
              with no pooling across positions,
      s_t   = ||k_t||_2                      -- the key-norm metric.
    Both are computed in float64 from the exact inputs and rounded once to
    float32, the precision in which the ranking decision is taken.
    """
    q = _f64(q_group)
    k = _f64(K)
    _check_finite(q, k)
    d = q.shape[1]
    if k.shape[0] == 0:
        return np.zeros(0, np.float32), np.zeros(0, np.float32)
    dots = k @ q.T                                  # [n, G], exact for bf16 data
    ell = dots.max(axis=1) * (1.0 / math.sqrt(d))
    s = np.sqrt(np.einsum("nd,nd->n", k, k))
    return ell.astype(np.float32), s.astype(np.float32)


def window_score_head(q_window, K, radius: int):
    """Observation-window metric with positional pooling (section 2.B: the
    calibration maps metrics of selection strategies such as SnapKV onto one
    probability space; "Goal": max-pooled logits).

    Reading: SnapKV scores a token by the attention the last few queries (an
    observation window) pay it, pooled over neighbouring positions so that
    the neighbours of an important token are kept with it.  In logit form:
      x_t  = max over the window's queries and the GQA group of q . k_t / sqrt(d)
             (float64 dots, rounded once to float32),
      x'_t = max of x_u over positions u in [t - r, t + r] inside the candidates.
    q_window: [w, G, d], row 0 the current query.  Returns x' float32 [n].
    """
    q = _f64(q_window)
    k = _f64(K)
    _check_finite(q, k)
    w, G, d = q.shape
    n = k.shape[0]
    if n == 0:
        return np.zeros(0, np.float32)
    dots = k @ q.reshape(w * G, d).T                # [n, w G]
    x = (dots.max(axis=1) * (1.0 / math.sqrt(d))).astype(np.float32)
    pooled = np.empty(n, np.float32)
    for t in range(n):
        pooled[t] = x[max(0, t - radius):min(n, t + radius + 1)].max()
    return pooled


# ---------------------------------------------------------------------------
# Logits Calibration (section 2.B "Mechanism"; section 3, second
# contribution).
# ---------------------------------------------------------------------------
@dataclass
class Calibration:
    shift: float      # c = fl32((x - shift) * scale)
    scale: float
    c: np.ndarray     # calibrated value per candidate, float32
    m: float          # max of c
    w: np.ndarray     # exp(c - m), float64
    Z: float          # sum of w


def softmax_entropy(x) -> float:
    """Entropy in nats of softmax(x) over the entries of x (float64):
    ln Z - sum(w * d) / Z with d = x - max x, w = exp(d), Z = sum w."""
    x64 = _f64(x)
    d = x64 - x64.max()
    w = np.exp(d)
    Z = math.fsum(w)
    return math.log(Z) - math.fsum(w * d) / Z


def entropy_temperature(ell, s) -> float:
    """Inverse temperature beta >= 0 for which softmax(beta * s) has the
    entropy of softmax(ell), the head's raw attention over the candidates.

    The entropy of softmax(beta * s) falls monotonically from ln n at
    beta = 0 towards ln(number of maxima of s).  The root is bracketed in
    [0, ENTROPY_SPAN / (max s - min s)] (at the upper end every
    non-maximal token weighs below e^-1024 of the top) and the bracket is
    halved ENTROPY_STEPS times: the midpoint's entropy above the target
    moves the lower end up, otherwise the upper end down; the result is the
    final midpoint.  A target beyond the bracket ends at its nearer end.
    Requires max s > min s."""
    s64 = _f64(s)
    target = softmax_entropy(ell)
    smax = float(s64.max())
    R = smax - float(s64.min())
    d = s64 - smax
    lo, hi = 0.0, ENTROPY_SPAN / R
    for _ in range(ENTROPY_STEPS):
        mid = 0.5 * (lo + hi)
        w = np.exp(mid * d)
        Z = math.fsum(w)
        H = math.log(Z) - mid * math.fsum(w * d) / Z
        if H > target:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def calibrate_head(ell, s, metric: int, calib: int = CALIB_SPREAD) -> Calibration:
    """Map one head's importance scores into a softmax probability space.

    The pages state that calibration maps a selection metric onto a
    normalised softmax by adjusting the temperature, keeps the metric's
    order, and maps onto the raw attention distribution.  Reading:
      * QK heads: temperature 1, c = ell.  The calibrated distribution is the
        raw attention distribution over the candidates.
      * key-norm and observation-window heads (s = the metric): a temperature
        chosen so the metric's spread equals the head's raw-logit spread:
        c = (s - mu_s) * sigma_ell / sigma_s, population moments over the
        candidates (the shift does not change the softmax).  A zero spread
        gives c = 0.
      * with calib = CALIB_ENTROPY instead, the temperature that gives the
        metric's softmax the entropy of the raw attention distribution (the
        pages tie Tier-2 budgets to attention entropy, section 2.A):
        c = (s - max s) * beta with beta from ``entropy_temperature``.  A
        metric with no spread gives c = 0.
    The softmax domain is the candidate set only (dense-tier tokens are kept
    by rule).  Weights w = exp(c - max c), Z = sum w, float64.
    """
    ell = np.asarray(ell, dtype=np.float32)
    s = np.asarray(s, dtype=np.float32)
    n = ell.shape[0]
    if metric == METRIC_QK:
        shift, scale = 0.0, 1.0
        c = ell.copy()
    elif metric in AUX_METRICS and calib == CALIB_ENTROPY:
        s64 = _f64(s)
        if n == 0 or s64.max() == s64.min():
            shift, scale = 0.0, 0.0
            c = np.zeros(n, np.float32)
        else:
            shift, scale = float(s64.max()), entropy_temperature(ell, s)
            c = ((s64 - shift) * scale).astype(np.float32)
    elif metric in AUX_METRICS:
        if calib != CALIB_SPREAD:
            raise ValueError(f"unknown calibration rule {calib}")
        if n == 0:
            shift, scale = 0.0, 0.0
            c = np.zeros(0, np.float32)
        else:
            s64 = _f64(s)
            l64 = _f64(ell)
            mu_s = float(np.mean(s64))
            sd_s = float(np.sqrt(np.mean((s64 - mu_s) ** 2)))
            mu_l = float(np.mean(l64))
            sd_l = float(np.sqrt(np.mean((l64 - mu_l) ** 2)))
            if sd_s == 0.0 or sd_l == 0.0:
                shift, scale = 0.0, 0.0
                c = np.zeros(n, np.float32)
            else:
                shift, scale = mu_s, sd_l / sd_s
                c = ((s64 - shift) * scale).astype(np.float32)
    else:
        raise ValueError(f"unknown metric {metric}")
    if n == 0:
        return Calibration(shift, scale, c, 0.0, np.zeros(0), 0.0)
    c64 = _f64(c)
    m = float(c64.max())
    w = np.exp(c64 - m)
    Z = math.fsum(w)
    return Calibration(shift, scale, c, m, w, Z)


# ---------------------------------------------------------------------------
# Calibrated Top-p selection (section 2.A, Tier 2; section 2.B "Outcome").
# ---------------------------------------------------------------------------
@dataclass
class Selection:
    order: np.ndarray      # candidate indices in rank order (c desc, position asc)
    k: int                 # size of the selected set
    selected: np.ndarray   # selected candidate indices, ascending
    prefix_excl: np.ndarray  # exclusive prefix mass / Z in rank order
    w_sorted: np.ndarray   # weights in rank order


def topp_head(c, w, Z, p, positions=None) -> Selection:
    """Smallest candidate set whose calibrated mass reaches p.

    Reading: Top-p here is a deterministic nucleus, not random sampling.
    Candidates are ranked by calibrated value, highest first, equal values by
    lower original position first.  k is the smallest k >= 1 with
    sum_{i<k} w_(i) >= p * Z, p taken as float32 and widened exactly.
    p >= 1 keeps every candidate; an empty candidate set selects nothing.
    """
    c = np.asarray(c, dtype=np.float32)
    n = c.shape[0]
    pos = np.arange(n) if positions is None else np.asarray(positions)
    p32 = float(np.float32(p))
    if p32 <= 0.0:
        raise ValueError("top_p must be > 0")
    if n == 0:
        e = np.zeros(0, np.int64)
        return Selection(e, 0, e, np.zeros(0), np.zeros(0))
    order = np.lexsort((pos, -_f64(c)))          # primary: c desc, then position asc
    ws = np.asarray(w, dtype=np.float64)[order]
    prefix = np.cumsum(ws)
    prefix_excl = np.concatenate(([0.0], prefix[:-1])) / Z
    if p32 >= 1.0:
        k = n
    else:
        target = p32 * Z
        hits = np.nonzero(prefix >= target)[0]
        k = int(hits[0]) + 1 if hits.size else n
    selected = np.sort(order[:k])
    return Selection(order, k, selected, prefix_excl, ws)


@dataclass
class BlockSelection:
    blocks: np.ndarray     # block ids (position // bs) of the candidates' blocks, ascending
    mass: np.ndarray       # calibrated mass of each block (float64)
    order: np.ndarray      # indices into `blocks` in rank order (mass desc, block id asc)
    k: int                 # number of kept blocks
    selected: np.ndarray   # kept candidate indices, ascending
    prefix_excl: np.ndarray  # exclusive prefix mass / Z in block rank order


def block_topp_head(w, Z, p, positions, bs: int) -> BlockSelection:
    """Smallest set of whole blocks whose calibrated mass reaches p.

    Reading of section 2.C ("Rewrite Cache": selected blocks are moved into
    contiguous ranges) and section 2.A (Tier 3 merges the oldest blocks):
    selection at the granularity of the paged cache's blocks.  Block j holds
    the candidates with position in [j bs, (j + 1) bs) (aligned to absolute
    positions, as the cache's pages are); its score is its calibrated mass,
    the sum of its candidates' weights w_t = exp(c_t - m).  Blocks are ranked
    by mass, highest first, equal masses by lower block id first; the kept
    blocks are the shortest rank prefix whose mass reaches p * Z (p taken as
    float32 and widened exactly); p >= 1 keeps every block.  Every candidate
    of a kept block is kept.  bs = 1 is token-level top-p.
    """
    pos = np.asarray(positions, np.int64)
    n = pos.shape[0]
    p32 = float(np.float32(p))
    if p32 <= 0.0 or bs < 1:
        raise ValueError("top_p must be > 0 and the block size >= 1")
    if n == 0:
        e = np.zeros(0, np.int64)
        return BlockSelection(e, np.zeros(0), e, 0, e, np.zeros(0))
    bid = pos // bs
    blocks, inv = np.unique(bid, return_inverse=True)
    mass = np.zeros(len(blocks))
    for t in range(n):                     # each candidate's weight into its block
        mass[inv[t]] += float(w[t])
    order = np.lexsort((blocks, -mass))    # primary: mass desc, then block id asc
    prefix = np.cumsum(mass[order])
    prefix_excl = np.concatenate(([0.0], prefix[:-1])) / Z
    if p32 >= 1.0:
        k = len(blocks)
    else:
        hits = np.nonzero(prefix >= p32 * Z)[0]
        k = int(hits[0]) + 1 if hits.size else len(blocks)
    kept = np.zeros(len(blocks), bool)
    kept[order[:k]] = True
    selected = np.nonzero(kept[inv])[0]
    return BlockSelection(blocks, mass, order, k, selected, prefix_excl)


# ---------------------------------------------------------------------------
# Condensed tier (section 2.A, Tier 3: oldest blocks compressed into
# constant-size storage by eviction or weighted merging).
# ---------------------------------------------------------------------------
MERGE_MEAN = 0       # chunk = plain mean of its evicted tokens
MERGE_WEIGHTED = 1   # chunk = attention-weighted mean of its evicted tokens
MERGE_FLOOR = -60.0  # log-weight floor of a token in weighted merging


def merge_weights(c, m):
    """Weights of evicted tokens for attention-weighted merging.

    Reading of "weighted merging" (section 2.A, Tier 3): a token enters its
    chunk with its calibrated attention weight exp(c - m), the quantity the
    top-p selection ranked it by.  The pages give no formula, and the weight
    needs a floor: exp(c - m) of a token far below the head's maximum is 0
    in any finite precision, which leaves the weighted mean of a chunk made
    only of such tokens undefined (0 / 0).  A weight below e^-60 counts as
    e^-60: such a chunk becomes the plain mean of its tokens (equal weights),
    and a chunk whose heaviest token has weight w_max moves by at most a
    relative n e^-60 / w_max (n tokens), nothing for any chunk holding a
    token within a few dozen nats of the maximum.  The value 60 is this
    reading's choice (about 26 decades below the heaviest token).
    """
    return np.exp(np.maximum(_f64(c) - float(m), MERGE_FLOOR))


def condense(K, V, evicted, positions, C: int, nchunks: int, weights=None, origin: int = 0):
    """Storage of evicted tokens in the condensed tier.

    Reading: chunks are aligned to the candidate range, chunk j holds the
    evicted tokens with position in [origin + jC, origin + (j+1)C) (origin =
    the first candidate position: 0, or the number of sink tokens).  Stored
    per chunk: the token count n and key / value sums such that sum / n is
    the chunk's representative key / value:
      mean merging (weights None): the plain sums;
      weighted merging: n * (sum_t a_t x_t) / (sum_t a_t), the weighted mean
      scaled by n, so both forms enter attention the same way.
    A chunk with no evicted token has count 0.
    """
    d = K.shape[1]
    ksum = np.zeros((nchunks, d))
    vsum = np.zeros((nchunks, d))
    wsum = np.zeros(nchunks)
    cnt = np.zeros(nchunks, np.int64)
    k64 = _f64(K)
    v64 = _f64(V)
    for n_i, i in enumerate(evicted):
        j = (int(positions[i]) - origin) // C
        a = 1.0 if weights is None else float(weights[n_i])
        ksum[j] += a * k64[i]
        vsum[j] += a * v64[i]
        wsum[j] += a
        cnt[j] += 1
    if weights is not None:
        nz = cnt > 0
        ksum[nz] *= (cnt[nz] / wsum[nz])[:, None]
        vsum[nz] *= (cnt[nz] / wsum[nz])[:, None]
    return ksum, vsum, cnt


# ---------------------------------------------------------------------------
# Decode attention over the three tiers.
# ---------------------------------------------------------------------------
def attend_head(q_group, dense_K, dense_V, sparse_K, sparse_V, ksum, vsum, cnt):
    """Softmax attention of each query row over dense, sparse and condensed.

    Dense and sparse entries use logit q.k / sqrt(d) and value v.  A non-empty
    chunk with count n enters once with key ksum/n and value vsum/n; reading:
    its logit carries + ln n, so that a chunk of n identical tokens weighs
    exactly as those n tokens would.  float64, max-subtracted.
    Returns [G, d] float64.
    """
    q = _f64(q_group)
    d = q.shape[1]
    scale = 1.0 / math.sqrt(d)
    keys = [_f64(dense_K), _f64(sparse_K)]
    vals = [_f64(dense_V), _f64(sparse_V)]
    bias = [np.zeros(len(dense_K)), np.zeros(len(sparse_K))]
    nz = np.nonzero(np.asarray(cnt) > 0)[0]
    if nz.size:
        n = np.asarray(cnt, dtype=np.float64)[nz]
        keys.append(np.asarray(ksum, np.float64)[nz] / n[:, None])
        vals.append(np.asarray(vsum, np.float64)[nz] / n[:, None])
        bias.append(np.log(n))
    Kall = np.concatenate(keys, axis=0).reshape(-1, d)
    Vall = np.concatenate(vals, axis=0).reshape(-1, d)
    ball = np.concatenate(bias)
    if Kall.shape[0] == 0:
        return np.zeros_like(q)
    logits = (q @ Kall.T) * scale + ball[None, :]
    logits -= logits.max(axis=1, keepdims=True)
    e = np.exp(logits)
    return (e @ Vall) / e.sum(axis=1, keepdims=True)


def full_attention(q_group, K, V):
    """Plain softmax attention of each query row over all rows of K/V."""
    q = _f64(q_group)
    d = q.shape[1]
    logits = (q @ _f64(K).T) / math.sqrt(d)
    logits -= logits.max(axis=1, keepdims=True)
    e = np.exp(logits)
    return (e @ _f64(V)) / e.sum(axis=1, keepdims=True)


# ---------------------------------------------------------------------------
# One decode step for one (sequence, KV head): the four-step pipeline of
# section 2.A (append, calibrate + top-p -> sparse mask, index
# regularisation, eviction / merging).
# ---------------------------------------------------------------------------
@dataclass
class HeadResult:
    A: int
    ell: np.ndarray
    s: np.ndarray
    cal: Calibration
    sel: Selection
    mask: np.ndarray       # uint8 [A]
    pos: np.ndarray        # compacted positions (ascending)
    Kc: np.ndarray         # compacted keys, bit copies of the input rows
    Vc: np.ndarray
    ksum: np.ndarray
    vsum: np.ndarray
    cnt: np.ndarray
    out: np.ndarray        # [G, d] float64
    extra: dict = field(default_factory=dict)
    sinks: int = 0         # leading positions held in the dense tier


def candidate_range(T: int, W: int, sinks: int = 0):
    """(first candidate position, number of candidates) of one step.

    Tier 1 keeps the last W tokens and, reading its mention of attention
    sinks (section 2.A, Tier 1) as the usual leading tokens, the first
    `sinks` positions; everything in between is a candidate for Tier 2:
    [S, T - W), empty when T <= S + W.
    """
    if sinks < 0:
        raise ValueError("sinks must be >= 0")
    A = aged_count(T, W)
    return sinks, max(A - sinks, 0)


def dense_positions(T: int, S: int, A: int) -> np.ndarray:
    """Positions of the dense tier: [0, T) without the candidates [S, S + A)."""
    return np.concatenate([np.arange(0, S if A else T), np.arange(S + A, T) if A else []]).astype(np.int64)


def keydiff_head(K):
    """Key-dissimilarity metric of one head's candidate keys.

    Section 2.B ("Goal") names similarity scores among the importance metrics
    the calibration brings into one probability space, and the pages list
    key-similarity-based eviction (KeyDiff) among related work.  Reading:
    s_t = -cos(k_t, mu) with mu = the sum of the candidate keys (the mean
    key's direction); a key whose direction differs most from the head's
    typical key ranks highest.  cos is taken as 0 when k_t or mu is the zero
    vector.  float64 from the exact inputs (the sum of bf16 or float32 keys),
    s = -(k_t . mu) / (||k_t|| ||mu||), rounded once to float32.
    """
    k = _f64(K)
    _check_finite(k)
    n = k.shape[0]
    if n == 0:
        return np.zeros(0, np.float32)
    mu = k.sum(axis=0)
    nm = float(np.sqrt(mu @ mu))
    nk = np.sqrt(np.einsum("nd,nd->n", k, k))
    dots = k @ mu
    s = np.zeros(n)
    ok = (nk > 0) & (nm > 0)
    s[ok] = -dots[ok] / (nk[ok] * nm)
    return s.astype(np.float32)


def redundancy_head(K):
    """R-KV redundancy metric of one head's candidate keys.

    Section 2.B ("Mechanism") names R-KV, a redundancy-aware strategy, among
    the selection strategies the calibration maps onto one softmax; the pages
    give no formula.  Reading: a candidate's redundancy is its mean cosine
    similarity to the other candidates, r_t = mean_{j != t} cos(k_t, k_j),
    and the metric is s_t = -r_t (the less a key repeats the others, the more
    it is worth keeping).  cos with a zero key is 0.  With unit keys
    u_j = k_j / ||k_j|| (u = 0 for a zero key) and nu = sum_j u_j, the sum over
    j != t is u_t . nu - [k_t != 0], so r_t = (u_t . nu - [k_t != 0]) / (A - 1),
    linear in the candidate count A; A = 1 gives r = 0.  float64 from the exact
    inputs, rounded once to float32.
    """
    k = _f64(K)
    _check_finite(k)
    n = k.shape[0]
    if n == 0:
        return np.zeros(0, np.float32)
    if n == 1:
        return np.zeros(1, np.float32)
    nk = np.sqrt(np.einsum("nd,nd->n", k, k))
    nz = nk > 0
    u = np.zeros_like(k)
    u[nz] = k[nz] / nk[nz, None]
    nu = u.sum(axis=0)
    r = (u @ nu - nz.astype(np.float64)) / (n - 1)
    return (-r).astype(np.float32)


def step_head(q_group, K, V, T: int, W: int, C: int, p: float, metric: int,
              sinks: int = 0, merge: int = MERGE_MEAN, q_hist=None,
              radius: int = 0, calib: int = CALIB_SPREAD, select_block: int = 0) -> HeadResult:
    """Single-step compression + attention of one KV head.

    K, V: [>=T, d] rows of this head's cache in position order (exact
    input values, any float dtype).  Candidates are [S, S + A) with
    (S, A) = candidate_range(T, W, sinks); the dense tier is every other
    position below T.  metric METRIC_WINDOW scores with ``window_score_head``
    over this query and q_hist (the previous queries, most recent first).
    Rewrite: the selected rows are copied, in ascending position order, into
    contiguous slots 0..k-1 (Rewrite Cache + Flatten Index to the maximum
    length, section 2.C).  Evicted candidates go to the condensed tier, mean-
    or attention-weighted-merged (``condense``).  select_block > 0 keeps whole
    blocks of that many positions (``block_topp_head``) instead of tokens.
    """
    S, A = candidate_range(T, W, sinks)
    cand_K = K[S:S + A]
    ell, s = score_head(q_group, cand_K)
    if metric == METRIC_KEYDIFF:
        s = keydiff_head(cand_K)
    if metric == METRIC_RKV:
        s = redundancy_head(cand_K)
    if metric == METRIC_WINDOW:
        # the window: this step's query, then the previous ones (q_hist [w-1, G, d])
        qw = [np.asarray(q_group)[None]]
        if q_hist is not None and len(q_hist):
            qw.append(np.asarray(q_hist))
        s = window_score_head(np.concatenate(qw, axis=0), cand_K, radius)
    cal = calibrate_head(ell, s, metric, calib)
    sel = topp_head(cal.c, cal.w, cal.Z, p)
    extra = {}
    if select_block > 0:
        bsel = block_topp_head(cal.w, cal.Z, p, S + np.arange(A), select_block)
        extra["blocks"] = bsel
        extra["block_size"] = select_block
        # the kept set is the blocks'; the token ranking stays for reference
        sel = Selection(sel.order, len(bsel.selected), bsel.selected, sel.prefix_excl,
                        sel.w_sorted)
    mask = np.zeros(A, np.uint8)
    mask[sel.selected] = 1
    evicted = np.nonzero(mask == 0)[0]
    nchunks = -(-A // C) if A else 0
    if merge == MERGE_MEAN:
        weights = None
    elif merge == MERGE_WEIGHTED:
        weights = merge_weights(cal.c[evicted], cal.m)
    else:
        raise ValueError("unknown merge rule")
    ksum, vsum, cnt = condense(K, V, S + evicted, np.arange(T), C, nchunks, weights, origin=S)
    pos = S + sel.selected
    Kc = np.asarray(K)[pos]
    Vc = np.asarray(V)[pos]
    dense = dense_positions(T, S, A)
    out = attend_head(q_group, np.asarray(K)[dense], np.asarray(V)[dense], Kc, Vc, ksum, vsum, cnt)
    return HeadResult(A, ell, s, cal, sel, mask, pos, Kc, Vc, ksum, vsum, cnt, out, extra, sinks=S)


def step(q, k_rows, v_rows, ctx_len, W, C, p, metric, sinks=0, merge=MERGE_MEAN):
    """Whole batch: q [B, Hq, d]; k_rows(b, h) / v_rows(b, h) return the
    [T_b, d] position-ordered rows of head h of sequence b; metric [Hkv].
    Query head g belongs to KV head g // G.  Returns {(b, h): HeadResult}.
    """
    q = np.asarray(q)
    B, Hq, d = q.shape
    Hkv = len(metric)
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    G = Hq // Hkv
    res = {}
    for b in range(B):
        T = int(ctx_len[b])
        for h in range(Hkv):
            res[(b, h)] = step_head(q[b, h * G:(h + 1) * G], k_rows(b, h), v_rows(b, h),
                                    T, W, C, p, int(metric[h]), sinks, merge)
    return res


# ---------------------------------------------------------------------------
# Multi-step lifecycle with in-place tiers (section 2.A: tokens move dense ->
# sparse -> condensed as they age; the sparse tier is re-selected each step).
# ---------------------------------------------------------------------------
@dataclass
class HeadState:
    """Tiers of one (layer, sequence, KV head) between decode steps.

    ring_K/ring_V: [W, d] dense window, the token at position t lives in slot
    t mod W.  pool_K/pool_V/pool_pos: the sparse tier, positions ascending.
    ksum/vsum/cnt: condensed chunks (running sums).
    """
    W: int
    C: int
    ring_K: np.ndarray
    ring_V: np.ndarray
    pool_K: np.ndarray
    pool_V: np.ndarray
    pool_pos: np.ndarray
    ksum: np.ndarray
    vsum: np.ndarray
    cnt: np.ndarray
    T: int                 # tokens seen so far (positions 0..T-1)
    # per chunk, the sums of |k| and |v| over the tokens merged so far: not
    # part of the method, the scale against which a float32 sum of the same
    # tokens is judged (relative error of a sum is bounded by that of
    # sum |x|)
    kabs: np.ndarray | None = None
    vabs: np.ndarray | None = None


def init_state(K, V, T0: int, W: int, C: int, nchunks: int) -> HeadState:
    """Initial tiers after a prefill of T0 tokens: dense = last W tokens,
    sparse pool = every older token, condensed = empty."""
    if T0 < W:
        raise ValueError("the multi-step lifecycle starts with a full window")
    d = K.shape[1]
    ring_K = np.zeros((W, d), K.dtype)
    ring_V = np.zeros((W, d), V.dtype)
    for t in range(T0 - W, T0):
        ring_K[t % W] = K[t]
        ring_V[t % W] = V[t]
    A = T0 - W
    return HeadState(W, C, ring_K, ring_V, np.array(K[:A]), np.array(V[:A]),
                     np.arange(A), np.zeros((nchunks, d)), np.zeros((nchunks, d)),
                     np.zeros(nchunks, np.int64), T0, np.zeros((nchunks, d)),
                     np.zeros((nchunks, d)))


def lifecycle_step(st: HeadState, q_group, k_new, v_new, p: float, metric: int):
    """One decode step of one head.

    (1) Append: the new token at position P = T goes into ring slot P mod W;
        the token it replaces (position P - W) leaves the window and is
        appended to the end of the sparse pool.
    (2) Score, calibrate and select top-p over the pool.
    (3) Rewrite: the kept pool rows are compacted, positions ascending.
    (4) Merge: every dropped pool token is added to the running sums of its
        position-aligned chunk; it never returns to another tier.
    Then attention over the ring, the rewritten pool and the chunks.
    Returns (out [G, d] float64, HeadResult-like dict of the step).
    """
    W, C = st.W, st.C
    P = st.T
    slot = P % W
    aged_pos = P - W
    st.pool_K = np.concatenate([st.pool_K, st.ring_K[slot][None]], axis=0)
    st.pool_V = np.concatenate([st.pool_V, st.ring_V[slot][None]], axis=0)
    st.pool_pos = np.concatenate([st.pool_pos, [aged_pos]])
    st.ring_K[slot] = k_new
    st.ring_V[slot] = v_new
    st.T = P + 1
    ell, s = score_head(q_group, st.pool_K)
    if metric == METRIC_KEYDIFF:
        s = keydiff_head(st.pool_K)
    if metric == METRIC_RKV:
        s = redundancy_head(st.pool_K)
    cal = calibrate_head(ell, s, metric)
    sel = topp_head(cal.c, cal.w, cal.Z, p, positions=st.pool_pos)
    keep = np.zeros(len(st.pool_pos), bool)
    keep[sel.selected] = True
    evicted = np.nonzero(~keep)[0]
    ks, vs, cn = condense(st.pool_K, st.pool_V, evicted, st.pool_pos, C, len(st.cnt))
    st.ksum += ks
    st.vsum += vs
    st.cnt += cn
    if st.kabs is not None:
        ka, va, _ = condense(np.abs(st.pool_K), np.abs(st.pool_V), evicted, st.pool_pos, C,
                             len(st.cnt))
        st.kabs += ka
        st.vabs += va
    n_before = len(st.pool_pos)
    st.pool_K = st.pool_K[keep]
    st.pool_V = st.pool_V[keep]
    st.pool_pos = st.pool_pos[keep]
    out = attend_head(q_group, st.ring_K, st.ring_V, st.pool_K, st.pool_V,
                      st.ksum, st.vsum, st.cnt)
    return out, {"n_candidates": n_before, "k": sel.k, "ell": ell, "s": s,
                 "cal": cal, "sel": sel}


# ---------------------------------------------------------------------------
# Rewrite versus Sparse Loading (section 2.C, "Techniques" and "Trade-off
# Management"): a selection is either rewritten into contiguous slots or
# left in place and loaded through its index; a Memory-Time Integral, with
# the budget thresholds L_lower and L_upper, decides per head.
# ---------------------------------------------------------------------------
POLICY_REWRITE = 0   # every head rewritten
POLICY_SPARSE = 1    # every head sparse-loaded
POLICY_MTI = 2       # thresholds, then the memory-time integral

MODE_REWRITE = 0
MODE_SPARSE = 1


def mti_head(A: int, k: int, W: int, horizon: int):
    """Memory-time integrals of serving one selection for `horizon` steps.

    The pages name the metric and what it balances (the one-off cost of the
    rewrite against the per-step gain) but give no formula.  Reading: the
    integral of the head's KV footprint over the time the steps take, both in
    units of one K or V row (the path is bandwidth-bound, so a step takes time
    in proportion to the rows it moves).  A horizon of N steps is the
    selection step plus N - 1 steps that reuse its tiers.

      footprint, sparse loading : A + W   every aged row stays where it is
      footprint, rewritten      : k + W   the kept rows only (the originals of
                                          the aged rows can be released)
      selection step, either    : 3A + 2W rows read (K to score, K and V to
                                          pool, the window's K and V)
      the rewrite's own cost    : 2k      rows written (K and V of each kept token)
      reuse step, either        : 2(k + W) rows read

    While the rewrite runs both copies of the kept rows exist (footprint
    A + W + k).  The window's growth during the horizon is the same in both
    modes and is left out.  Exact integers: (mti_rewrite, mti_sparse).
    """
    if min(A, k, W) < 0 or k > A or horizon < 1:
        raise ValueError("need 0 <= k <= A, W >= 0, horizon >= 1")
    foot_sparse = A + W
    foot_rewrite = k + W
    select_rows = 3 * A + 2 * W
    rewrite_rows = 2 * k
    reuse_rows = 2 * (k + W)
    mti_sparse = foot_sparse * select_rows + (horizon - 1) * foot_sparse * reuse_rows
    mti_rewrite = ((foot_sparse + k) * (select_rows + rewrite_rows)
                   + (horizon - 1) * foot_rewrite * reuse_rows)
    return mti_rewrite, mti_sparse


def plan_head(A: int, k: int, W: int, policy: int, horizon: int = 1,
              l_lower: int = 0, l_upper: int = 2 ** 31 - 1) -> int:
    """Rewrite (0) or sparse loading (1) for one head's selection.

    Reading of the budget thresholds: a budget k at or below L_lower is
    always rewritten (small, cheap to move, frees the most memory); one at or
    above L_upper is always loaded in place (a near-complete selection gains
    little from moving); in between the smaller memory-time integral wins,
    a tie going to sparse loading (nothing is moved).
    """
    if policy == POLICY_REWRITE:
        return MODE_REWRITE
    if policy == POLICY_SPARSE:
        return MODE_SPARSE
    if policy != POLICY_MTI:
        raise ValueError("unknown policy")
    if k <= l_lower:
        return MODE_REWRITE
    if k >= l_upper:
        return MODE_SPARSE
    mr, ms = mti_head(A, k, W, horizon)
    return MODE_REWRITE if mr < ms else MODE_SPARSE


def reuse_head(q_group, K, V, T_now: int, sel: HeadResult):
    """Attention at a later decode step that reuses an earlier selection.

    Reading: the tiers of the selection step serve the following steps
    unchanged; the tokens that left the W-window after the selection are
    not yet scored and stay dense, so at context length T_now the dense tier
    is [A_sel, T_now).  The kept rows are the cache rows at the selection's
    positions -- rewritten copies or, with sparse loading, the originals,
    which hold the same values.
    """
    if T_now < sel.sinks + sel.A:
        raise ValueError("the context only grows")
    dense = dense_positions(T_now, sel.sinks, sel.A)
    return attend_head(q_group, np.asarray(K)[dense], np.asarray(V)[dense],
                       np.asarray(K)[sel.pos], np.asarray(V)[sel.pos],
                       sel.ksum, sel.vsum, sel.cnt)


# ---------------------------------------------------------------------------
# Head-wise allocation of the rewritten tier (section 2.C, "Metadata": a
# head-wise block manager for head-adaptive allocation under static shapes;
# "Techniques": Flatten Index to the maximum length or to the sum).
# ---------------------------------------------------------------------------
def tier_alloc(table, held, free_ids, free_top: int, counts, modes, tier_block: int, cap: int):
    """One selection's block allocation for a block-managed rewritten tier.

    Reading of section 2.C ("Metadata": a head-wise block manager allocates
    head-adaptive budgets under static shapes; the pages give no allocation
    rule).  The rewritten tier is a pool of blocks of `tier_block` rows with a
    stack of free block ids; head i = (b, h) lists its blocks in table[i].
    Every selection re-lays the tier:
      1. every head, in (b, h) order, pushes its held blocks (table order)
         onto the free stack and holds none;
      2. every rewritten head, in (b, h) order, needs ceil(k / tier_block)
         blocks (k = its kept count clamped to [0, cap]) and pops them, one
         after another from the top of the stack, into table entries 0, 1, ...;
         a head whose need exceeds what the heads before it left is
         sparse-loaded instead and takes none (as pack_heads does for rows).
    table: [B][Hkv][maxb]; held, counts, modes: [B][Hkv]; free_ids: [blocks].
    Returns (table, held, free_ids, free_top, modes), new arrays; table
    entries at or past a head's held count are left as they were.
    """
    table = np.array(table, np.int64, copy=True)
    held = np.array(held, np.int64, copy=True)
    free = [int(x) for x in np.asarray(free_ids)[:free_top]]
    modes = np.array(modes, np.uint8, copy=True)
    counts = np.asarray(counts, np.int64)
    B, Hkv = counts.shape
    for b in range(B):
        for h in range(Hkv):
            for j in range(int(held[b, h])):
                free.append(int(table[b, h, j]))
            held[b, h] = 0
    avail = len(free)
    run = 0
    for b in range(B):
        for h in range(Hkv):
            need = 0
            if modes[b, h] == MODE_REWRITE:
                k = min(max(int(counts[b, h]), 0), cap)
                need = -(-k // tier_block)
            if run + need > avail:
                if modes[b, h] == MODE_REWRITE:
                    modes[b, h] = MODE_SPARSE
            else:
                for j in range(need):
                    table[b, h, j] = free.pop()
                held[b, h] = need
            run += need
    top = len(free)
    ids = np.asarray(free_ids, np.int64).copy()
    ids[:top] = free                      # the stack's live entries; the rest unspecified
    return table, held, ids, top, modes


def pack_heads(counts, modes, packed_rows: int):
    """Offsets of every head's rewritten rows in one shared region.

    Reading of the "sum" form of the Flatten Index: instead of a region of
    the maximum length per head, the heads' kept rows are laid end to end in
    one region of `packed_rows` rows, in (sequence, KV head) order.  A
    rewritten head needs k rows, a sparse-loaded head none; head i starts at
    the sum of the needs of the heads before it.  A rewritten head whose rows
    would end past the region is served by sparse loading instead (its rows
    stay in the cache), so every head's attention is unchanged.
    counts, modes: [B][Hkv].  Returns (offsets int64 [B][Hkv], modes uint8).
    """
    counts = np.asarray(counts, np.int64)
    modes = np.asarray(modes, np.uint8).copy()
    flat_k = counts.ravel()
    flat_m = modes.ravel()
    offsets = np.zeros(flat_k.size, np.int64)
    run = 0
    for i in range(flat_k.size):
        need = int(flat_k[i]) if flat_m[i] == MODE_REWRITE else 0
        offsets[i] = run
        if run + need > packed_rows:
            flat_m[i] = MODE_SPARSE
        run += need
    return offsets.reshape(counts.shape), flat_m.reshape(modes.shape)
