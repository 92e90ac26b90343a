"""Wave-index oracle: the method step by step, in float64 NumPy.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import
this module.  It shares nothing with the HIP library.

Sources, cited as [tag section]:
  [RI-es]  "RetroInfer: A Vector Storage Engine for Scalable Long-Context LLM Inference",
           technical summary (gist.science/es/paper/2505.02922)
  [RI-pt]  same paper, lay explainer (gist.science/pt/paper/2505.02922)
  [RI-ar]  same paper, lay text + technical summary (gist.science/ar/paper/2505.02922)
  [SM64]   Steele, Lea, Flood, "Fast Splittable Pseudorandom Number Generators", OOPSLA 2014
  [DM01]   Dhillon, Modha, "Concept Decompositions for Large Sparse Text Data using Clustering",
           Machine Learning 42, 2001 (spherical k-means)
  [FKV-es] "FreeKV: Boosting KV Cache Retrieval for Efficient LLM Inference", technical summary
           (gist.science/es), section A items 1-2 (speculative retrieval, correction by a
           cosine threshold between consecutive queries)

What the pages fix: each decode query's attention is split into a steady zone (sink tokens and the
local window, exact), a retrieval zone (the clusters of a spherical-k-means index most similar to
the query, exact) and an estimation zone (every other cluster, approximated from its centroid and
its value sum) [RI-es 2.A items 1-3; RI-ar 2.a]; the index is built by k-means over segments of
the sequence [RI-es 3, "Clustering Segmentado"; RI-ar 2.a, last paragraph].  The estimation term
for a cluster of n_c tokens with mean key mu_c and value sum SV_c is n_c * exp(<q, mu_c>/sqrt(d))
* (SV_c / n_c) in the numerator and n_c * exp(<q, mu_c>/sqrt(d)) in the denominator, and the zone
results are merged with log-sum-exp.  Everything the pages leave open is a "reading", marked R<n>
below where the code takes it.

Parity pins (tests/test_oracle.py), per function:
  round_to_dtype ........ pinned: torch's float->bfloat16 conversion on random and edge values
  canonical_scores ...... pinned: exact rational dot products (fractions.Fraction) where exact,
                          and the fp64 error bound otherwise
  splitmix64 ............ pinned: published known-answer vector (seed 1234567)
  init_rows ............. pinned: uniform over permutations by exhaustive count on tiny n,
                          distinct and in range; the seed-mixing rule itself is a reading (R13)
  spherical_kmeans_segment pinned: zero-noise blobs recover the labels, sizes and directions;
                          objective non-decreasing; fixed-point consistency; brute-force Lloyd on
                          tiny inputs against exhaustive-search cluster labels
  finalize_index ........ pinned: CSR invariants, bit copies, recomputed sums; exactly: the
                          ascending-position float64 sum on a cancellation case where pairwise
                          and reversed orders differ, and the two-step float64 -> float32 ->
                          bfloat16 rounding on a double-rounding case
  build_index ........... pinned: segment independence, single-segment equivalence
  decode ................ pinned: all-retrieved equals dense softmax attention (textbook, and
                          torch SDPA in float64); keys equal to centroids make the estimate exact;
                          one token per cluster makes the estimate exact for any k; top-k equals
                          brute-force ranking with forced ties
  decode_gated .......... pinned: a threshold above 1 never reuses (equals decode); reusing a
                          step's own selection equals decode; reusing "every cluster" equals
                          dense attention; exact cosines of q with q, 2q and -q decide as
                          their closed forms; one drifting head makes its whole KV group
                          re-select; the refreshed selection equals decode's for every head
  bound_data ............ pinned: numpy's own norms within one float32 ulp and never below them;
                          a cluster of identical keys has radius 0
  bound_terms,
  prior_bounds,
  decode_bounded ........ pinned: the a-posteriori bound covers the distance to dense softmax
                          attention (textbook and torch SDPA) on random workloads and is
                          nearly attained (within 2x) by a closed-form two-member cluster; the
                          zone is the smallest meeting eps, A(k) is non-increasing, eps = 0
                          gives dense attention with bound 0, a forced k reproduces decode
Approximation quality against dense attention is "parity unpinned": the pages claim only
comparable accuracy, with no figure.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Tuple

import numpy as np

__all__ = [
    "round_to_dtype", "canonical_scores", "splitmix64", "segment_state", "init_rows",
    "steady_positions", "clustered_range", "segment_bounds", "spherical_kmeans_segment",
    "Index", "finalize_index", "build_index", "decode", "decode_head", "decode_gated",
    "query_cosine", "BoundData", "bound_data", "sum_roundoff", "bound_terms", "prior_bounds",
    "decode_bounded",
]

MASK64 = (1 << 64) - 1


# --------------------------------------------------------------------------------------------
# Storage rounding (reading R16): float64 -> float32 by round-to-nearest-even, then, for bf16,
# float32 -> bfloat16 by round-to-nearest-even.  Two steps, always.
# --------------------------------------------------------------------------------------------
def round_to_dtype(x, dtype: str) -> np.ndarray:
    """Round float64 values to the storage dtype; returns float64 holding the rounded values."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return f.astype(np.float64)
    if dtype != "bf16":
        raise ValueError(dtype)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    r = np.where(np.isnan(f), np.uint64(0x7FC0), r)
    return (r << np.uint64(16)).astype(np.uint32).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------------------------
# Canonical score (reading R22): sigma(x, y) = sum_j x_j * y_j where every product is exact in
# float64 (inputs carry at most 24 significant bits) and the sum runs in float64 in ascending j.
# Ranking by <q, mu_c> follows the pages' "attention-aware" index [RI-es 2.A; RI-ar 2.a].
# --------------------------------------------------------------------------------------------
def canonical_scores(X: np.ndarray, Y: np.ndarray) -> np.ndarray:
    """sigma[i, c] = sum over j ascending of X[i, j] * Y[c, j], float64, one rounding per add."""
    X = np.asarray(X, dtype=np.float64)
    Y = np.asarray(Y, dtype=np.float64)
    n, d = X.shape
    m = Y.shape[0]
    YT = np.ascontiguousarray(Y.T)
    out = np.empty((n, m))
    tmp = np.empty((min(n, 256), m))
    for r0 in range(0, n, 256):          # rows are independent; chunking only bounds memory
        Xr = X[r0:r0 + 256]
        acc = np.zeros((Xr.shape[0], m))
        t = tmp[:Xr.shape[0]]
        for j in range(d):
            np.multiply(Xr[:, j:j + 1], YT[j][None, :], out=t)
            acc += t
        out[r0:r0 + Xr.shape[0]] = acc
    return out


def _seq_sum_rows(rows: np.ndarray) -> np.ndarray:
    """Sum of the rows of a [n, d] array in float64, strictly in ascending row order."""
    acc = np.zeros(rows.shape[1])
    for r in rows:
        acc = acc + r
    return acc


def _seq_sum(v: np.ndarray) -> float:
    acc = 0.0
    for x in v:
        acc = acc + float(x)
    return acc


def _grouped_seq_sums(X: np.ndarray, members_sorted: np.ndarray, starts: np.ndarray,
                      counts: np.ndarray) -> np.ndarray:
    """Per-group sums of X rows, each group summed in float64 in its listed (ascending) order.

    ``members_sorted`` lists row indices group after group; group c owns
    ``members_sorted[starts[c] : starts[c] + counts[c]]``.  Step r adds the r-th member of every
    group that has one, so each group's sum is the plain left-to-right sum of its rows.
    """
    G = counts.shape[0]
    acc = np.zeros((G, X.shape[1]))
    maxc = int(counts.max()) if G else 0
    for r in range(maxc):
        act = np.nonzero(counts > r)[0]
        acc[act] = acc[act] + X[members_sorted[starts[act] + r]]
    return acc


# --------------------------------------------------------------------------------------------
# Seeded initialisation (reading R13): SplitMix64 [SM64] drives a partial Fisher-Yates shuffle of
# the segment's rows; the first Cs_eff = min(Cs, n_s) shuffled rows seed the clusters.
# --------------------------------------------------------------------------------------------
def splitmix64(state: int) -> Tuple[int, int]:
    """One SplitMix64 step [SM64]: returns (new_state, output)."""
    state = (state + 0x9E3779B97F4A7C15) & MASK64
    z = state
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return state, z ^ (z >> 31)


def segment_state(seed: int, b: int, g: int, s: int) -> int:
    """Initial SplitMix64 state of segment s of (sequence b, KV head g) (reading R13)."""
    sid = ((int(b) << 40) | (int(g) << 20) | int(s)) & MASK64
    return (int(seed) ^ ((sid * 0xD1B54A32D192ED03) & MASK64)) & MASK64


def init_rows(n: int, count: int, state: int) -> List[int]:
    """First ``count`` entries of a partial Fisher-Yates shuffle of range(n).

    Draw r (r = 0, 1, ...) takes x = SplitMix64 output, j = r + (x mod (n - r)), swaps a[r], a[j].
    """
    a = list(range(n))
    for r in range(count):
        state, x = splitmix64(state)
        j = r + x % (n - r)
        a[r], a[j] = a[j], a[r]
    return a[:count]


def _unit_rounded(x: np.ndarray, dtype: str) -> np.ndarray:
    """round_dtype(x / ||x||), the norm summed in float64 in ascending coordinate order.
    A zero vector (or one whose squared norm is zero) maps to the zero vector."""
    nrm2 = _seq_sum(x * x)
    if not nrm2 > 0.0:
        return np.zeros_like(x)
    return round_to_dtype(x / math.sqrt(nrm2), dtype)


# --------------------------------------------------------------------------------------------
# Zones and segments
# --------------------------------------------------------------------------------------------
def steady_positions(N: int, sink: int, window: int) -> np.ndarray:
    """Steady zone: the first ``sink`` and the last ``window`` positions, ascending, no repeats.

    Sink tokens and the local window are always attended exactly [RI-es 2.A item 1; RI-pt 2.A;
    RI-ar 2.a].  Reading R9: they are excluded from clustering, so the zones partition [0, N).
    """
    s = set(range(0, min(sink, N))) | set(range(max(N - window, 0), N))
    return np.array(sorted(s), dtype=np.int64)


def clustered_range(N: int, sink: int, window: int) -> Tuple[int, int]:
    """[lo, hi) of positions that are clustered (empty when the steady zone covers everything)."""
    if sink + window >= N:
        return (N, N)
    return (sink, N - window)


def segment_bounds(Nc: int, seg_len: int) -> List[Tuple[int, int]]:
    """Consecutive chunks of ``seg_len`` clustered tokens; the last may be shorter.  ``seg_len``
    of 0 means one segment.  Segmenting the sequence before k-means is the pages' way of cutting
    index-build time [RI-es 3; RI-ar 2.a] (reading R11 for the chunk rule)."""
    if Nc <= 0:
        return []
    L = Nc if seg_len <= 0 else seg_len
    return [(a, min(a + L, Nc)) for a in range(0, Nc, L)]


# --------------------------------------------------------------------------------------------
# Spherical k-means on one segment [RI-es 2.A item 2; RI-ar 2.a; DM01]
# --------------------------------------------------------------------------------------------
def spherical_kmeans_segment(Kseg: np.ndarray, Cs: int, iters: int, dtype: str, state: int,
                             history: bool = False):
    """Lloyd iterations of spherical k-means over one segment's keys.

    Returns (assign [n] local cluster ids of the last assignment, sums [Cs, d] float64 key sums of
    that assignment, counts [Cs]) and, if ``history``, a list of (assign, mhat) per iteration,
    where mhat is the set of centroid directions the assignment was made against.

    Per iteration (readings R3, R4, R7, R12):
      assign : a_i = argmax_j sigma(k_i, mhat_j) over j < Cs_eff, ties to the lower j
      sums   : m_j = sum of the member keys in float64, ascending i; n_j = member count
      update : mhat_j = round_dtype(m_j / sqrt(sum_t m_jt^2)) if n_j > 0 (sums ascending t),
               else mhat_j is kept
    """
    Kseg = np.asarray(Kseg, dtype=np.float64)
    n, d = Kseg.shape
    cs_eff = min(Cs, n)
    mhat = np.zeros((Cs, d))
    for j, r in enumerate(init_rows(n, cs_eff, state)):
        mhat[j] = _unit_rounded(Kseg[r], dtype)
    hist = []
    assign = np.zeros(n, dtype=np.int64)
    sums = np.zeros((Cs, d))
    counts = np.zeros(Cs, dtype=np.int64)
    for _ in range(iters):
        if cs_eff == 0:
            break
        sc = canonical_scores(Kseg, mhat[:cs_eff])
        assign = np.argmax(sc, axis=1).astype(np.int64)     # first maximum = lower id on ties
        if history:
            hist.append((assign.copy(), mhat.copy()))
        counts = np.bincount(assign, minlength=Cs).astype(np.int64)
        order = np.argsort(assign, kind="stable")           # members of each cluster, ascending i
        starts = np.concatenate([[0], np.cumsum(counts)[:-1]]).astype(np.int64)
        sums = _grouped_seq_sums(Kseg, order, starts, counts)
        for j in range(cs_eff):
            if counts[j] > 0:
                nrm2 = _seq_sum(sums[j] * sums[j])
                if nrm2 > 0.0:
                    mhat[j] = round_to_dtype(sums[j] / math.sqrt(nrm2), dtype)
    if history:
        return assign, sums, counts, hist
    return assign, sums, counts


# --------------------------------------------------------------------------------------------
# The index
# --------------------------------------------------------------------------------------------
@dataclasses.dataclass
class Index:
    """Wave index of a batch: every array is float64 (holding dtype values) or int64."""
    centroids: np.ndarray     # [B,Hkv,C,d]  mean key mu_c (reading R1)
    value_sums: np.ndarray    # [B,Hkv,C,d]  sum of member values
    sizes: np.ndarray         # [B,Hkv,C]
    offsets: np.ndarray       # [B,Hkv,C+1]
    perm: np.ndarray          # [B,Hkv,Nc]   absolute token positions, cluster-major
    k_perm: np.ndarray        # [B,Hkv,Nc,d]
    v_perm: np.ndarray        # [B,Hkv,Nc,d]
    k_steady: np.ndarray      # [B,Hkv,NS,d]
    v_steady: np.ndarray      # [B,Hkv,NS,d]
    C: int
    Nc: int


def finalize_index(K: np.ndarray, V: np.ndarray, labels: np.ndarray, sink: int, window: int,
                   C: int, dtype: str) -> Index:
    """Index from a cluster label per clustered token ([B,Hkv,Nc], values in [0, C)).

    sizes n_c; offsets = exclusive prefix sum; perm = clusters in id order, ascending position
    inside a cluster; mu_c = round_dtype(sum k / n_c); SV_c = round_dtype(sum v); both sums in
    float64 in ascending position; empty clusters get n = 0, mu = 0, SV = 0 (reading R7).
    Centroids and value sums are what the estimation zone uses [RI-ar 2.a]; the cluster-major copy
    of K and V plays the role of the pages' contiguous execution buffer [RI-ar 2.b].
    """
    B, Hkv, N, d = K.shape
    steady = steady_positions(N, sink, window)
    lo, hi = clustered_range(N, sink, window)
    Nc = hi - lo
    mu = np.zeros((B, Hkv, C, d))
    sv = np.zeros((B, Hkv, C, d))
    sizes = np.zeros((B, Hkv, C), dtype=np.int64)
    offsets = np.zeros((B, Hkv, C + 1), dtype=np.int64)
    perm = np.zeros((B, Hkv, Nc), dtype=np.int64)
    for b in range(B):
        for g in range(Hkv):
            lab = np.asarray(labels[b, g], dtype=np.int64)
            assert lab.shape == (Nc,) and (Nc == 0 or (lab.min() >= 0 and lab.max() < C))
            cnt = np.bincount(lab, minlength=C).astype(np.int64)
            off = np.concatenate([[0], np.cumsum(cnt)]).astype(np.int64)
            order = np.argsort(lab, kind="stable")
            pos = lo + order
            Kc = K[b, g, lo:hi]
            Vc = V[b, g, lo:hi]
            ksum = _grouped_seq_sums(Kc, order, off[:-1], cnt)
            vsum = _grouped_seq_sums(Vc, order, off[:-1], cnt)
            ne = cnt > 0
            mu[b, g, ne] = round_to_dtype(ksum[ne] / cnt[ne][:, None], dtype)
            sv[b, g, ne] = round_to_dtype(vsum[ne], dtype)
            sizes[b, g] = cnt
            offsets[b, g] = off
            perm[b, g] = pos
    bidx = np.arange(B)[:, None, None]
    gidx = np.arange(Hkv)[None, :, None]
    return Index(
        centroids=mu, value_sums=sv, sizes=sizes, offsets=offsets, perm=perm,
        k_perm=K[bidx, gidx, perm], v_perm=V[bidx, gidx, perm],
        k_steady=K[:, :, steady], v_steady=V[:, :, steady], C=C, Nc=Nc)


def build_index(K: np.ndarray, V: np.ndarray, sink: int, window: int, seg_len: int,
                clusters_per_seg: int, iters: int, seed: int, dtype: str,
                return_labels: bool = False):
    """Segmented spherical k-means over the clustered range of every (b, g), then finalize.

    Cluster ids are global per (b, g): segment s owns ids [s*Cs, (s+1)*Cs) (reading R11).
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, Hkv, N, d = K.shape
    lo, hi = clustered_range(N, sink, window)
    Nc = hi - lo
    segs = segment_bounds(Nc, seg_len)
    Cs = clusters_per_seg
    C = len(segs) * Cs
    labels = np.zeros((B, Hkv, Nc), dtype=np.int64)
    for b in range(B):
        for g in range(Hkv):
            for s, (a, e) in enumerate(segs):
                assign, _, _ = spherical_kmeans_segment(
                    K[b, g, lo + a:lo + e], Cs, iters, dtype, segment_state(seed, b, g, s))
                labels[b, g, a:e] = s * Cs + assign
    idx = finalize_index(K, V, labels, sink, window, C, dtype)
    return (idx, labels) if return_labels else idx


# --------------------------------------------------------------------------------------------
# Decode [RI-es 2.A items 1-3; RI-ar 2.a]
# --------------------------------------------------------------------------------------------
def _select(sigma: np.ndarray, sizes: np.ndarray, k: int) -> np.ndarray:
    """Retrieval zone: the k_eff = min(k, #non-empty) non-empty clusters first in the order
    (-sigma_c, c) -- highest score first, lower id on ties (readings R2, R5, R6, R8).  Returned in
    ascending id order."""
    cand = np.nonzero(sizes > 0)[0]
    k_eff = min(int(k), cand.size)
    order = np.lexsort((cand, -sigma[cand]))                # primary -sigma, then id
    return np.sort(cand[order[:k_eff]])


def decode_head(q: np.ndarray, idx: Index, b: int, g: int, k: int, scale: float,
                R: Optional[np.ndarray] = None):
    """One query head's decode step.  Returns (o [d], lse, sel_ids ascending).  The retrieval zone
    is the head's top-k unless ``R`` (ascending cluster ids) is given."""
    mu = idx.centroids[b, g]
    sizes = idx.sizes[b, g]
    off = idx.offsets[b, g]
    sigma = canonical_scores(q[None, :], mu)[0] if idx.C > 0 else np.zeros(0)
    if R is None:
        R = _select(sigma, sizes, k)

    # exact part: steady rows and every row of the retrieved clusters [RI-es 2.A items 1-2]
    rows = [np.arange(off[c], off[c + 1]) for c in R]
    rows = np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64)
    Kx = np.concatenate([idx.k_steady[b, g], idx.k_perm[b, g][rows]])
    Vx = np.concatenate([idx.v_steady[b, g], idx.v_perm[b, g][rows]])
    if Kx.shape[0]:
        lg = (Kx @ q) * scale
        m1 = lg.max()
        p = np.exp(lg - m1)
        den1 = p.sum()
        num1 = p @ Vx
    else:
        m1, den1, num1 = -np.inf, 0.0, np.zeros(q.shape[0])

    # estimation part: every other non-empty cluster from its centroid, size and value sum
    # [RI-es 2.A item 3; RI-ar 2.a]:  den += n_c e^{s_c},  num += n_c e^{s_c} (SV_c / n_c)
    est = np.setdiff1d(np.nonzero(sizes > 0)[0], R)
    if est.size:
        s = sigma[est] * scale
        m2 = s.max()
        w = np.exp(s - m2)
        n_c = sizes[est].astype(np.float64)
        den2 = (n_c * w).sum()
        num2 = ((n_c * w)[:, None] * (idx.value_sums[b, g][est] / n_c[:, None])).sum(axis=0)
    else:
        m2, den2, num2 = -np.inf, 0.0, np.zeros(q.shape[0])

    # log-sum-exp merge of the two partial softmax states (an empty part contributes nothing)
    M = max(m1, m2)
    a1 = math.exp(m1 - M) if den1 > 0 else 0.0
    a2 = math.exp(m2 - M) if den2 > 0 else 0.0
    den = a1 * den1 + a2 * den2
    o = (a1 * num1 + a2 * num2) / den
    lse = M + math.log(den)
    return o, lse, R


def decode(Q: np.ndarray, idx: Index, Hq: int, k: int, scale: Optional[float] = None):
    """Batched GQA decode: Q [B,Hq,d] -> (o [B,Hq,d] float64, lse [B,Hq], sel [B,Hq,k] int64).

    Query head h uses KV head h // (Hq / Hkv) (reading R17); sel_ids are ascending, padded
    with -1.
    """
    Q = np.asarray(Q, dtype=np.float64)
    B, _, d = Q.shape
    Hkv = idx.centroids.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = np.zeros((B, Hq, d))
    lse = np.zeros((B, Hq))
    sel = np.full((B, Hq, k), -1, dtype=np.int64)
    for b in range(B):
        for h in range(Hq):
            oh, lh, R = decode_head(Q[b, h], idx, b, h // G, k, scale)
            o[b, h], lse[b, h] = oh, lh
            sel[b, h, :R.size] = R
    return o, lse, sel


# --------------------------------------------------------------------------------------------
# Selection reuse across decode steps with a cosine gate [FKV-es A items 1-2].  Consecutive
# queries are similar, so a KV head keeps the clusters its query heads retrieved at the previous
# step unless the queries moved: the cosine C between the current and the previous query of a
# head is computed, and a KV head whose query heads all have C >= tau reuses their previous
# retrieval zones (reading R26); every other KV head selects afresh.  Scoring still runs for
# every head, because the estimation zone (every non-empty cluster outside the reused zone)
# needs the current query's scores (reading R27).  For the heads that kept their zone, the
# selection of the current query is not skipped but postponed past this step's attention: it is
# what the next step reuses, so a kept zone is always one step old (``refresh``, reading R28).
# --------------------------------------------------------------------------------------------
def query_cosine(q: np.ndarray, q_prev: np.ndarray) -> float:
    """<q, q'> / (||q|| ||q'||) from canonical sums (ascending coordinate order, exact products),
    IEEE float64 square roots and division; 0 when either query is zero (reading R26)."""
    dot = canonical_scores(q[None, :], q_prev[None, :])[0, 0]
    n1 = canonical_scores(q[None, :], q[None, :])[0, 0]
    n2 = canonical_scores(q_prev[None, :], q_prev[None, :])[0, 0]
    if n1 == 0.0 or n2 == 0.0:
        return 0.0
    return float(dot / (math.sqrt(n1) * math.sqrt(n2)))


def decode_gated(Q: np.ndarray, Q_prev: np.ndarray, sel_prev: np.ndarray, idx: Index, Hq: int, k: int,
                 tau: float, scale: Optional[float] = None, refresh: bool = False):
    """Batched decode with selection reuse: as ``decode``, except that a KV head whose query heads
    all satisfy query_cosine(q, q_prev) >= tau takes each head's retrieval zone from ``sel_prev``
    [B,Hq,k] (cluster ids; entries outside [0, C) are skipped and repeats count once).  Returns
    (o, lse, sel, reused [B,Hkv] bool); sel is the zone each head attended over, or with
    ``refresh`` the top-k of the current query for every head (the postponed selection)."""
    Q = np.asarray(Q, dtype=np.float64)
    Q_prev = np.asarray(Q_prev, dtype=np.float64)
    B, _, d = Q.shape
    Hkv = idx.centroids.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = np.zeros((B, Hq, d))
    lse = np.zeros((B, Hq))
    sel = np.full((B, Hq, k), -1, dtype=np.int64)
    reused = np.zeros((B, Hkv), dtype=bool)
    for b in range(B):
        for g in range(Hkv):
            heads = range(g * G, (g + 1) * G)
            reuse = all(query_cosine(Q[b, h], Q_prev[b, h]) >= tau for h in heads)
            reused[b, g] = reuse
            for h in heads:
                R = None
                if reuse:
                    # the previous zone: its ids in [0, C), each once (-1 pads the list)
                    prev = np.asarray(sel_prev[b, h])
                    R = np.unique(prev[(prev >= 0) & (prev < idx.C)]).astype(np.int64)
                oh, lh, Rh = decode_head(Q[b, h], idx, b, g, k, scale, R)
                o[b, h], lse[b, h] = oh, lh
                if refresh and reuse:
                    sigma = canonical_scores(Q[b, h][None, :], idx.centroids[b, g])[0] if idx.C > 0 else np.zeros(0)
                    Rh = _select(sigma, idx.sizes[b, g], k)
                sel[b, h, :Rh.size] = Rh
    return o, lse, sel, reused


# --------------------------------------------------------------------------------------------
# Accuracy-bounded estimation.  The pages promise a controlled error bound for the estimation
# zone [RI-es 2.A item 3; RI-ar 2.a, "accuracy-bound attention estimation"] but state no formula;
# the bound below is derived here (reading R29).  For a query q, scale s, a cluster c with stored
# mean key mu_c, n_c members, radius r_c = max ||k_i - mu_c|| and largest value norm V_c:
#   every member's weight e_i = exp(s <q, k_i>) lies within exp(+-s ||q|| r_c) of
#   e_c = exp(s <q, mu_c>), so |e_i - e_c| <= e_c (exp(x_c) - 1) with x_c = s ||q|| r_c, and
#   e_i >= e_c exp(-x_c).
# With E the estimated clusters, D_x the exact part's denominator, o the dense output and o^ the
# method's, o - o^ = [sum_E sum_i (e_i - e_c)(v_i - o^) + sum_E e_c (SumV_c - SV_c)] / D, hence
#   ||o - o^|| <= sum_E [n_c e_c (exp(x_c) - 1)(V_c + ||o^||) + e_c u n_c V_c]
#                 / (D_x + sum_E n_c e_c exp(-x_c))
# where u bounds the relative rounding of the stored value sums SV_c (sum_roundoff).  Before the
# attention, D_x >= sum over the retrieved clusters of n_c e_c exp(-x_c) and ||o^|| <=
# (1 + u) V_all (the largest value norm of the context) give the a-priori bound A(k) of the zone
# made of the k first clusters in the selection order; the zone size is the smallest k with
# A(k) <= eps, capped at top_k (reading R30).
# --------------------------------------------------------------------------------------------
@dataclasses.dataclass
class BoundData:
    """Per-cluster data of the bound, float64 arrays holding float32 values rounded up."""
    radius: np.ndarray        # [B,Hkv,C]  max ||k_i - mu_c|| over the members (0 if empty)
    vnorm: np.ndarray         # [B,Hkv,C]  max ||v_i|| over the members (0 if empty)
    vmax: np.ndarray          # [B,Hkv]    max ||v|| over every token, steady zone included


def _sqrt_up_f32(d2: float) -> float:
    """Smallest float32 f >= 0 with f * f >= d2: the square root of d2 >= 0 rounded up to float32
    (f * f is exact in float64, so the test is exact)."""
    f = np.float32(math.sqrt(d2))
    if float(f) * float(f) < d2:
        f = np.nextafter(f, np.float32(np.inf))
    else:
        while f > 0:
            p = np.nextafter(f, np.float32(0))
            if float(p) * float(p) < d2:
                break
            f = p
    return float(f)


def _seq_sq_norms(X: np.ndarray) -> np.ndarray:
    """Row-wise sum over j ascending of X[:, j]^2 in float64 (rounded square, then rounded add)."""
    acc = np.zeros(X.shape[0])
    for j in range(X.shape[1]):
        acc = acc + X[:, j] * X[:, j]
    return acc


def bound_data(idx: Index) -> BoundData:
    """Radius and value norms of every cluster, and the largest value norm of each (b, g): the
    squared distances and norms are sums over coordinates in ascending order (differences and
    squares rounded to float64), maximised over the members, then square-rooted and rounded up to
    float32 (reading R31)."""
    B, Hkv, C = idx.sizes.shape
    radius = np.zeros((B, Hkv, C))
    vnorm = np.zeros((B, Hkv, C))
    vmax = np.zeros((B, Hkv))
    for b in range(B):
        for g in range(Hkv):
            off = idx.offsets[b, g]
            dk = np.zeros(idx.Nc)
            for c in np.nonzero(idx.sizes[b, g] > 0)[0]:
                rows = slice(off[c], off[c + 1])
                dk[rows] = _seq_sq_norms(idx.k_perm[b, g, rows] - idx.centroids[b, g, c][None, :])
            dv = _seq_sq_norms(idx.v_perm[b, g])
            for c in np.nonzero(idx.sizes[b, g] > 0)[0]:
                rows = slice(off[c], off[c + 1])
                radius[b, g, c] = _sqrt_up_f32(dk[rows].max())
                vnorm[b, g, c] = _sqrt_up_f32(dv[rows].max())
            ds = _seq_sq_norms(idx.v_steady[b, g])
            top = max(dv.max() if dv.size else 0.0, ds.max() if ds.size else 0.0)
            vmax[b, g] = _sqrt_up_f32(top)
    return BoundData(radius=radius, vnorm=vnorm, vmax=vmax)


def sum_roundoff(dtype: str) -> float:
    """Relative rounding bound of the stored value sums: float64 -> float32 (2^-24), then for
    bf16 float32 -> bfloat16 (2^-8), compounded (2^-8 + 2^-24 + 2^-32 < 2^-8 + 2^-23)."""
    return {"bf16": 2.0 ** -8 + 2.0 ** -23, "f32": 2.0 ** -24}[dtype]


def bound_terms(q: np.ndarray, idx: Index, bd: BoundData, b: int, g: int, scale: float, dtype: str):
    """Per-cluster terms of the bound for one query head, in the frame m* = max over non-empty
    clusters of s sigma_c: w_c = n_c exp(s sigma_c - m*), a_c = w_c (exp(x_c) - 1),
    err_c = a_c (V_c + (1 + u) V_all) + w_c u V_c, lo_c = w_c exp(-x_c); zero for empty clusters.
    Returns (sigma, order, m*, w, a, err, lo) with ``order`` the non-empty clusters in the
    selection order (-sigma_c, c)."""
    sizes = idx.sizes[b, g]
    sigma = canonical_scores(q[None, :], idx.centroids[b, g])[0] if idx.C > 0 else np.zeros(0)
    ne = np.nonzero(sizes > 0)[0]
    order = ne[np.lexsort((ne, -sigma[ne]))]
    qn = math.sqrt(canonical_scores(q[None, :], q[None, :])[0, 0])
    u = sum_roundoff(dtype)
    w = np.zeros(idx.C)
    a = np.zeros(idx.C)
    err = np.zeros(idx.C)
    lo = np.zeros(idx.C)
    mstar = float((scale * sigma[ne]).max()) if ne.size else 0.0
    if ne.size:
        x = scale * qn * bd.radius[b, g, ne]
        w[ne] = sizes[ne] * np.exp(scale * sigma[ne] - mstar)
        a[ne] = w[ne] * np.expm1(x)
        err[ne] = a[ne] * (bd.vnorm[b, g, ne] + (1 + u) * bd.vmax[b, g]) + w[ne] * u * bd.vnorm[b, g, ne]
        lo[ne] = w[ne] * np.exp(-x)
    return sigma, order, mstar, w, a, err, lo


def prior_bounds(err: np.ndarray, lo: np.ndarray, order: np.ndarray) -> np.ndarray:
    """A(k) for k = 0 .. len(order): the err_c of the clusters after the first k of ``order``,
    summed, over the sum of every lo_c."""
    den = lo[order].sum()
    tail = err[order][::-1].cumsum()[::-1]            # tail[k] = sum of err over order[k:]
    A = np.zeros(order.size + 1)
    if order.size:
        A[:-1] = tail / den
    return A


def decode_bounded(Q: np.ndarray, idx: Index, bd: BoundData, Hq: int, k_max: int, eps: float,
                   dtype: str, scale: Optional[float] = None, k_force: Optional[np.ndarray] = None):
    """Decode with accuracy-bounded zone sizing: each head retrieves the k first clusters of its
    selection order, k the smallest in [0, min(k_max, #non-empty)] with A(k) <= eps (else the
    cap).  ``k_force`` [B,Hq] imposes k instead.  Returns (o, lse, sel [B,Hq,k_max], k [B,Hq],
    A(k) [B,Hq], bound [B,Hq]) with bound the a-posteriori bound on ||o - dense attention||."""
    Q = np.asarray(Q, dtype=np.float64)
    B, _, d = Q.shape
    Hkv = idx.centroids.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    u = sum_roundoff(dtype)
    o = np.zeros((B, Hq, d))
    lse = np.zeros((B, Hq))
    sel = np.full((B, Hq, k_max), -1, dtype=np.int64)
    ks = np.zeros((B, Hq), dtype=np.int64)
    prior = np.zeros((B, Hq))
    post = np.zeros((B, Hq))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            q = Q[b, h]
            sigma, order, mstar, w, a, err, lo = bound_terms(q, idx, bd, b, g, scale, dtype)
            A = prior_bounds(err, lo, order)
            cap = min(int(k_max), order.size)
            if k_force is not None:
                k = int(k_force[b, h])
            else:
                ok = np.nonzero(A[:cap + 1] <= eps)[0]
                k = int(ok[0]) if ok.size else cap
            R = np.sort(order[:k])
            oh, lh, _ = decode_head(q, idx, b, g, k, scale, R)
            o[b, h], lse[b, h] = oh, lh
            sel[b, h, :k] = R
            ks[b, h] = k
            prior[b, h] = A[k]
            # exact part's denominator in the frame m*: steady rows and the zone's rows
            off = idx.offsets[b, g]
            rows = np.concatenate([np.arange(off[c], off[c + 1]) for c in R]) if k else np.zeros(0, np.int64)
            Kx = np.concatenate([idx.k_steady[b, g], idx.k_perm[b, g][rows]])
            Dx = float(np.exp((Kx @ q) * scale - mstar).sum()) if Kx.shape[0] else 0.0
            E = order[k:]
            num = (a[E] * (bd.vnorm[b, g, E] + np.linalg.norm(oh))).sum() + (w[E] * u * bd.vnorm[b, g, E]).sum()
            post[b, h] = num / (Dx + lo[E].sum()) if E.size else 0.0
    return o, lse, sel, ks, prior, post
