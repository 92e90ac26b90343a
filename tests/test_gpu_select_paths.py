"""GPU parity of wi_decode on indexes shaped to drive every branch of the per-head top-k select.

The select bounds the k-th largest score from the 8 best scores of each 128-cluster tile, gathers
the candidates from those summaries (scanning a tile in full only when its 8th best passes the
bound), and falls back to a radix select over every score when the candidates overflow LDS, when
more than 256 tiles need a full scan, or when the summaries themselves do not fit.  Each case
below forces one of those branches; all are checked against the oracle to the same gates as the
other decode tests (ids bit-exact, outputs to the dtype tolerance).

The last two cases run more than 256 query heads, where the select runs at half the block size.

Indexes come from oracle.finalize_index on random labels (no k-means), so that cluster counts,
empty clusters and crowding can be chosen directly.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from kv_vector_index_amd import synth
from kv_vector_index_amd import wave_index as wi
from wi_testutil import assert_decode_parity, device, upload_index

pytestmark = pytest.mark.gpu

SINK, WINDOW = 4, 16


def _case(C, tokens_per_cluster, Hq, Hkv, dtype, seed, empty_frac=0.1, crowd=0, crowd_heads=1, crowd_noise=0.05):
    """Random unit keys, Gaussian values, random labels with ~empty_frac empty clusters.  With
    crowd > 0, clusters 0 .. crowd-1 (all in the first tiles) hold keys close to one direction u
    (exactly u with crowd_noise 0: equal mean keys, so equal scores) and the first `crowd_heads`
    query heads of every group point at u."""
    rng = np.random.default_rng(seed)
    d = 128
    Nc = C * tokens_per_cluster
    N = Nc + SINK + WINDOW
    K = rng.standard_normal((1, Hkv, N, d))
    V = rng.standard_normal((1, Hkv, N, d))
    Q = 1.5 * rng.standard_normal((1, Hq, d)) / math.sqrt(d) * 8.0
    labels = np.empty((1, Hkv, Nc), dtype=np.int64)
    G = Hq // Hkv
    for g in range(Hkv):
        ids = np.arange(C)
        empty = rng.random(C) < empty_frac
        if crowd:
            empty[:crowd] = False
        live = ids[~empty]
        lab = np.concatenate([live, rng.choice(live, Nc - live.size)])
        rng.shuffle(lab)
        labels[0, g] = lab
        if crowd:
            u = rng.standard_normal(d)
            u /= np.linalg.norm(u)
            pos = SINK + np.nonzero(lab < crowd)[0]
            K[0, g, pos] = u + crowd_noise * rng.standard_normal((pos.size, d))
            for j in range(crowd_heads):
                Q[0, g * G + j] = 6.0 * u + 0.1 * rng.standard_normal(d)
    K /= np.linalg.norm(K, axis=-1, keepdims=True)
    dev = device()
    Kt, Vt, Qt = (synth.cast(x, dtype, dev) for x in (K, V, Q))
    K64, V64, Q64 = (synth.as_float64(t) for t in (Kt, Vt, Qt))
    idx = oracle.finalize_index(K64, V64, labels, SINK, WINDOW, C, dtype)
    return idx, Qt, Q64


def _check(idx, Qt, Q64, Hq, k, dtype):
    gi = upload_index(idx, dtype, device())
    o, lse, sel = wi.decode(gi, Qt, k)
    torch.cuda.synchronize()
    ro, rl, rs = oracle.decode(Q64, idx, Hq, k, 1 / math.sqrt(128))
    assert_decode_parity(o, lse, sel, ro, rl, rs, dtype)


def test_select_crowded_tile_is_scanned_in_full():
    # 40 of the best clusters sit in the first tile: its 8th best passes the bound
    idx, Qt, Q64 = _case(C=1024, tokens_per_cluster=3, Hq=8, Hkv=2, dtype="bf16", seed=1, crowd=40)
    _check(idx, Qt, Q64, Hq=8, k=50, dtype="bf16")


@pytest.mark.parametrize("seed", [11, 12, 13])
def test_select_threshold_above_the_summary_bound(seed):
    # crowded first tiles scanned in full: the k-th largest lies above the summaries' bound (more
    # than k - 1 clusters above it) or is the bound itself (nothing beyond the summaries above it)
    idx, Qt, Q64 = _case(C=1024, tokens_per_cluster=3, Hq=8, Hkv=2, dtype="bf16", seed=seed, crowd=40,
                         crowd_heads=4)
    for k in (6, 20, 45, 60):
        _check(idx, Qt, Q64, Hq=8, k=k, dtype="bf16")


def test_select_threshold_above_the_bound_among_many_candidates():
    # 700 crowded clusters and k = 600: more candidates than one wave ranks from its registers
    idx, Qt, Q64 = _case(C=2048, tokens_per_cluster=2, Hq=4, Hkv=1, dtype="bf16", seed=15, crowd=700,
                         crowd_heads=2)
    _check(idx, Qt, Q64, Hq=4, k=600, dtype="bf16")


def test_select_threshold_within_a_few_equal_scores():
    # 12 clusters with equal mean keys lead two heads of each group: the k-th largest is their
    # common score a few keys above the summaries' bound (found by walking up the distinct keys),
    # and the ties are broken by id
    idx, Qt, Q64 = _case(C=1024, tokens_per_cluster=3, Hq=8, Hkv=2, dtype="bf16", seed=16, crowd=12,
                         crowd_heads=2, crowd_noise=0.0)
    for k in (5, 10, 14):
        _check(idx, Qt, Q64, Hq=8, k=k, dtype="bf16")


def test_select_threshold_among_many_equal_scores():
    # 200 clusters with equal mean keys, the k-th largest among them: more than a wave's worth of
    # candidates share its histogram bin (the whole block searches), and the ties are broken by id
    idx, Qt, Q64 = _case(C=1024, tokens_per_cluster=3, Hq=8, Hkv=2, dtype="bf16", seed=14, crowd=200,
                         crowd_heads=2, crowd_noise=0.0)
    for k in (150, 230):
        _check(idx, Qt, Q64, Hq=8, k=k, dtype="bf16")


def test_select_candidates_overflow_to_radix_over_all_scores():
    # k = 3000 of 8192 clusters: more candidates than the LDS list holds
    idx, Qt, Q64 = _case(C=8192, tokens_per_cluster=2, Hq=4, Hkv=1, dtype="bf16", seed=2)
    _check(idx, Qt, Q64, Hq=4, k=3000, dtype="bf16")


def test_select_many_full_tiles_and_long_lists():
    # 288 tiles, k = 5000: nearly every tile's 8th best passes (more than 256 full tiles), and the
    # retrieved list is longer than the select keeps in LDS
    idx, Qt, Q64 = _case(C=36864, tokens_per_cluster=2, Hq=2, Hkv=1, dtype="bf16", seed=3)
    _check(idx, Qt, Q64, Hq=2, k=5000, dtype="bf16")


def test_select_list_published_in_several_rounds():
    # k = 9000 retrieved clusters: more than one publishing round of the select workgroup
    idx, Qt, Q64 = _case(C=36864, tokens_per_cluster=2, Hq=2, Hkv=1, dtype="bf16", seed=4)
    _check(idx, Qt, Q64, Hq=2, k=9000, dtype="bf16")


def test_select_without_tile_summaries():
    # 547 tiles: 4376 summary entries exceed what the select stages, so every score is visited
    idx, Qt, Q64 = _case(C=70000, tokens_per_cluster=1, Hq=4, Hkv=2, dtype="bf16", seed=5)
    _check(idx, Qt, Q64, Hq=4, k=120, dtype="bf16")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_select_many_empty_clusters(dtype):
    # 70% empty clusters: tiles with fewer than 8 non-empty ones, zero summary slots
    idx, Qt, Q64 = _case(C=2048, tokens_per_cluster=2, Hq=8, Hkv=2, dtype=dtype, seed=6, empty_frac=0.7)
    _check(idx, Qt, Q64, Hq=8, k=200, dtype=dtype)


def test_select_crowded_heads_with_all_retrieved_neighbour():
    # one head per group crowds the first tile, others are random; k covers every non-empty
    # cluster for a tiny index (the all-retrieved branch) in the same call as crowded heads
    idx, Qt, Q64 = _case(C=256, tokens_per_cluster=4, Hq=8, Hkv=2, dtype="bf16", seed=7, crowd=24,
                         crowd_heads=2)
    _check(idx, Qt, Q64, Hq=8, k=30, dtype="bf16")
    _check(idx, Qt, Q64, Hq=8, k=256, dtype="bf16")


def test_select_half_size_blocks_crowded_and_empty():
    # 272 query heads: the select runs two heads per CU at 512 threads; crowded first tiles for
    # two heads of every group, 10% empty clusters
    idx, Qt, Q64 = _case(C=1024, tokens_per_cluster=3, Hq=272, Hkv=34, dtype="bf16", seed=8, crowd=40,
                         crowd_heads=2)
    _check(idx, Qt, Q64, Hq=272, k=50, dtype="bf16")


def test_select_half_size_blocks_radix_fallback():
    # 264 query heads with more candidates than the LDS list holds (radix select over all scores)
    idx, Qt, Q64 = _case(C=4096, tokens_per_cluster=1, Hq=264, Hkv=33, dtype="f32", seed=9)
    _check(idx, Qt, Q64, Hq=264, k=2500, dtype="f32")
