"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test names what it pins: a library routine (torch's bf16 conversion, torch SDPA), exact
rational arithmetic (fractions.Fraction), a published known-answer vector, a closed form the pages
imply (all clusters retrieved = dense attention; keys equal to centroids = exact estimate), or
brute force on tiny inputs.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from kv_vector_index_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ storage rounding
def test_round_to_dtype_matches_torch_bf16():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
        [0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 3.3895313892515355e38, 1e-40, -1e-45,
         1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -30],
    ])
    ref = torch.from_numpy(x).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_to_dtype(x, "bf16")
    np.testing.assert_array_equal(got.view(np.uint64), ref.view(np.uint64))
    assert np.isnan(oracle.round_to_dtype(np.array([np.nan]), "bf16")).all()


def test_round_to_dtype_f32_is_ieee_single():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(1000) * 1e3
    ref = torch.from_numpy(x).to(torch.float32).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_to_dtype(x, "f32"), ref)


# ------------------------------------------------------------------ canonical score
def _exact_dot(x, y):
    return sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x, y)), Fraction(0))


def test_canonical_scores_equal_exact_rational_for_bf16_inputs():
    rng = np.random.default_rng(3)
    X = oracle.round_to_dtype(rng.standard_normal((12, 16)), "bf16")
    Y = oracle.round_to_dtype(rng.standard_normal((9, 16)), "bf16")
    S = oracle.canonical_scores(X, Y)
    for i in range(X.shape[0]):
        for c in range(Y.shape[0]):
            # bf16 products have 16 significant bits and these sums span few binades: exact
            assert Fraction(S[i, c]) == _exact_dot(X[i], Y[c])


def test_canonical_scores_within_fp64_bound_for_f32_inputs():
    rng = np.random.default_rng(4)
    X = oracle.round_to_dtype(rng.standard_normal((6, 128)), "f32")
    Y = oracle.round_to_dtype(rng.standard_normal((5, 128)), "f32")
    S = oracle.canonical_scores(X, Y)
    gamma = 128 * 2.0 ** -53 / (1 - 128 * 2.0 ** -53)
    for i in range(6):
        for c in range(5):
            ex = _exact_dot(X[i], Y[c])
            bound = gamma * float(np.abs(X[i] * Y[c]).sum())
            assert abs(float(Fraction(S[i, c]) - ex)) <= bound


def test_canonical_scores_sum_in_ascending_coordinate_order():
    # 1 + 2^-53 rounds back to 1 (ties to even) twice in ascending order; any other order that
    # adds the two small terms first would give 1 + 2^-52.
    X = np.array([[1.0, 1.0, 1.0]])
    Y = np.array([[1.0, 2.0 ** -53, 2.0 ** -53]])
    assert oracle.canonical_scores(X, Y)[0, 0] == 1.0
    Y2 = np.array([[2.0 ** -53, 2.0 ** -53, 1.0]])
    assert oracle.canonical_scores(X, Y2)[0, 0] == 1.0 + 2.0 ** -52


# ------------------------------------------------------------------ seeded init
def _golden_splitmix():
    vals = []
    with open(os.path.join(GOLDEN, "splitmix64_seed1234567.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                vals.append(int(line))
    return vals


def test_splitmix64_known_answer():
    want = _golden_splitmix()
    s = 1234567
    got = []
    for _ in range(len(want)):
        s, x = oracle.splitmix64(s)
        got.append(x)
    assert got == want


def test_init_rows_distinct_in_range():
    for n, cnt, st in [(1, 1, 5), (7, 3, 9), (100, 100, 11), (8192, 512, 13), (10, 0, 1)]:
        r = oracle.init_rows(n, cnt, st)
        assert len(r) == cnt and len(set(r)) == cnt and all(0 <= v < n for v in r)


def test_init_rows_uniform_over_permutations():
    # Fisher-Yates with an unbiased source visits every permutation equally often.
    n = 4
    counts = {p: 0 for p in itertools.permutations(range(n))}
    trials = 24000
    for t in range(trials):
        counts[tuple(oracle.init_rows(n, n, oracle.segment_state(t, 0, 0, 0)))] += 1
    exp = trials / 24
    chi2 = sum((c - exp) ** 2 / exp for c in counts.values())
    assert chi2 < 60.0            # 23 dof; p ~ 4e-5


# ------------------------------------------------------------------ zones and segments
def test_zones_partition_the_context():
    for N, S, W in [(100, 4, 10), (10, 4, 10), (14, 4, 10), (15, 4, 10), (1, 0, 0), (5, 0, 3)]:
        st = oracle.steady_positions(N, S, W)
        lo, hi = oracle.clustered_range(N, S, W)
        allpos = np.concatenate([st, np.arange(lo, hi)])
        assert sorted(allpos.tolist()) == list(range(N))


def test_segment_bounds():
    assert oracle.segment_bounds(0, 8) == []
    assert oracle.segment_bounds(20, 8) == [(0, 8), (8, 16), (16, 20)]
    assert oracle.segment_bounds(20, 0) == [(0, 20)]
    assert len(oracle.segment_bounds(131004, 8192)) == 16


# ------------------------------------------------------------------ spherical k-means
def _blob_segment(n, d, blobs, rng, noise):
    cen = rng.standard_normal((blobs, d))
    lab = rng.integers(0, blobs, n)
    K = cen[lab] + noise * rng.standard_normal((n, d))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    return K, lab


def test_kmeans_zero_noise_recovers_blobs():
    rng = np.random.default_rng(5)
    n, d, Cs = 300, 32, 12
    state = oracle.segment_state(77, 0, 0, 0)
    init = oracle.init_rows(n, Cs, state)
    lab = rng.integers(0, Cs, n)
    lab[init] = np.arange(Cs)                    # seeded init picks one token of every blob
    cen = rng.standard_normal((Cs, d))
    cen /= np.linalg.norm(cen, axis=1, keepdims=True)
    for dt in ("bf16", "f32"):
        K = oracle.round_to_dtype(cen, dt)[lab]  # every token is exactly its blob's direction
        assign, sums, counts = oracle.spherical_kmeans_segment(K, Cs, 3, dt, state)
        np.testing.assert_array_equal(assign, lab)
        np.testing.assert_array_equal(counts, np.bincount(lab, minlength=Cs))
        np.testing.assert_array_equal(sums / counts[:, None], oracle.round_to_dtype(cen, dt))


def test_kmeans_assignment_is_exact_argmax_with_lower_id_ties():
    # brute force with exact rationals: every assignment made in every iteration picks a
    # centroid of maximal exact score, the lowest id among equals; duplicated keys force ties.
    rng = np.random.default_rng(6)
    K, _ = _blob_segment(40, 8, 3, rng, 0.4)
    K = oracle.round_to_dtype(K, "bf16")
    init = oracle.init_rows(40, 6, 1234)
    K[init[1]] = K[init[0]]                    # two seed rows equal -> duplicated centroids
    K[init[4]] = K[init[0]]
    assign, _, _, hist = oracle.spherical_kmeans_segment(K, 6, 4, "bf16", 1234, history=True)
    assert np.array_equal(hist[0][1][0], hist[0][1][1])
    for a, mh in hist:
        cs_eff = 6
        for i in range(K.shape[0]):
            sc = [_exact_dot(K[i], mh[c]) for c in range(cs_eff)]
            best = max(sc)
            assert a[i] == min(c for c in range(cs_eff) if sc[c] == best)


def test_kmeans_objective_non_decreasing_f32():
    rng = np.random.default_rng(7)
    K, _ = _blob_segment(400, 16, 10, rng, 0.5)
    K = oracle.round_to_dtype(K, "f32")
    _, _, _, hist = oracle.spherical_kmeans_segment(K, 10, 8, "f32", 99, history=True)
    J = []
    for a, mh in hist:
        J.append(sum(float(K[i] @ mh[a[i]]) for i in range(K.shape[0])))
    for t in range(1, len(J)):
        assert J[t] >= J[t - 1] - 1e-5


def test_kmeans_update_is_normalised_member_sum():
    # after the update the next assignment's centroids are unit vectors along the member sums
    rng = np.random.default_rng(8)
    K, _ = _blob_segment(200, 16, 5, rng, 0.3)
    K = oracle.round_to_dtype(K, "f32")
    _, _, _, hist = oracle.spherical_kmeans_segment(K, 5, 3, "f32", 3, history=True)
    (a0, _), (_, m1) = hist[0], hist[1]
    for j in range(5):
        mem = K[a0 == j]
        if len(mem):
            s = mem.sum(axis=0)
            np.testing.assert_allclose(m1[j], s / np.linalg.norm(s), rtol=0, atol=1e-6)


def test_kmeans_short_segment_leaves_extra_clusters_empty():
    rng = np.random.default_rng(9)
    K, _ = _blob_segment(5, 8, 2, rng, 0.3)
    assign, sums, counts = oracle.spherical_kmeans_segment(K, 8, 2, "f32", 1)
    assert counts[5:].sum() == 0 and counts.sum() == 5 and assign.max() < 5


# ------------------------------------------------------------------ index finalize + build
def _small_workload(**kw):
    w = synth.Workload("t", 1, 4, 2, 128, 600, "bf16", 16, 4, 20, 256, 16, 4, 5)
    return w.replace(**kw)


def _inputs(w, seed=0):
    K, V, Q = synth.make_instance(w, seed)
    return (synth.as_float64(synth.cast(K, w.dtype)), synth.as_float64(synth.cast(V, w.dtype)),
            synth.as_float64(synth.cast(Q, w.dtype)))


def test_csr_invariants():
    w = _small_workload()
    K, V, Q = _inputs(w)
    idx = oracle.build_index(K, V, w.sink, w.window, w.seg_len, w.clusters_per_seg, w.iters,
                             11, w.dtype)
    lo, hi = oracle.clustered_range(w.N, w.sink, w.window)
    assert idx.C == 3 * w.clusters_per_seg and idx.Nc == hi - lo
    for b in range(w.B):
        for g in range(w.Hkv):
            sz, off, perm = idx.sizes[b, g], idx.offsets[b, g], idx.perm[b, g]
            assert sz.sum() == idx.Nc and off[0] == 0
            np.testing.assert_array_equal(np.diff(off), sz)
            assert sorted(perm.tolist()) == list(range(lo, hi))
            for c in range(idx.C):
                run = perm[off[c]:off[c + 1]]
                assert np.all(np.diff(run) > 0)
                seg = (run - lo) // w.seg_len
                assert np.all(seg == c // w.clusters_per_seg)
                np.testing.assert_array_equal(idx.k_perm[b, g, off[c]:off[c + 1]], K[b, g, run])
                if sz[c]:
                    vs = oracle.round_to_dtype(V[b, g, run].sum(axis=0), "f32")
                    np.testing.assert_allclose(idx.value_sums[b, g, c], vs, rtol=1e-2, atol=1e-2)
                    mu = K[b, g, run].mean(axis=0)
                    np.testing.assert_allclose(idx.centroids[b, g, c], mu, rtol=1e-2, atol=4e-3)
                else:
                    assert not idx.centroids[b, g, c].any() and not idx.value_sums[b, g, c].any()
            st = oracle.steady_positions(w.N, w.sink, w.window)
            np.testing.assert_array_equal(idx.k_steady[b, g], K[b, g, st])


def _one_cluster_index(K_rows, V_rows, dtype):
    """finalize_index over a context of len(K_rows) clustered tokens (no steady zone), all in
    cluster 0 of 2 (cluster 1 stays empty)."""
    n = len(K_rows)
    K = np.zeros((1, 1, n, 128))
    V = np.zeros((1, 1, n, 128))
    K[0, 0] = np.asarray(K_rows)[:, None]
    V[0, 0] = np.asarray(V_rows)[:, None]
    return oracle.finalize_index(K, V, np.zeros((1, 1, n), dtype=np.int64), 0, 0, 2, dtype)


def test_finalize_sums_members_in_ascending_position_order_f32():
    # members at positions 0..3 holding 2^60, 1, -2^60, 1 (all exact in float32).  Left to right in
    # float64: 2^60 + 1 rounds to 2^60, minus 2^60 gives 0, plus 1 gives 1.  Other orders give
    # other values: pairwise (2^60 + 1) + (-2^60 + 1) = 0, right to left 0, exact 2.  So the value
    # sum must be exactly 1 and the mean key exactly 1/4.
    big = 2.0 ** 60
    idx = _one_cluster_index([big, 1.0, -big, 1.0], [big, 1.0, -big, 1.0], "f32")
    assert idx.sizes[0, 0, 0] == 4 and idx.sizes[0, 0, 1] == 0
    assert np.all(idx.value_sums[0, 0, 0] == 1.0)
    assert np.all(idx.centroids[0, 0, 0] == 0.25)
    assert not idx.value_sums[0, 0, 1].any() and not idx.centroids[0, 0, 1].any()


def test_finalize_rounds_float64_to_float32_to_bfloat16_in_two_steps():
    # bf16 storage of x = 1 + 2^-8 + 2^-30: x is just above the midpoint of the bf16 neighbours 1
    # and 1 + 2^-7, so rounding it directly would give 1 + 2^-7; rounded to float32 first it becomes
    # exactly the midpoint 1 + 2^-8 (2^-30 is below half a float32 ulp), which then rounds to the
    # even neighbour 1.  Value sum: members 1, 2^-8, 2^-30; mean key: members 4, 2^-6, 2^-28, 0
    # (sum 4 x, so the mean is x).  Every member is exact in bf16 and the float64 sums are exact.
    idx = _one_cluster_index([4.0, 2.0 ** -6, 2.0 ** -28, 0.0], [1.0, 2.0 ** -8, 2.0 ** -30, 0.0], "bf16")
    assert np.all(idx.value_sums[0, 0, 0] == 1.0)
    assert np.all(idx.centroids[0, 0, 0] == 1.0)
    # a float32-exact value past the midpoint rounds up, as plain round-to-nearest does
    idx = _one_cluster_index([4.0, 2.0 ** -6, 2.0 ** -20, 0.0], [1.0, 2.0 ** -8, 2.0 ** -22, 0.0], "bf16")
    assert np.all(idx.value_sums[0, 0, 0] == 1.0 + 2.0 ** -7)
    assert np.all(idx.centroids[0, 0, 0] == 1.0 + 2.0 ** -7)


def test_segments_are_independent_and_single_segment_matches_unsegmented():
    w = _small_workload(B=1, Hkv=1, Hq=1, N=300, seg_len=100, clusters_per_seg=6)
    K, V, _ = _inputs(w)
    _, lab_a = oracle.build_index(K, V, w.sink, w.window, 100, 6, 4, 5, "bf16", True)
    K2 = K.copy()
    K2[0, 0, w.sink + 150] = K2[0, 0, w.sink + 160]   # change a key of segment 1 only
    _, lab_b = oracle.build_index(K2, V, w.sink, w.window, 100, 6, 4, 5, "bf16", True)
    np.testing.assert_array_equal(lab_a[..., :100], lab_b[..., :100])
    Nc = idx_nc = w.N - w.sink - w.window
    _, lab_c = oracle.build_index(K, V, w.sink, w.window, 0, 6, 4, 5, "bf16", True)
    _, lab_d = oracle.build_index(K, V, w.sink, w.window, Nc + 50, 6, 4, 5, "bf16", True)
    np.testing.assert_array_equal(lab_c, lab_d)
    assert idx_nc == Nc


# ------------------------------------------------------------------ decode
def _dense(q, K, V, scale):
    qt = torch.from_numpy(q)[None, None, None, :]
    Kt = torch.from_numpy(K)[None, None]
    Vt = torch.from_numpy(V)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)[0, 0, 0]
    lse = torch.logsumexp((Kt[0, 0] @ qt[0, 0, 0]) * scale, dim=0)
    return o.numpy(), float(lse)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_all_clusters_retrieved_equals_dense_attention(dtype):
    w = _small_workload(dtype=dtype)
    K, V, Q = _inputs(w)
    idx = oracle.build_index(K, V, w.sink, w.window, w.seg_len, w.clusters_per_seg, w.iters,
                             3, dtype)
    scale = 1 / math.sqrt(w.d)
    o, lse, sel = oracle.decode(Q, idx, w.Hq, idx.C + 5, scale)
    G = w.Hq // w.Hkv
    for b in range(w.B):
        for h in range(w.Hq):
            ro, rl = _dense(Q[b, h], K[b, h // G], V[b, h // G], scale)
            np.testing.assert_allclose(o[b, h], ro, rtol=0, atol=1e-13)
            assert abs(lse[b, h] - rl) < 1e-12
            ne = np.nonzero(idx.sizes[b, h // G])[0]
            np.testing.assert_array_equal(sel[b, h, :ne.size], ne)
            assert np.all(sel[b, h, ne.size:] == -1)


def test_estimate_is_exact_when_member_keys_equal_centroid():
    # f32 storage and values on a 2^-10 grid keep every stored value sum exact, so the only
    # approximation left is the one the estimation zone makes, which vanishes here.
    w = _small_workload(B=1, Hkv=2, Hq=4, dtype="f32")
    K, V, Q = _inputs(w)
    V = np.round(V * 1024) / 1024
    idx, lab = oracle.build_index(K, V, w.sink, w.window, w.seg_len, w.clusters_per_seg,
                                  w.iters, 4, "f32", return_labels=True)
    lo, hi = oracle.clustered_range(w.N, w.sink, w.window)
    Kc = K.copy()
    for b in range(w.B):
        for g in range(w.Hkv):
            for c in range(idx.C):
                mem = lo + np.nonzero(lab[b, g] == c)[0]
                if mem.size:
                    Kc[b, g, mem] = idx.centroids[b, g, c]
    idx2 = oracle.finalize_index(Kc, V, lab, w.sink, w.window, idx.C, "f32")
    np.testing.assert_array_equal(idx2.centroids, idx.centroids)
    scale = 1 / math.sqrt(w.d)
    G = w.Hq // w.Hkv
    for k in (0, 3):
        o, lse, _ = oracle.decode(Q, idx2, w.Hq, k, scale)
        for h in range(w.Hq):
            ro, rl = _dense(Q[0, h], Kc[0, h // G], V[0, h // G], scale)
            np.testing.assert_allclose(o[0, h], ro, rtol=0, atol=1e-12)
            assert abs(lse[0, h] - rl) < 1e-12


def test_one_token_per_cluster_makes_estimate_exact_for_any_k():
    w = _small_workload(B=1, Hkv=1, Hq=2, N=200, seg_len=0, dtype="f32")
    K, V, Q = _inputs(w)
    lo, hi = oracle.clustered_range(w.N, w.sink, w.window)
    Nc = hi - lo
    idx = oracle.build_index(K, V, w.sink, w.window, 0, Nc, 2, 8, "f32")
    assert np.all(idx.sizes == 1)
    scale = 1 / math.sqrt(w.d)
    for k in (0, 1, 7, Nc):
        o, lse, _ = oracle.decode(Q, idx, w.Hq, k, scale)
        for h in range(w.Hq):
            ro, rl = _dense(Q[0, h], K[0, 0], V[0, 0], scale)
            np.testing.assert_allclose(o[0, h], ro, rtol=0, atol=1e-12)
            assert abs(lse[0, h] - rl) < 1e-12


def test_topk_matches_brute_force_with_forced_ties():
    rng = np.random.default_rng(10)
    d, C = 8, 24
    mu = oracle.round_to_dtype(rng.standard_normal((C, d)), "bf16")
    mu[5] = mu[2]
    mu[17] = mu[2]
    mu[9] = mu[11]
    sizes = rng.integers(0, 4, C)
    sizes[[2, 5, 17, 9, 11]] = 1
    q = oracle.round_to_dtype(rng.standard_normal(d), "bf16")
    off = np.concatenate([[0], np.cumsum(sizes)])
    Nc = int(off[-1])
    idx = oracle.Index(
        centroids=mu[None, None], value_sums=np.zeros((1, 1, C, d)), sizes=sizes[None, None],
        offsets=off[None, None], perm=np.arange(Nc)[None, None],
        k_perm=np.zeros((1, 1, Nc, d)), v_perm=np.zeros((1, 1, Nc, d)),
        k_steady=np.zeros((1, 1, 0, d)), v_steady=np.zeros((1, 1, 0, d)), C=C, Nc=Nc)
    exact = [_exact_dot(q, mu[c]) for c in range(C)]
    for k in range(0, C + 2):
        _, _, sel = oracle.decode(q[None, None], idx, 1, k, 1.0)
        ranked = sorted([c for c in range(C) if sizes[c] > 0], key=lambda c: (-exact[c], c))
        want = sorted(ranked[:k])
        got = [int(c) for c in sel[0, 0] if c >= 0]
        assert got == want


def test_steady_only_context_is_dense():
    w = _small_workload(N=20, sink=4, window=20)
    K, V, Q = _inputs(w)
    idx = oracle.build_index(K, V, w.sink, w.window, 8, 4, 3, 1, "bf16")
    assert idx.C == 0 and idx.Nc == 0
    o, lse, sel = oracle.decode(Q, idx, w.Hq, 5)
    G = w.Hq // w.Hkv
    for h in range(w.Hq):
        ro, rl = _dense(Q[0, h], K[0, h // G], V[0, h // G], 1 / math.sqrt(w.d))
        np.testing.assert_allclose(o[0, h], ro, atol=1e-13, rtol=0)
    assert np.all(sel == -1)


def test_nan_query_propagates():
    w = _small_workload(B=1, Hq=2, Hkv=1)
    K, V, Q = _inputs(w)
    idx = oracle.build_index(K, V, w.sink, w.window, w.seg_len, 8, 2, 1, "bf16")
    Q[0, 1, 3] = np.nan
    o, lse, _ = oracle.decode(Q, idx, w.Hq, 2)
    assert np.isnan(o[0, 1]).all() and np.isnan(lse[0, 1])
    assert np.isfinite(o[0, 0]).all()


# ------------------------------------------------------------------ generator
def test_generator_is_seeded_and_shaped():
    w = _small_workload()
    K, V, Q = synth.make_instance(w, 5)
    K2, _, Q2 = synth.make_instance(w, 5)
    assert K.shape == (w.B, w.Hkv, w.N, w.d) and Q.shape == (w.B, w.Hq, w.d)
    np.testing.assert_array_equal(K, K2)
    np.testing.assert_array_equal(Q, Q2)
    np.testing.assert_allclose(np.linalg.norm(K, axis=-1), 1.0, rtol=1e-12)
    K3, _, _ = synth.make_instance(w, 6)
    assert not np.array_equal(K, K3)


# ------------------------------------------------------------------ selection reuse (FreeKV)
def _gated_setup(seed=0):
    w = _small_workload()
    K, V, Q = _inputs(w, seed)
    idx = oracle.build_index(K, V, w.sink, w.window, w.seg_len, w.clusters_per_seg, w.iters, 3, "bf16")
    return w, K, V, Q, idx


def test_query_cosine_closed_forms():
    # cos(q, q) = 1 up to the rounding of sqrt(a) * sqrt(a) (within 1e-15); 2q and -q scale
    # every product exactly; a zero query gives 0; e3 against e3 + e7 is 1/sqrt(2)
    rng = np.random.default_rng(1)
    q = oracle.round_to_dtype(rng.standard_normal(128), "bf16")
    assert abs(oracle.query_cosine(q, q) - 1.0) <= 1e-15
    assert abs(oracle.query_cosine(q, 2 * q) - 1.0) <= 1e-15
    assert abs(oracle.query_cosine(q, -q) + 1.0) <= 1e-15
    assert oracle.query_cosine(q, np.zeros(128)) == 0.0
    e = np.zeros(128)
    e[3] = 1.0
    f = np.zeros(128)
    f[3], f[7] = 1.0, 1.0
    assert abs(oracle.query_cosine(e, f) - 1 / math.sqrt(2)) <= 1e-16


def test_gated_threshold_above_one_never_reuses():
    w, K, V, Q, idx = _gated_setup()
    o, lse, sel = oracle.decode(Q, idx, w.Hq, w.top_k)
    junk = np.zeros_like(sel)                     # cluster 0 only, never the real selection
    go, gl, gs, reused = oracle.decode_gated(Q, Q, junk, idx, w.Hq, w.top_k, 1.5)
    assert not reused.any()
    np.testing.assert_array_equal(gs, sel)
    np.testing.assert_array_equal(go, o)
    np.testing.assert_array_equal(gl, lse)


def test_gated_reusing_own_selection_equals_decode():
    w, K, V, Q, idx = _gated_setup(1)
    o, lse, sel = oracle.decode(Q, idx, w.Hq, w.top_k)
    go, gl, gs, reused = oracle.decode_gated(Q, Q, sel, idx, w.Hq, w.top_k, 0.999)
    assert reused.all()
    np.testing.assert_array_equal(gs, sel)
    np.testing.assert_allclose(go, o, rtol=0, atol=0)
    np.testing.assert_array_equal(gl, lse)


def test_gated_reusing_every_cluster_is_dense_attention():
    w, K, V, Q, idx = _gated_setup(2)
    G = w.Hq // w.Hkv
    allc = np.full((w.B, w.Hq, idx.C), -1, dtype=np.int64)
    for b in range(w.B):
        for h in range(w.Hq):
            ne = np.nonzero(idx.sizes[b, h // G])[0]
            allc[b, h, :ne.size] = ne
    go, gl, gs, reused = oracle.decode_gated(Q, Q, allc, idx, w.Hq, idx.C, -2.0)
    assert reused.all()
    scale = 1 / math.sqrt(w.d)
    for b in range(w.B):
        for h in range(w.Hq):
            ro, rl = _dense(Q[b, h], K[b, h // G], V[b, h // G], scale)
            np.testing.assert_allclose(go[b, h], ro, rtol=0, atol=1e-13)
            assert abs(gl[b, h] - rl) < 1e-12


def test_gated_one_drifting_head_reselects_its_whole_group():
    w, K, V, Q, idx = _gated_setup(3)
    G = w.Hq // w.Hkv
    o, lse, sel = oracle.decode(Q, idx, w.Hq, w.top_k)
    junk = np.full_like(sel, -1)
    junk[..., 0] = 0                              # a stale one-cluster selection
    Qp = Q.copy()
    Qp[0, G] = -Q[0, G]                           # head G (first head of KV group 1) turns around
    go, gl, gs, reused = oracle.decode_gated(Q, Qp, junk, idx, w.Hq, w.top_k, 0.5)
    assert reused[0, 0] and not reused[0, 1]
    # group 0 takes the stale zone, group 1 selects afresh for every one of its heads
    for h in range(G):
        assert list(gs[0, h][gs[0, h] >= 0]) == [0]
    np.testing.assert_array_equal(gs[0, G:2 * G], sel[0, G:2 * G])
    np.testing.assert_array_equal(go[0, G:2 * G], o[0, G:2 * G])


def test_gated_refresh_postpones_rather_than_skips_the_selection():
    # with refresh, every head's sel is the current query's own top-k (what the next step keeps),
    # while the outputs still come from the kept stale zones
    w, K, V, Q, idx = _gated_setup(4)
    G = w.Hq // w.Hkv
    o, lse, sel = oracle.decode(Q, idx, w.Hq, w.top_k)
    junk = np.full_like(sel, -1)
    junk[..., 0] = 0
    Qp = Q.copy()
    Qp[0, G] = -Q[0, G]
    go, gl, gs, reused = oracle.decode_gated(Q, Qp, junk, idx, w.Hq, w.top_k, 0.5)
    fo, fl, fs, freused = oracle.decode_gated(Q, Qp, junk, idx, w.Hq, w.top_k, 0.5, refresh=True)
    np.testing.assert_array_equal(freused, reused)
    np.testing.assert_array_equal(fo, go)
    np.testing.assert_array_equal(fl, gl)
    np.testing.assert_array_equal(fs, sel)
    assert not np.array_equal(gs, sel)


# ------------------------------------------------------------------ accuracy-bounded estimation
def _bounded_setup(seed=0, dtype="bf16", q_scale=1.5, key_noise=0.3):
    w = _small_workload(dtype=dtype, q_scale=q_scale, key_noise=key_noise)
    K, V, Q = _inputs(w, seed)
    idx = oracle.build_index(K, V, w.sink, w.window, w.seg_len, w.clusters_per_seg, w.iters, 3, dtype)
    return w, K, V, Q, idx, oracle.bound_data(idx)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bound_data_matches_a_brute_force_norm(dtype):
    # radius and value norms from numpy's own norm (another summation): within one float32 ulp,
    # and never below the exact distance
    w, K, V, Q, idx, bd = _bounded_setup(1, dtype)
    for g in range(w.Hkv):
        off = idx.offsets[0, g]
        for c in np.nonzero(idx.sizes[0, g])[0]:
            kr = idx.k_perm[0, g, off[c]:off[c + 1]]
            r = np.linalg.norm(kr - idx.centroids[0, g, c], axis=1).max()
            vn = np.linalg.norm(idx.v_perm[0, g, off[c]:off[c + 1]], axis=1).max()
            for got, ref in ((bd.radius[0, g, c], r), (bd.vnorm[0, g, c], vn)):
                assert got >= ref * (1 - 1e-15)
                assert got <= np.nextafter(np.float32(ref), np.float32(np.inf)) * (1 + 1e-7)
        allv = np.concatenate([idx.v_perm[0, g], idx.v_steady[0, g]])
        vm = np.linalg.norm(allv, axis=1).max()
        assert vm * (1 - 1e-15) <= bd.vmax[0, g] <= np.nextafter(np.float32(vm), np.float32(np.inf)) * (1 + 1e-7)
        assert bd.vmax[0, g] >= bd.vnorm[0, g].max()
        assert (bd.radius[0, g][idx.sizes[0, g] == 0] == 0).all()


def test_cluster_of_identical_keys_has_radius_zero():
    rng = np.random.default_rng(2)
    d, C = 128, 4
    u = oracle.round_to_dtype(rng.standard_normal(d) / math.sqrt(d), "bf16")
    K = oracle.round_to_dtype(rng.standard_normal((1, 1, 12, d)) / math.sqrt(d), "bf16")
    V = oracle.round_to_dtype(rng.standard_normal((1, 1, 12, d)), "bf16")
    labels = np.array([[[0, 1, 0, 2, 0, 3, 0, 1]]])
    K[0, 0, 2:10][labels[0, 0] == 0] = u          # clustered positions 2..9 (sink 2, window 2)
    idx = oracle.finalize_index(K, V, labels, 2, 2, C, "bf16")
    bd = oracle.bound_data(idx)
    # cluster 0: four copies of u; 1: two different keys; 2 and 3: one key each (its own mean)
    assert bd.radius[0, 0, 0] == 0.0 and bd.radius[0, 0, 1] > 0
    assert bd.radius[0, 0, 2] == 0.0 and bd.radius[0, 0, 3] == 0.0
    _, _, _, w_, a_, err, _ = oracle.bound_terms(rng.standard_normal(d), idx, bd, 0, 0, 1 / math.sqrt(d), "bf16")
    assert a_[0] == 0.0 and err[0] == w_[0] * oracle.sum_roundoff("bf16") * bd.vnorm[0, 0, 0]


@pytest.mark.parametrize("seed,dtype,q_scale,key_noise", [(3, "bf16", 1.5, 0.3), (4, "f32", 1.5, 0.3),
                                                          (5, "bf16", 6.0, 0.1), (6, "bf16", 1.0, 1.0)])
@pytest.mark.parametrize("eps", [0.02, 0.3, 3.0])
def test_bounded_decode_error_is_within_its_bound(seed, dtype, q_scale, key_noise, eps):
    # the derived bound against dense softmax attention over the same stored keys and values
    w, K, V, Q, idx, bd = _bounded_setup(seed, dtype, q_scale, key_noise)
    k_max = idx.C
    o, lse, sel, ks, prior, post = oracle.decode_bounded(Q, idx, bd, w.Hq, k_max, eps, dtype)
    G = w.Hq // w.Hkv
    scale = 1 / math.sqrt(w.d)
    for h in range(w.Hq):
        ro, _ = _dense(Q[0, h], K[0, h // G], V[0, h // G], scale)
        err = float(np.linalg.norm(o[0, h] - ro))
        assert err <= post[0, h] * (1 + 1e-9) + 1e-12, (h, err, post[0, h])
        assert post[0, h] <= prior[0, h] * (1 + 1e-12) + 1e-300
        assert prior[0, h] <= eps                   # k_max covers every cluster: never capped


def test_bounded_zone_is_the_smallest_that_meets_eps():
    w, K, V, Q, idx, bd = _bounded_setup(7)
    G = w.Hq // w.Hkv
    scale = 1 / math.sqrt(w.d)
    for eps in (0.0, 0.05, 0.5, 5.0, np.inf):
        o, lse, sel, ks, prior, post = oracle.decode_bounded(Q, idx, bd, w.Hq, idx.C, eps, "bf16")
        for h in range(w.Hq):
            sigma, order, mstar, w_, a_, err, lo = oracle.bound_terms(Q[0, h], idx, bd, 0, h // G, scale, "bf16")
            A = oracle.prior_bounds(err, lo, order)
            assert (np.diff(A) <= 0).all()
            k = ks[0, h]
            assert A[k] <= eps and (k == 0 or A[k - 1] > eps)
            assert list(sel[0, h][:k]) == sorted(order[:k]) and (sel[0, h][k:] == -1).all()
        if eps == 0.0:                              # everything retrieved: dense, bound 0
            assert (ks == (idx.sizes[0] > 0).sum(axis=1).repeat(G)[None]).all() and (post == 0).all()
        if eps == np.inf:
            assert (ks == 0).all()


def test_bounded_zone_is_capped_by_top_k_and_forced_k_reproduces_decode():
    w, K, V, Q, idx, bd = _bounded_setup(8)
    o, lse, sel, ks, prior, post = oracle.decode_bounded(Q, idx, bd, w.Hq, 3, 0.0, "bf16")
    assert (ks == 3).all() and (prior > 0).all()
    ro, rl, rs = oracle.decode(Q, idx, w.Hq, 3)
    np.testing.assert_array_equal(sel, rs)
    np.testing.assert_array_equal(o, ro)
    kf = np.array([[0, 1, 2, 5]])
    o2, _, sel2, ks2, _, _ = oracle.decode_bounded(Q, idx, bd, w.Hq, 5, 0.0, "bf16", k_force=kf)
    np.testing.assert_array_equal(ks2, kf)
    for h in range(w.Hq):
        ro, rl, rs = oracle.decode(Q, idx, w.Hq, int(kf[0, h]))
        np.testing.assert_array_equal(o2[0, h], ro[0, h])
        np.testing.assert_array_equal(sel2[0, h][:kf[0, h]], rs[0, h])


def test_bound_is_nearly_attained_by_two_opposite_members():
    # one cluster {mu + r e0, mu - r e0} with values +e2 and -e2 (their sum is 0), two steady
    # tokens with zero key and zero value, q = t e0: the cluster's estimate contributes nothing to
    # the numerator while the exact attention leans towards +e2.  Exact error (in closed form)
    # sinh-like / (2 + 2 cosh x), the bound 2 (e^x - 1 + u) / (2 + 2 e^-x); the ratio is about
    # 0.64 at x = 0.44, so a bound off by a factor of 2 either way fails
    d = 128
    s = 1 / math.sqrt(d)
    K = np.zeros((1, 1, 4, d))
    V = np.zeros((1, 1, 4, d))
    K[0, 0, 1, 1], K[0, 0, 1, 0] = 0.5, 0.25
    K[0, 0, 2, 1], K[0, 0, 2, 0] = 0.5, -0.25
    V[0, 0, 1, 2], V[0, 0, 2, 2] = 1.0, -1.0
    idx = oracle.finalize_index(K, V, np.zeros((1, 1, 2), dtype=np.int64), 1, 1, 1, "bf16")
    bd = oracle.bound_data(idx)
    assert bd.radius[0, 0, 0] == 0.25 and bd.vnorm[0, 0, 0] == 1.0 and bd.vmax[0, 0] == 1.0
    q = np.zeros(d)
    q[0] = 20.0
    o, lse, sel, ks, prior, post = oracle.decode_bounded(q[None, None], idx, bd, 1, 1, np.inf, "bf16")
    assert ks[0, 0] == 0 and np.abs(o).max() == 0.0
    x = s * 20.0 * 0.25
    exact = (math.exp(x) - math.exp(-x)) / (2 + math.exp(x) + math.exp(-x))
    ro, _ = _dense(q, K[0, 0], V[0, 0], s)
    assert abs(np.linalg.norm(ro) - exact) < 1e-12
    bound = 2 * (math.expm1(x) + oracle.sum_roundoff("bf16")) / (2 + 2 * math.exp(-x))
    assert abs(post[0, 0] - bound) < 1e-12
    assert 0.5 * post[0, 0] < exact <= post[0, 0]
