"""GPU parity of the accuracy-bounded estimation: wi_bound_data (per-cluster radius and value
norms, bit-exact against oracle.bound_data) and wi_decode_bounded (the zone of each head sized
to meet an error bound).

The device decides each head's zone size on fp32 terms when rigorous bounds on their rounding
certify the decision, and otherwise recomputes the terms in fp64 from canonical scores; either
way the size must equal the oracle's decision (smallest k with A(k) <= eps, A on canonical fp64
scores, with the scale and eps the device received: both cross the boundary as fp32).  Only a
head with some A(j) within 1e-9 of eps (relative), which fp64 rounding may decide either way, is
held to validity instead.  Given that k, the zone (bit-exact ids), the outputs (the decode
tolerances) and the bound after attention (relative 1e-3) are compared with the oracle run at
the same k.  Cases with eps just beside an A(j), and clusters with identical centroids, drive
the fp64 decision and the canonical re-ranking of ties at the zone boundary.
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

D = 128
K_TOL = 1e-9                      # relative distance of eps to an A(j) that fp64 may decide either way
SCALE32 = float(np.float32(1 / math.sqrt(D)))     # the scale the device receives


def _f32(x: float) -> float:
    return float(np.float32(x))


def _decision(A, cap, eps):
    """The oracle's zone size: the smallest k in [0, cap] with A(k) <= eps, else cap."""
    ok = np.nonzero(A[:cap + 1] <= eps)[0]
    return int(ok[0]) if ok.size else cap


def _ambiguous(A, cap, eps):
    a = A[:cap + 1]
    return bool(np.isfinite(eps) and eps > 0 and (np.abs(a - eps) <= K_TOL * eps).any())


def _check_k(A, cap, eps, k, where):
    """k equals the oracle's decision; a head whose A(j) comes within fp64 rounding of eps only
    needs a valid k (A(k) <= eps, A(k - 1) > eps, each within that rounding)."""
    assert 0 <= k <= cap, (where, k, cap)
    if not _ambiguous(A, cap, eps):
        assert k == _decision(A, cap, eps), (where, k, _decision(A, cap, eps), eps)
    else:
        if k < cap:
            assert A[k] <= eps * (1 + K_TOL), (where, k, A[k], eps)
        if k > 0:
            assert A[k - 1] > eps * (1 - K_TOL), (where, k, A[k - 1], eps)


def _workload_index(dtype, seed, N=2048, Hq=8, Hkv=2, seg_len=512, cps=32, key_noise=0.3, q_scale=1.5):
    w = synth.Workload("b", 1, Hq, Hkv, D, N, dtype, 24, 4, 32, seg_len, cps, 4, 16,
                       key_noise=key_noise, q_scale=q_scale)
    K, V, Q = synth.make_instance(w, seed)
    dev = device()
    Kt, Vt, Qt = (synth.cast(x, dtype, dev) for x in (K, V, Q))
    K64, V64, Q64 = (synth.as_float64(t) for t in (Kt, Vt, Qt))
    idx = oracle.build_index(K64, V64, w.sink, w.window, seg_len, cps, w.iters, 5, dtype)
    return w, idx, Qt, Q64


def _random_label_index(dtype, seed, C=1024, tpc=2, Hkv=2, empty_frac=0.3):
    rng = np.random.default_rng(seed)
    Nc = C * tpc
    N = Nc + 4 + 16
    K = rng.standard_normal((1, Hkv, N, D))
    K /= np.linalg.norm(K, axis=-1, keepdims=True)
    V = rng.standard_normal((1, Hkv, N, D))
    labels = np.empty((1, Hkv, Nc), dtype=np.int64)
    for g in range(Hkv):
        live = np.nonzero(rng.random(C) >= empty_frac)[0]
        lab = np.concatenate([live, rng.choice(live, Nc - live.size)])
        rng.shuffle(lab)
        labels[0, g] = lab
    dev = device()
    Kt, Vt = (synth.cast(x, dtype, dev) for x in (K, V))
    K64, V64 = (synth.as_float64(t) for t in (Kt, Vt))
    return oracle.finalize_index(K64, V64, labels, 4, 16, C, dtype)


def _bound_on_device(gi, idx, dtype):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    radius, vnorm, vmax = wi.bound_data(gi, idx.sizes.shape[0], idx.sizes.shape[1], tdt)
    torch.cuda.synchronize()
    return radius, vnorm, vmax


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bound_data_bit_exact(dtype):
    for idx in (_workload_index(dtype, 1)[1], _random_label_index(dtype, 2)):
        gi = upload_index(idx, dtype, device())
        radius, vnorm, vmax = _bound_on_device(gi, idx, dtype)
        ref = oracle.bound_data(idx)
        np.testing.assert_array_equal(radius.cpu().numpy().astype(np.float64), ref.radius)
        np.testing.assert_array_equal(vnorm.cpu().numpy().astype(np.float64), ref.vnorm)
        np.testing.assert_array_equal(vmax.cpu().numpy().astype(np.float64), ref.vmax)


def _check_bounded(idx, Qt, Q64, Hq, top_k, eps, dtype):
    gi = upload_index(idx, dtype, device())
    bound = _bound_on_device(gi, idx, dtype)
    bd = oracle.bound_data(idx)
    n_exact = torch.zeros(1, dtype=torch.int32, device=device())
    o, lse, sel, k_used, err = wi.decode_bounded(gi, Qt, bound, top_k, eps, n_exact=n_exact)
    torch.cuda.synchronize()
    k_dev = k_used.cpu().numpy().astype(np.int64)
    B, G = Q64.shape[0], Hq // idx.sizes.shape[1]
    e32 = _f32(eps)
    for b in range(B):
        for h in range(Hq):
            _, order, _, _, _, errc, lo = oracle.bound_terms(Q64[b, h], idx, bd, b, h // G, SCALE32, dtype)
            A = oracle.prior_bounds(errc, lo, order)
            _check_k(A, min(top_k, order.size), e32, int(k_dev[b, h]), (b, h))
    ro, rl, rs, rk, rprior, rpost = oracle.decode_bounded(Q64, idx, bd, Hq, top_k, eps, dtype, k_force=k_dev)
    assert_decode_parity(o, lse, sel, ro, rl, rs, dtype)
    e = err.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(e, rpost, rtol=2e-3, atol=1e-30)
    return k_dev, e, int(n_exact.item())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bounded_decode_over_a_range_of_eps(dtype):
    w, idx, Qt, Q64 = _workload_index(dtype, 3)
    ks = []
    for eps in (0.0, 0.01, 0.1, 1.0, 10.0, float("inf")):
        k, e, _ = _check_bounded(idx, Qt, Q64, w.Hq, idx.C, eps, dtype)
        ks.append(k)
        assert (e <= eps * (1 + 1e-3) + 1e-30).all() or eps == 0.0
    n_ne = (idx.sizes[0] > 0).sum(axis=1).repeat(w.Hq // w.Hkv)
    assert (ks[0][0] == n_ne).all() and (ks[-1] == 0).all()
    for a, b in zip(ks, ks[1:]):                  # a larger eps never needs a larger zone
        assert (b <= a).all()
    assert len({int(k.sum()) for k in ks}) >= 4  # the sweep really moves the zone


def test_bounded_decode_capped_and_sharp_queries():
    # sharp queries on tight clusters (|q| ~ 70: exp(s |q| r_c) makes the bound demanding); then
    # top_k caps every head
    w, idx, Qt, Q64 = _workload_index("bf16", 4, key_noise=0.1, q_scale=6.0)
    for eps in (0.05, 5.0):
        _check_bounded(idx, Qt, Q64, w.Hq, idx.C, eps, "bf16")
    k, _, _ = _check_bounded(idx, Qt, Q64, w.Hq, 3, 0.0, "bf16")
    assert (k == 3).all()


def test_bounded_decode_with_empty_clusters_and_many_heads():
    idx = _random_label_index("bf16", 5, C=512, tpc=3, Hkv=34)
    rng = np.random.default_rng(5)
    Hq = 272
    Qt = synth.cast(3.0 * rng.standard_normal((1, Hq, D)), "bf16", device())
    Q64 = synth.as_float64(Qt)
    for eps in (0.5, 5.0):
        _check_bounded(idx, Qt, Q64, Hq, 200, eps, "bf16")


def test_bounded_decode_bound_covers_dense_attention():
    # the device's own bound against dense softmax attention over the stored keys and values
    w, idx, Qt, Q64 = _workload_index("bf16", 6)
    gi = upload_index(idx, "bf16", device())
    bound = _bound_on_device(gi, idx, "bf16")
    G = w.Hq // w.Hkv
    K = np.concatenate([idx.k_steady, idx.k_perm], axis=2)
    V = np.concatenate([idx.v_steady, idx.v_perm], axis=2)
    for eps in (0.05, 1.0, float("inf")):
        o, lse, sel, k_used, err = wi.decode_bounded(gi, Qt, bound, idx.C, eps)
        torch.cuda.synchronize()
        o = o.cpu().numpy().astype(np.float64)
        err = err.cpu().numpy().astype(np.float64)
        for h in range(w.Hq):
            lg = (K[0, h // G] @ Q64[0, h]) / math.sqrt(D)
            p = np.exp(lg - lg.max())
            dense = (p @ V[0, h // G]) / p.sum()
            assert np.linalg.norm(o[0, h] - dense) <= err[0, h] * (1 + 1e-3) + 2e-5, (eps, h)


def _slice_group(idx, g):
    f = lambda a: a[:, g:g + 1]
    return oracle.Index(centroids=f(idx.centroids), value_sums=f(idx.value_sums), sizes=f(idx.sizes),
                        offsets=f(idx.offsets), perm=f(idx.perm), k_perm=f(idx.k_perm), v_perm=f(idx.v_perm),
                        k_steady=f(idx.k_steady), v_steady=f(idx.v_steady), C=idx.C, Nc=idx.Nc)


def test_bounded_full_size_sampled_groups():
    """The benchmarked shape (B=1, 32/8 heads, 128K, top 164 of 8192 clusters) on an index the
    oracle finalizes from the generator's blob labels: the bound data of two KV groups bit-exact,
    and the sampled heads' zone sizes equal to the oracle's decisions and their zones, outputs
    and bounds equal to the oracle's at that k."""
    from wi_testutil import inputs
    dev = device()
    w = synth.WORKLOADS["gqa_128k_bf16"]
    Kt, Vt, Qt, K64, V64, Q64, labels = inputs(w, 0, dev, with_labels=True)
    lo, hi = oracle.clustered_range(w.N, w.sink, w.window)
    lab = (np.arange(hi - lo) // w.seg_len) * w.clusters_per_seg + labels[:, :, lo:hi] % w.clusters_per_seg
    C = len(oracle.segment_bounds(hi - lo, w.seg_len)) * w.clusters_per_seg
    idx = oracle.finalize_index(K64, V64, lab, w.sink, w.window, C, w.dtype)
    gi = upload_index(idx, w.dtype, dev)
    bound = _bound_on_device(gi, idx, "bf16")
    G = w.Hq // w.Hkv
    for eps in (40.0, 400.0):
        o, lse, sel, k_used, err = wi.decode_bounded(gi, Qt, bound, w.top_k, eps)
        torch.cuda.synchronize()
        k_dev = k_used.cpu().numpy().astype(np.int64)
        for g in (2, 7):
            sub = _slice_group(idx, g)
            bd = oracle.bound_data(sub)
            if eps == 40.0:
                for got, ref in ((bound[0][:, g:g + 1], bd.radius), (bound[1][:, g:g + 1], bd.vnorm),
                                 (bound[2][:, g:g + 1], bd.vmax)):
                    np.testing.assert_array_equal(got.cpu().numpy().astype(np.float64), ref)
            for h in (g * G, g * G + G - 1):
                _, order, _, _, _, errc, lov = oracle.bound_terms(Q64[0, h], sub, bd, 0, 0, SCALE32, "bf16")
                A = oracle.prior_bounds(errc, lov, order)
                k = int(k_dev[0, h])
                _check_k(A, min(w.top_k, order.size), _f32(eps), k, h)
                ro, rl, rs, _, _, rpost = oracle.decode_bounded(Q64[:, h:h + 1], sub, bd, 1, w.top_k, eps, "bf16",
                                                                k_force=np.array([[k]]))
                assert_decode_parity(o[:, h:h + 1], lse[:, h:h + 1], sel[:, h:h + 1], ro, rl, rs, "bf16")
                np.testing.assert_allclose(float(err[0, h]), rpost[0, 0], rtol=2e-3)
        if eps == 400.0:
            assert (k_dev < w.top_k).any()            # a loose enough bound shrinks some zones


def _twin_index(dtype, seed, pairs=256, tpc=3, Hkv=2):
    """Clusters 2m and 2m + 1 hold copies of the same keys and values: equal centroids, scores,
    sizes, radii and value norms, so that every zone boundary may fall between two clusters that
    tie exactly and only the id decides."""
    rng = np.random.default_rng(seed)
    C = 2 * pairs
    Nc = C * tpc
    N = Nc + 4 + 16
    K = rng.standard_normal((1, Hkv, N, D))
    K /= np.linalg.norm(K, axis=-1, keepdims=True)
    V = rng.standard_normal((1, Hkv, N, D))
    labels = np.empty((1, Hkv, Nc), dtype=np.int64)
    for g in range(Hkv):
        half = np.repeat(np.arange(pairs), tpc)          # tokens of pair m in the first half
        src = 4 + np.arange(Nc // 2)
        K[0, g, 4 + Nc // 2:4 + Nc] = K[0, g, src]
        V[0, g, 4 + Nc // 2:4 + Nc] = V[0, g, src]
        labels[0, g] = np.concatenate([2 * half, 2 * half + 1])
    dev = device()
    Kt, Vt = (synth.cast(x, dtype, dev) for x in (K, V))
    K64, V64 = (synth.as_float64(t) for t in (Kt, Vt))
    return oracle.finalize_index(K64, V64, labels, 4, 16, C, dtype)


def _eps_beside(A, j, rel):
    """An fp32 eps at A(j) (1 + rel), with its side of A(j) kept after the rounding to fp32."""
    e = _f32(A[j] * (1 + rel))
    assert (e > A[j]) == (rel > 0) and e != A[j]
    return e


def test_bounded_decision_with_eps_inside_fp32_rounding():
    # eps a relative 1e-6 above or below some head's A(j): within the fp32 terms' error, so that
    # head can only decide in fp64; every head must still match the oracle
    w, idx, Qt, Q64 = _workload_index("bf16", 3)
    bd = oracle.bound_data(idx)
    G = w.Hq // w.Hkv
    total_exact = 0
    for h, rel in ((0, 1e-6), (3, -1e-6), (5, 1e-6)):
        _, order, _, _, _, errc, lo = oracle.bound_terms(Q64[0, h], idx, bd, 0, h // G, SCALE32, "bf16")
        A = oracle.prior_bounds(errc, lo, order)
        j = int(np.argmin(np.abs(np.log(A[:order.size]) - np.log(0.3))))   # a mid-sized zone
        eps = _eps_beside(A, j, rel)
        k, _, n_exact = _check_bounded(idx, Qt, Q64, w.Hq, idx.C, eps, "bf16")
        assert k[0, h] == _decision(A, order.size, eps)
        total_exact += n_exact
    assert total_exact >= 3                       # those heads decided in fp64


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bounded_decode_ties_at_the_zone_boundary(dtype):
    idx = _twin_index(dtype, 7)
    rng = np.random.default_rng(7)
    Hq = 8
    Qt = synth.cast(2.0 * rng.standard_normal((1, Hq, D)), dtype, device())
    Q64 = synth.as_float64(Qt)
    bd = oracle.bound_data(idx)
    _, order, _, _, _, errc, lo = oracle.bound_terms(Q64[0, 0], idx, bd, 0, 0, SCALE32, dtype)
    A = oracle.prior_bounds(errc, lo, order)
    # zones of odd size end inside a tied pair: eps midway between A(2m) and A(2m + 1)
    for m in (3, 40, 150):
        eps = _f32(math.sqrt(A[2 * m] * A[2 * m + 1]))
        k, _, _ = _check_bounded(idx, Qt, Q64, Hq, idx.C, eps, dtype)
        assert k[0, 0] == 2 * m + 1
    # eps beside a split point, decided in fp64
    k, _, n_exact = _check_bounded(idx, Qt, Q64, Hq, idx.C, _eps_beside(A, 21, 1e-6), dtype)
    assert k[0, 0] == _decision(A, order.size, _eps_beside(A, 21, 1e-6)) and n_exact >= 1
