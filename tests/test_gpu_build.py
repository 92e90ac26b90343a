"""GPU parity of wi_build_index against the CPU oracle: every index buffer bit-exact (sizes,
offsets, perm, cluster-major copies, steady copies, mean keys and value sums), at small sizes for
whole builds and at full size on sampled segments (segments are independent)."""
import math

import numpy as np
import pytest
import torch

import oracle
from kv_vector_index_amd import synth
from kv_vector_index_amd import wave_index as wi
from wi_testutil import assert_decode_parity, device, index_to_numpy, inputs

pytestmark = pytest.mark.gpu

FIELDS = ("sizes", "offsets", "perm", "centroids", "value_sums", "k_perm", "v_perm", "k_steady", "v_steady")


def _assert_index_equal(gpu: dict, ref: oracle.Index):
    for f in FIELDS:
        a, b = gpu[f], getattr(ref, f)
        assert a.shape == b.shape, f
        if a.dtype.kind == "f":
            np.testing.assert_array_equal(a.view(np.uint64), b.view(np.uint64), err_msg=f)
        else:
            np.testing.assert_array_equal(a, b, err_msg=f)


def _build_both(w, seed, build_seed, dev=None):
    dev = dev or device()
    Kt, Vt, Qt, K64, V64, Q64 = inputs(w, seed, dev)
    gi = wi.build_index(Kt, Vt, w.sink, w.window, w.seg_len, w.clusters_per_seg, w.iters, build_seed)
    torch.cuda.synchronize()
    ref = oracle.build_index(K64, V64, w.sink, w.window, w.seg_len, w.clusters_per_seg, w.iters,
                             build_seed, w.dtype)
    return gi, ref, Qt, Q64


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_build_parity_small_ragged(dtype):
    # 3 full segments of 700 plus a last one of 10 tokens (< 40 clusters: 30 stay empty)
    w = synth.Workload("b", 2, 4, 2, 128, 4 + 20 + 3 * 700 + 10, dtype, 30, 4, 20, 700, 40, 4, 5)
    gi, ref, _, _ = _build_both(w, 1, 99)
    _assert_index_equal(index_to_numpy(gi), ref)


def test_build_parity_one_segment_and_many_clusters():
    w = synth.Workload("b", 1, 1, 1, 128, 3000, "bf16", 50, 0, 0, 0, 600, 3, 5)
    gi, ref, _, _ = _build_both(w, 2, 7)
    _assert_index_equal(index_to_numpy(gi), ref)


def test_build_parity_chunked_centroids_f32():
    # 300 clusters per segment: more than one LDS chunk of fp32 centroid directions
    w = synth.Workload("b", 1, 1, 1, 128, 2000, "f32", 40, 0, 0, 0, 300, 3, 5)
    gi, ref, _, _ = _build_both(w, 4, 11)
    _assert_index_equal(index_to_numpy(gi), ref)


def test_build_parity_many_segments_several_passes_per_block():
    # 8 KV heads x 64 segments: more segments than one assignment block each can cover with a
    # single pass, so every block loops over several key passes
    w = synth.Workload("b", 1, 8, 8, 128, 64 * 1100 + 12, "f32", 30, 4, 8, 1100, 20, 2, 5)
    gi, ref, _, _ = _build_both(w, 6, 21)
    _assert_index_equal(index_to_numpy(gi), ref)


def test_build_parity_duplicate_keys_force_ties():
    dev = device()
    w = synth.Workload("b", 1, 2, 1, 128, 1200, "bf16", 8, 2, 2, 400, 24, 4, 3)
    K, V, _ = synth.make_instance(w, 5)
    K[0, 0, 100:400] = K[0, 0, 50]       # a third of segment 0 is one repeated key
    K[0, 0, 600:650] = K[0, 0, 610]
    Kt, Vt = synth.cast(K, "bf16", dev), synth.cast(V, "bf16", dev)
    gi = wi.build_index(Kt, Vt, w.sink, w.window, w.seg_len, w.clusters_per_seg, w.iters, 3)
    torch.cuda.synchronize()
    ref = oracle.build_index(synth.as_float64(Kt), synth.as_float64(Vt), w.sink, w.window,
                             w.seg_len, w.clusters_per_seg, w.iters, 3, "bf16")
    _assert_index_equal(index_to_numpy(gi), ref)


def test_build_steady_only():
    w = synth.Workload("b", 1, 2, 2, 128, 40, "f32", 8, 16, 32, 64, 8, 2, 1)
    gi, ref, _, _ = _build_both(w, 3, 1)
    assert gi.C == 0 and gi.Nc == 0
    _assert_index_equal(index_to_numpy(gi), ref)


def test_build_and_decode_single_head_8k_f32_end_to_end():
    w = synth.WORKLOADS["single_head_8k_f32"]
    gi, ref, Qt, Q64 = _build_both(w, 0, 0)
    _assert_index_equal(index_to_numpy(gi), ref)
    o, lse, sel = wi.decode(gi, Qt, w.top_k)
    torch.cuda.synchronize()
    ro, rl, rs = oracle.decode(Q64, ref, w.Hq, w.top_k, 1 / math.sqrt(w.d))
    assert_decode_parity(o, lse, sel, ro, rl, rs, w.dtype)


@pytest.mark.parametrize("name,segments", [
    ("build_128k_bf16", [(0, 0, 0), (0, 7, 15)]),
    ("gqa_128k_bf16", [(0, 3, 15)]),          # the ragged last segment (8124 tokens)
])
def test_build_full_size_sampled_segments(name, segments):
    dev = device()
    w = synth.WORKLOADS[name]
    Kt, Vt, Qt, K64, V64, Q64 = inputs(w, 0, dev)
    seed = 12345
    gi = wi.build_index(Kt, Vt, w.sink, w.window, w.seg_len, w.clusters_per_seg, w.iters, seed)
    torch.cuda.synchronize()
    g_np = index_to_numpy(gi)
    lo, hi = oracle.clustered_range(w.N, w.sink, w.window)
    segs = oracle.segment_bounds(hi - lo, w.seg_len)
    Cs = w.clusters_per_seg
    for b, g, s in segments:
        a0, a1 = segs[s]
        assign, sums, counts = oracle.spherical_kmeans_segment(
            K64[b, g, lo + a0:lo + a1], Cs, w.iters, w.dtype, oracle.segment_state(seed, b, g, s))
        c0 = s * Cs
        np.testing.assert_array_equal(g_np["sizes"][b, g, c0:c0 + Cs], counts)
        off = g_np["offsets"][b, g, c0:c0 + Cs + 1]
        assert off[0] == a0 and off[-1] == a1
        for j in range(Cs):
            run = g_np["perm"][b, g, off[j]:off[j + 1]]
            want = lo + a0 + np.nonzero(assign == j)[0]
            np.testing.assert_array_equal(run, want)
            if counts[j]:
                mu = oracle.round_to_dtype(sums[j] / counts[j], w.dtype)
                np.testing.assert_array_equal(g_np["centroids"][b, g, c0 + j], mu)
                np.testing.assert_array_equal(g_np["k_perm"][b, g, off[j]:off[j + 1]], K64[b, g, want])
    # whole-index invariants at full size
    for b in range(w.B):
        for g in range(w.Hkv):
            assert g_np["sizes"][b, g].sum() == hi - lo
            np.testing.assert_array_equal(np.diff(g_np["offsets"][b, g]), g_np["sizes"][b, g])
            assert np.array_equal(np.sort(g_np["perm"][b, g]), np.arange(lo, hi))
