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


def test_build_parity_more_uncertain_keys_than_rescore_workgroups():
    # 3000 copies of one key in a 4096-key segment: the seeded init picks several of them, whose
    # clusters share one direction, so every copy ties between them in every iteration and goes
    # to the fp64 re-decision (about 750 keys for each of the segment's four assignment blocks).
    # The lower cluster id must win every tie.
    dev = device()
    w = synth.Workload("b", 1, 1, 1, 128, 4096 + 12, "bf16", 16, 4, 8, 4096, 64, 3, 4)
    K, V, _ = synth.make_instance(w, 8)
    K[0, 0, 4:3004] = K[0, 0, 2000]
    state = oracle.segment_state(13, 0, 0, 0)
    seeds = oracle.init_rows(4096, 64, state)
    assert sum(1 for r in seeds if r < 3000) >= 2      # tied centroids exist from the start
    Kt, Vt = synth.cast(K, "bf16", dev), synth.cast(V, "bf16", dev)
    gi = wi.build_index(Kt, Vt, w.sink, w.window, w.seg_len, w.clusters_per_seg, w.iters, 13)
    torch.cuda.synchronize()
    ref = oracle.build_index(synth.as_float64(Kt), synth.as_float64(Vt), w.sink, w.window,
                             w.seg_len, w.clusters_per_seg, w.iters, 13, "bf16")
    got = index_to_numpy(gi)
    _assert_index_equal(got, ref)
    assert int(got["sizes"].max()) >= 3000


def test_build_parity_uncertain_keys_past_the_block_list():
    # 8 KV heads x 16 segments of 8192 tokens: two assignment blocks per segment, each over 4096
    # keys.  8000 copies of one key in head 0's first segment, among which the init picks 15 of
    # the 16 seeds: every copy ties in every iteration, so each of that segment's blocks has about
    # 4000 keys to re-decide, more than its 2048-entry LDS list holds; the rest are marked in place
    # and found again by the block.
    dev = device()
    w = synth.Workload("b", 1, 8, 8, 128, 16 * 8192 + 12, "bf16", 16, 4, 8, 8192, 16, 2, 4)
    K, V, _ = synth.make_instance(w, 9)
    K[0, 0, 4:8004] = K[0, 0, 3000]
    seeds = oracle.init_rows(8192, 16, oracle.segment_state(13, 0, 0, 0))
    assert sum(1 for r in seeds if r < 8000) >= 2
    Kt, Vt = synth.cast(K, "bf16", dev), synth.cast(V, "bf16", dev)
    gi = wi.build_index(Kt, Vt, w.sink, w.window, w.seg_len, w.clusters_per_seg, w.iters, 13)
    torch.cuda.synchronize()
    ref = oracle.build_index(synth.as_float64(Kt), synth.as_float64(Vt), w.sink, w.window,
                             w.seg_len, w.clusters_per_seg, w.iters, 13, "bf16")
    got = index_to_numpy(gi)
    _assert_index_equal(got, ref)
    assert int(got["sizes"].max()) >= 8000


def test_build_parity_one_cluster_holds_a_whole_65536_token_segment():
    # every key of a segment of the largest supported length is the same: all 65536 tokens go to
    # cluster 0 (ties to the lower id), the largest count the CSR's 16-bit per-wave tables reach
    dev = device()
    w = synth.Workload("b", 1, 1, 1, 128, 65536 + 12, "bf16", 4, 4, 8, 65536, 4, 2, 1)
    K, V, _ = synth.make_instance(w, 3)
    K[0, 0, :] = K[0, 0, 100]
    Kt, Vt = synth.cast(K, "bf16", dev), synth.cast(V, "bf16", dev)
    gi = wi.build_index(Kt, Vt, w.sink, w.window, w.seg_len, w.clusters_per_seg, w.iters, 2)
    torch.cuda.synchronize()
    ref = oracle.build_index(synth.as_float64(Kt), synth.as_float64(Vt), w.sink, w.window,
                             w.seg_len, w.clusters_per_seg, w.iters, 2, "bf16")
    got = index_to_numpy(gi)
    _assert_index_equal(got, ref)
    assert int(got["sizes"].max()) == 65536


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
    ("gqa_128k_bf16", [(0, 3, 15)]),                        # the ragged last segment (8124 tokens)
    ("gqa_1m_bf16", [(0, 7, 127), (0, 0, 64)]),             # 128 segments per KV head
    ("gqa_128k_b16_bf16", [(15, 2, 7), (15, 7, 15)]),      # the last sequence of the batch
])
def test_build_full_size_sampled_segments(name, segments):
    """The full-size build of a workload, with the oracle's k-means and finalize run on sampled
    segments (segments are clustered independently): sizes, offsets, perm, mean keys, value sums
    and the cluster-major K and V rows of the segment bit for bit, and whole-index invariants."""
    dev = device()
    w = synth.WORKLOADS[name]
    if w.B * w.N <= 131072:
        Kt, Vt, _ = inputs(w, 0, dev)[:3]
    else:       # host float64 generation of 1M tokens or 16 sequences is slow: the device recipe
        Kt, Vt, _ = synth.make_instance_device(w, 0, dev)
    seed = 12345
    gi = wi.build_index(Kt, Vt, w.sink, w.window, w.seg_len, w.clusters_per_seg, w.iters, seed)
    torch.cuda.synchronize()
    lo, hi = oracle.clustered_range(w.N, w.sink, w.window)
    segs = oracle.segment_bounds(hi - lo, w.seg_len)
    Cs = w.clusters_per_seg
    f64 = lambda t: t.detach().cpu().to(torch.float64).numpy()
    for b, g, s in segments:
        print(f"[build {name}] segment (b={b}, g={g}, s={s})", flush=True)
        a0, a1 = segs[s]
        Kseg = f64(Kt[b, g, lo + a0:lo + a1])
        Vseg = f64(Vt[b, g, lo + a0:lo + a1])
        assign, _, counts = oracle.spherical_kmeans_segment(Kseg, Cs, w.iters, w.dtype,
                                                            oracle.segment_state(seed, b, g, s))
        ref = oracle.finalize_index(Kseg[None, None], Vseg[None, None], assign[None, None], 0, 0, Cs, w.dtype)
        c0, c1 = s * Cs, (s + 1) * Cs
        off = gi.offsets[b, g, c0:c1 + 1].cpu().numpy().astype(np.int64)
        assert off[0] == a0 and off[-1] == a1
        np.testing.assert_array_equal(gi.sizes[b, g, c0:c1].cpu().numpy(), counts)
        np.testing.assert_array_equal(off - a0, ref.offsets[0, 0])
        np.testing.assert_array_equal(gi.perm[b, g, a0:a1].cpu().numpy(), lo + a0 + ref.perm[0, 0])
        for f, want in (("centroids", ref.centroids[0, 0]), ("value_sums", ref.value_sums[0, 0])):
            got = f64(getattr(gi, f)[b, g, c0:c1])
            np.testing.assert_array_equal(got.view(np.uint64), want.view(np.uint64), err_msg=f)
        for f, want in (("k_perm", ref.k_perm[0, 0]), ("v_perm", ref.v_perm[0, 0])):
            np.testing.assert_array_equal(f64(getattr(gi, f)[b, g, a0:a1]), want, err_msg=f)
    # whole-index invariants at full size
    sizes, offs, perm = gi.sizes.cpu().numpy(), gi.offsets.cpu().numpy(), gi.perm.cpu().numpy()
    for b in range(w.B):
        for g in range(w.Hkv):
            assert sizes[b, g].sum() == hi - lo
            np.testing.assert_array_equal(np.diff(offs[b, g]), sizes[b, g])
            assert np.array_equal(np.sort(perm[b, g]), np.arange(lo, hi))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_build_value_sums_ascending_order_and_two_step_rounding(dtype):
    """Values do not move the clustering, so members of chosen clusters can carry values whose
    float64 sum depends on the order (f32: 2^60, 1, -2^60, 1 sums to 1 left to right, 0 pairwise
    or right to left) or whose rounding depends on the float32 step (bf16: 1 + 2^-8 + 2^-30 stores
    as 1, not 1 + 2^-7).  The clusters are chosen from the oracle's build; both sides must give
    exactly those values."""
    dev = device()
    w = synth.Workload("b", 1, 2, 2, 128, 3000, dtype, 20, 4, 16, 1000, 24, 3, 5)
    K, V, _ = synth.make_instance(w, 8)
    Kt = synth.cast(K, dtype, dev)
    K64 = synth.as_float64(Kt)
    V64 = synth.as_float64(synth.cast(V, dtype))
    ref0 = oracle.build_index(K64, V64, w.sink, w.window, w.seg_len, w.clusters_per_seg, w.iters, 4, dtype)
    pattern = [2.0 ** 60, 1.0, -(2.0 ** 60), 1.0] if dtype == "f32" else [1.0, 2.0 ** -8, 2.0 ** -30]
    planted = []
    for b, h in ((0, 0), (0, 1)):
        sz = ref0.sizes[b, h]
        for c in np.nonzero(sz >= len(pattern))[0][:3]:
            run = ref0.perm[b, h, ref0.offsets[b, h, c]:ref0.offsets[b, h, c + 1]]   # ascending positions
            V64[b, h, run] = 0.0
            V64[b, h, run[:len(pattern)]] = np.asarray(pattern)[:, None]
            planted.append((b, h, c))
    assert len(planted) == 6
    Vt = synth.cast(V64, dtype, dev)
    gi = wi.build_index(Kt, Vt, w.sink, w.window, w.seg_len, w.clusters_per_seg, w.iters, 4)
    torch.cuda.synchronize()
    g = index_to_numpy(gi)
    ref = oracle.build_index(K64, V64, w.sink, w.window, w.seg_len, w.clusters_per_seg, w.iters, 4, dtype)
    for b, h, c in planted:
        assert np.all(ref.value_sums[b, h, c] == 1.0), (b, h, c)
    _assert_index_equal(g, ref)
