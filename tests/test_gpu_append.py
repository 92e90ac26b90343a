"""GPU checks of wi_index_append_segment: growing an index by the segment of tokens that left the
local window gives, bit for bit, the index a full build of the grown context gives (segments are
clustered independently, each from its own seed), and that index matches the oracle's."""
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


def _equal(a: wi.Index, b: wi.Index):
    assert (a.C, a.Nc, a.n_steady) == (b.C, b.Nc, b.n_steady)
    for f in FIELDS:
        x, y = getattr(a, f), getattr(b, f)
        assert x.shape == y.shape, f
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y), f


def _grow(w, seed, build_seed, segments_before):
    """Index of the first N - k * seg_len tokens grown segment by segment to N, and the full build."""
    dev = device()
    Kt, Vt, Qt, K64, V64, Q64 = inputs(w, seed, dev)
    L = w.seg_len
    n0 = w.N - segments_before * L
    idx = wi.build_index(Kt[:, :, :n0].contiguous(), Vt[:, :, :n0].contiguous(), w.sink, w.window, L,
                         w.clusters_per_seg, w.iters, build_seed)
    for n in range(n0 + L, w.N + 1, L):
        idx = wi.append_segment(idx, Kt[:, :, :n].contiguous(), Vt[:, :, :n].contiguous(), w.sink, w.window,
                                L, w.clusters_per_seg, w.iters, build_seed)
    full = wi.build_index(Kt, Vt, w.sink, w.window, L, w.clusters_per_seg, w.iters, build_seed)
    torch.cuda.synchronize()
    return idx, full, (Kt, Vt, Qt, K64, V64, Q64)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_append_one_segment_equals_full_build(dtype):
    # 2 x 2 KV heads, 3 segments of 700 tokens (40 clusters each) grown to 4
    w = synth.Workload("a", 2, 4, 2, 128, 4 + 20 + 4 * 700, dtype, 30, 4, 20, 700, 40, 4, 5)
    grown, full, _ = _grow(w, 1, 77, 1)
    _equal(grown, full)


def test_append_first_segment_and_a_chain_of_segments():
    # from the steady zone alone (no clustered token yet) to 3 segments, one at a time
    w = synth.Workload("a", 1, 8, 2, 128, 8 + 32 + 3 * 512, "bf16", 24, 8, 32, 512, 32, 3, 5)
    grown, full, _ = _grow(w, 2, 5, 3)
    _equal(grown, full)


def test_append_matches_oracle_and_decodes():
    w = synth.Workload("a", 1, 8, 2, 128, 4 + 16 + 3 * 600, "bf16", 20, 4, 16, 600, 30, 4, 12)
    grown, full, (Kt, Vt, Qt, K64, V64, Q64) = _grow(w, 3, 9, 2)
    _equal(grown, full)
    ref = oracle.build_index(K64, V64, w.sink, w.window, w.seg_len, w.clusters_per_seg, w.iters, 9, w.dtype)
    got = index_to_numpy(grown)
    for f in FIELDS:
        a, b = got[f], getattr(ref, f)
        if a.dtype.kind == "f":
            np.testing.assert_array_equal(a.view(np.uint64), b.view(np.uint64), err_msg=f)
        else:
            np.testing.assert_array_equal(a, b, err_msg=f)
    o, lse, sel = wi.decode(grown, Qt, w.top_k)
    torch.cuda.synchronize()
    ro, rl, rs = oracle.decode(Q64, ref, w.Hq, w.top_k, 1 / math.sqrt(w.d))
    assert_decode_parity(o, lse, sel, ro, rl, rs, w.dtype)


def test_append_full_size_segment_bf16():
    # the 128K workload grown by one segment of 8192 tokens: 8 KV heads x 17 segments of 512
    # clusters, compared with the full build (segments before the last are copies)
    w = synth.WORKLOADS["build_128k_bf16"].replace(N=131072 + 8192)
    grown, full, _ = _grow(w, 0, 12345, 1)
    _equal(grown, full)
