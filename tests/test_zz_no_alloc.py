"""wi_decode_noalloc (the library's static workspace) against wi_decode (a caller workspace):
the same kernels, so the results must be identical bit for bit, on two calls in a row of which
the second is smaller, and both must meet the oracle's gates."""
import math

import pytest
import torch

import oracle
from kv_vector_index_amd import synth
from kv_vector_index_amd import wave_index as wi
from wi_testutil import assert_decode_parity, device, inputs, upload_index

pytestmark = pytest.mark.gpu


def _case(w, seed, build_seed):
    dev = device()
    Kt, Vt, Qt, K64, V64, Q64 = inputs(w, seed, dev)
    idx = oracle.build_index(K64, V64, w.sink, w.window, w.seg_len, w.clusters_per_seg, w.iters,
                             build_seed, w.dtype)
    return idx, upload_index(idx, w.dtype, dev), Qt, Q64


def _noalloc(gi, B, Hq, Hkv, top_k, q):
    dev = q.device
    p = wi.decode_params(gi, B, Hq, Hkv, top_k, q.dtype)
    out = torch.full((B, Hq, 128), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=dev)
    sel = torch.full((B, Hq, top_k), -7, dtype=torch.int32, device=dev)
    wi.wi_decode_noalloc(p, gi.view(), q.data_ptr(), out.data_ptr(), lse.data_ptr(), sel.data_ptr(),
                         torch.cuda.current_stream().cuda_stream)
    return out, lse, sel


def test_decode_noalloc_equals_decode_on_two_calls_second_smaller():
    big = synth.Workload("big", 2, 16, 4, 128, 9000, "bf16", 40, 4, 32, 2048, 64, 3, 29)
    small = synth.Workload("small", 1, 4, 1, 128, 1500, "f32", 12, 4, 16, 512, 16, 3, 5)
    for w, seed in ((big, 3), (small, 4)):
        print(f"[no-alloc] workload {w.name} B={w.B} Hq={w.Hq} N={w.N} {w.dtype}", flush=True)
        idx, gi, Qt, Q64 = _case(w, seed, 9)
        o1, l1, s1 = wi.decode(gi, Qt, w.top_k)
        o2, l2, s2 = _noalloc(gi, w.B, w.Hq, w.Hkv, w.top_k, Qt)
        torch.cuda.synchronize()
        assert torch.equal(s1, s2)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        ro, rl, rs = oracle.decode(Q64, idx, w.Hq, w.top_k, 1 / math.sqrt(w.d))
        assert_decode_parity(o2, l2, s2, ro, rl, rs, w.dtype)
