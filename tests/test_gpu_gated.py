"""GPU parity of wi_decode_gated: decode that keeps the previous step's retrieval zone for every KV
head whose query heads all moved by a cosine of at least tau, and selects afresh elsewhere.

The oracle (oracle.decode_gated) takes the same gate from canonical fp64 sums, so the gate
decision, the zones and the reuse flags are compared bit-exactly; outputs to the dtype tolerance.
Every sel_prev handed to the oracle comes from the oracle itself (its decode of the previous
queries, or a hand-made list), never from the device.

Indexes come from oracle.finalize_index on random labels, so that cluster counts and empty
clusters can be chosen directly.
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

SINK, WINDOW, D = 4, 16, 128


def _index(C, tokens_per_cluster, Hkv, dtype, seed, B=1, empty_frac=0.1):
    rng = np.random.default_rng(seed)
    Nc = C * tokens_per_cluster
    N = Nc + SINK + WINDOW
    K = rng.standard_normal((B, Hkv, N, D))
    K /= np.linalg.norm(K, axis=-1, keepdims=True)
    V = rng.standard_normal((B, Hkv, N, D))
    labels = np.empty((B, Hkv, Nc), dtype=np.int64)
    for b in range(B):
        for g in range(Hkv):
            live = np.nonzero(rng.random(C) >= empty_frac)[0]
            lab = np.concatenate([live, rng.choice(live, Nc - live.size)])
            rng.shuffle(lab)
            labels[b, g] = lab
    dev = device()
    Kt, Vt = (synth.cast(x, dtype, dev) for x in (K, V))
    K64, V64 = (synth.as_float64(t) for t in (Kt, Vt))
    return oracle.finalize_index(K64, V64, labels, SINK, WINDOW, C, dtype)


def _queries(Q, dtype):
    """Device copy of Q in dtype and its exact float64 copy."""
    Qt = synth.cast(Q, dtype, device())
    return Qt, synth.as_float64(Qt)


def _drift(rng, Q, groups_moving, G, small=0.02, large=3.0):
    """Q plus a small perturbation everywhere, and a large one on the heads of `groups_moving`
    (a tuple of (b, g))."""
    Qn = Q + small * rng.standard_normal(Q.shape) * np.abs(Q).mean()
    for b, g in groups_moving:
        Qn[b, g * G:(g + 1) * G] = large * rng.standard_normal((G, Q.shape[-1]))
    return Qn


def _run(gi, Qt, Qpt, sel_prev, k, tau):
    sp = torch.from_numpy(np.ascontiguousarray(sel_prev).astype(np.int32)).to(device())
    o, lse, sel, reused = wi.decode_gated(gi, Qt, Qpt, sp, k, tau)
    torch.cuda.synchronize()
    return o, lse, sel, reused


def _check(o, lse, sel, reused, ro, rl, rs, rr, dtype):
    np.testing.assert_array_equal(reused.cpu().numpy().astype(bool), rr)
    assert_decode_parity(o, lse, sel, ro, rl, rs, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gated_mixed_reuse_matches_oracle(dtype):
    # 2 sequences x 4 KV heads of 4 query heads; three groups jump, the other five barely move
    rng = np.random.default_rng(11)
    B, Hkv, G, C, k = 2, 4, 4, 768, 40
    Hq = Hkv * G
    idx = _index(C, 3, Hkv, dtype, seed=11, B=B)
    gi = upload_index(idx, dtype, device())
    Qp = 1.5 * rng.standard_normal((B, Hq, D))
    Qn = _drift(rng, Qp, [(0, 1), (1, 0), (1, 3)], G)
    Qpt, Qp64 = _queries(Qp, dtype)
    Qt, Q64 = _queries(Qn, dtype)
    _, _, rs_prev = oracle.decode(Qp64, idx, Hq, k)
    ro, rl, rs, rr = oracle.decode_gated(Q64, Qp64, rs_prev, idx, Hq, k, tau=0.9)
    assert rr.sum() == 5 and not rr[0, 1] and not rr[1, 0] and not rr[1, 3]
    # the reused zones are stale: some head's fresh top-k differs from what it keeps
    _, _, rs_fresh = oracle.decode(Q64, idx, Hq, k)
    assert (rs_fresh != rs).any()
    _check(*_run(gi, Qt, Qpt, rs_prev, k, 0.9), ro, rl, rs, rr, dtype)


def test_gated_chained_steps_follow_the_oracle_chain():
    # five steps; each step's sel feeds the next; the moving groups change from step to step
    dtype = "bf16"
    rng = np.random.default_rng(12)
    B, Hkv, G, C, k = 1, 8, 4, 1024, 64
    Hq = Hkv * G
    idx = _index(C, 2, Hkv, dtype, seed=12, B=B)
    gi = upload_index(idx, dtype, device())
    Q = 1.5 * rng.standard_normal((B, Hq, D))
    Qpt, Qp64 = _queries(Q, dtype)
    _, _, rs = oracle.decode(Qp64, idx, Hq, k)
    sel_dev = torch.from_numpy(rs.astype(np.int32)).to(device())
    moving = [[(0, 0), (0, 5)], [], [(0, 1), (0, 2), (0, 3)], [(0, g) for g in range(8)], [(0, 7)]]
    for step, mv in enumerate(moving):
        Q = _drift(rng, Q, mv, G, small=0.05)
        Qt, Q64 = _queries(Q, dtype)
        ro, rl, rs_new, rr = oracle.decode_gated(Q64, Qp64, rs, idx, Hq, k, tau=0.95)
        assert int(rr.sum()) == Hkv - len(mv), step
        o, lse, sel, reused = wi.decode_gated(gi, Qt, Qpt, sel_dev, k, 0.95)
        torch.cuda.synchronize()
        _check(o, lse, sel, reused, ro, rl, rs_new, rr, dtype)
        Qpt, Qp64, rs, sel_dev = Qt, Q64, rs_new, sel


def test_gated_stale_lists_with_repeats_padding_and_out_of_range_ids():
    # sel_prev written by hand: -1 padding, repeats, ids >= C, negative ids and empty clusters
    dtype = "f32"
    rng = np.random.default_rng(13)
    B, Hkv, G, C, k = 1, 2, 4, 512, 48
    Hq = Hkv * G
    idx = _index(C, 3, Hkv, dtype, seed=13, empty_frac=0.3)
    gi = upload_index(idx, dtype, device())
    Qp = 1.5 * rng.standard_normal((B, Hq, D))
    Qn = _drift(rng, Qp, [], G)
    Qpt, Qp64 = _queries(Qp, dtype)
    Qt, Q64 = _queries(Qn, dtype)
    sel_prev = rng.integers(-3, C + 40, size=(B, Hq, k))
    sel_prev[0, 0, 10:] = -1
    sel_prev[0, 1, :] = sel_prev[0, 1, 0]                        # one id repeated
    sel_prev[0, 2, :] = -1                                       # nothing kept
    empty = np.nonzero(idx.sizes[0, 0] == 0)[0][:k // 2]
    assert empty.size > 0
    sel_prev[0, 3, :empty.size] = empty                          # empty clusters only
    sel_prev[0, 3, empty.size:] = C + 7
    ro, rl, rs, rr = oracle.decode_gated(Q64, Qp64, sel_prev, idx, Hq, k, tau=0.5)
    assert rr.all()
    _check(*_run(gi, Qt, Qpt, sel_prev, k, 0.5), ro, rl, rs, rr, dtype)


def test_gated_tau_above_one_is_plain_decode_and_zero_queries_reuse_at_tau_zero():
    dtype = "bf16"
    rng = np.random.default_rng(14)
    B, Hkv, G, C, k = 1, 2, 4, 512, 32
    Hq = Hkv * G
    idx = _index(C, 2, Hkv, dtype, seed=14)
    gi = upload_index(idx, dtype, device())
    Qp = 1.5 * rng.standard_normal((B, Hq, D))
    Qpt, Qp64 = _queries(Qp, dtype)
    Qt, Q64 = _queries(Qp, dtype)                                # the same queries: cos = 1
    _, _, rs_prev = oracle.decode(Qp64, idx, Hq, k)
    sel_prev = np.roll(rs_prev, 1, axis=1)                       # another head's zone
    o, lse, sel, reused = _run(gi, Qt, Qpt, sel_prev, k, 1.0000001)
    assert reused.sum().item() == 0
    ro, rl, rs = oracle.decode(Q64, idx, Hq, k)
    assert_decode_parity(o, lse, sel, ro, rl, rs, dtype)
    o2, _, sel2 = wi.decode(gi, Qt, k)
    torch.cuda.synchronize()
    assert torch.equal(sel2, sel) and torch.equal(o2, o)
    # a zero query has cosine 0: its group reuses at tau <= 0 and not above
    Qz = Qp.copy()
    Qz[0, 5] = 0.0
    Qzt, Qz64 = _queries(Qz, dtype)
    for tau, want in ((0.0, [True, True]), (1e-6, [True, False])):
        ro, rl, rs, rr = oracle.decode_gated(Qz64, Qp64, sel_prev, idx, Hq, k, tau=tau)
        assert rr[0].tolist() == want
        _check(*_run(gi, Qzt, Qpt, sel_prev, k, tau), ro, rl, rs, rr, dtype)


def test_gated_reused_zone_covering_every_cluster_is_dense_attention():
    dtype = "f32"
    rng = np.random.default_rng(15)
    B, Hkv, G, C = 1, 2, 2, 256
    Hq = Hkv * G
    idx = _index(C, 2, Hkv, dtype, seed=15)
    gi = upload_index(idx, dtype, device())
    k = 300
    Qp = 1.5 * rng.standard_normal((B, Hq, D))
    Qpt, Qp64 = _queries(Qp, dtype)
    Qt, Q64 = _queries(_drift(rng, Qp, [], G), dtype)
    sel_prev = np.full((B, Hq, k), -1)
    sel_prev[:, :, :C] = np.arange(C)[::-1]
    ro, rl, rs, rr = oracle.decode_gated(Q64, Qp64, sel_prev, idx, Hq, k, tau=0.9)
    assert rr.all()
    _check(*_run(gi, Qt, Qpt, sel_prev, k, 0.9), ro, rl, rs, rr, dtype)


def test_gated_long_zones_published_from_global_lists():
    # top_k = 5000 > 4096: the select keeps the retrieved list in global memory
    dtype = "bf16"
    rng = np.random.default_rng(16)
    B, Hkv, G, C, k = 1, 1, 2, 8192, 5000
    Hq = Hkv * G
    idx = _index(C, 1, Hkv, dtype, seed=16)
    gi = upload_index(idx, dtype, device())
    Qp = 8.0 * rng.standard_normal((B, Hq, D)) / math.sqrt(D)
    Qpt, Qp64 = _queries(Qp, dtype)
    Qt, Q64 = _queries(_drift(rng, Qp, [], G), dtype)
    _, _, rs_prev = oracle.decode(Qp64, idx, Hq, k)
    ro, rl, rs, rr = oracle.decode_gated(Q64, Qp64, rs_prev, idx, Hq, k, tau=0.9)
    assert rr.all()
    _check(*_run(gi, Qt, Qpt, rs_prev, k, 0.9), ro, rl, rs, rr, dtype)


def test_gated_many_heads_half_size_select_blocks():
    # 272 query heads (34 KV heads of 8): the select runs at 512 threads; every third group moves
    dtype = "bf16"
    rng = np.random.default_rng(17)
    B, Hkv, G, C, k = 1, 34, 8, 512, 24
    Hq = Hkv * G
    idx = _index(C, 2, Hkv, dtype, seed=17)
    gi = upload_index(idx, dtype, device())
    Qp = 1.5 * rng.standard_normal((B, Hq, D))
    Qpt, Qp64 = _queries(Qp, dtype)
    Qt, Q64 = _queries(_drift(rng, Qp, [(0, g) for g in range(0, Hkv, 3)], G), dtype)
    _, _, rs_prev = oracle.decode(Qp64, idx, Hq, k)
    ro, rl, rs, rr = oracle.decode_gated(Q64, Qp64, rs_prev, idx, Hq, k, tau=0.9)
    assert int(rr.sum()) == Hkv - len(range(0, Hkv, 3))
    _check(*_run(gi, Qt, Qpt, rs_prev, k, 0.9), ro, rl, rs, rr, dtype)


# ------------------------------------------------------------------ postponed selection (refresh)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_refresh_gives_every_head_its_current_top_k(dtype):
    rng = np.random.default_rng(21)
    B, Hkv, G, C, k = 2, 4, 4, 768, 40
    Hq = Hkv * G
    idx = _index(C, 3, Hkv, dtype, seed=21, B=B)
    gi = upload_index(idx, dtype, device())
    Qp = 1.5 * rng.standard_normal((B, Hq, D))
    Qpt, Qp64 = _queries(Qp, dtype)
    Qt, Q64 = _queries(_drift(rng, Qp, [(0, 2), (1, 1)], G), dtype)
    _, _, rs_prev = oracle.decode(Qp64, idx, Hq, k)
    ro, rl, rs, rr = oracle.decode_gated(Q64, Qp64, rs_prev, idx, Hq, k, tau=0.9, refresh=True)
    assert rr.sum() == 6
    sp = torch.from_numpy(rs_prev.astype(np.int32)).to(device())
    o, lse, sel, reused = wi.decode_gated(gi, Qt, Qpt, sp, k, 0.9, refresh=True)
    torch.cuda.synchronize()
    _check(o, lse, sel, reused, ro, rl, rs, rr, dtype)


def test_refresh_chain_keeps_zones_one_step_old():
    # FreeKV's scheme over six steps: each step attends over the previous step's fresh top-k
    # where its queries stayed within tau, and hands its own fresh top-k to the next step
    dtype = "bf16"
    rng = np.random.default_rng(22)
    B, Hkv, G, C, k = 1, 8, 4, 1024, 64
    Hq = Hkv * G
    idx = _index(C, 2, Hkv, dtype, seed=22)
    gi = upload_index(idx, dtype, device())
    Q = 1.5 * rng.standard_normal((B, Hq, D))
    Qpt, Qp64 = _queries(Q, dtype)
    _, _, rs = oracle.decode(Qp64, idx, Hq, k)
    sel_dev = torch.from_numpy(rs.astype(np.int32)).to(device())
    moving = [[], [(0, 3)], [], [(0, g) for g in range(0, 8, 2)], [], [(0, 6)]]
    stale = 0
    for step, mv in enumerate(moving):
        Q = _drift(rng, Q, mv, G, small=0.1)
        Qt, Q64 = _queries(Q, dtype)
        ro, rl, rs_new, rr = oracle.decode_gated(Q64, Qp64, rs, idx, Hq, k, tau=0.95, refresh=True)
        assert int(rr.sum()) == Hkv - len(mv), step
        _, _, rs_fresh = oracle.decode(Q64, idx, Hq, k)
        np.testing.assert_array_equal(rs_new, rs_fresh)
        stale += int((rs != rs_fresh).any(axis=-1).sum())
        o, lse, sel, reused = wi.decode_gated(gi, Qt, Qpt, sel_dev, k, 0.95, refresh=True)
        torch.cuda.synchronize()
        _check(o, lse, sel, reused, ro, rl, rs_new, rr, dtype)
        Qpt, Qp64, rs, sel_dev = Qt, Q64, rs_new, sel
    assert stale > 0                              # some kept zones really were out of date


def test_refresh_after_plain_decode_leaves_sel_ids_alone_and_runs_on_another_stream():
    dtype = "bf16"
    rng = np.random.default_rng(23)
    B, Hkv, G, C, k = 1, 2, 4, 512, 32
    Hq = Hkv * G
    idx = _index(C, 2, Hkv, dtype, seed=23)
    gi = upload_index(idx, dtype, device())
    Qp = 1.5 * rng.standard_normal((B, Hq, D))
    Qpt, Qp64 = _queries(Qp, dtype)
    Qt, Q64 = _queries(_drift(rng, Qp, [], G), dtype)
    p = wi.decode_params(gi, B, Hq, Hkv, k, Qt.dtype)
    p.d = D
    p.dtype = wi._dtype_code(Qt)
    need = wi.wi_decode_workspace_bytes(p)
    ws = torch.empty(need, dtype=torch.uint8, device=device())
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=device())
    sel = torch.empty((B, Hq, k), dtype=torch.int32, device=device())
    view = gi.view()
    stream = torch.cuda.current_stream().cuda_stream
    # after a plain decode the refresh has nothing to do
    wi.wi_decode(p, view, Qt.data_ptr(), out.data_ptr(), None, sel.data_ptr(), ws.data_ptr(), need, stream)
    sel.fill_(-7)
    wi.wi_select_refresh(p, view, Qt.data_ptr(), sel.data_ptr(), ws.data_ptr(), need, stream)
    torch.cuda.synchronize()
    assert bool((sel == -7).all())
    # gated step on the current stream, refresh on a side stream ordered after it by an event
    _, _, rs_prev = oracle.decode(Qp64, idx, Hq, k)
    ro, rl, rs, rr = oracle.decode_gated(Q64, Qp64, rs_prev, idx, Hq, k, tau=0.9, refresh=True)
    assert rr.all()
    sp = torch.from_numpy(rs_prev.astype(np.int32)).to(device())
    lse = torch.empty((B, Hq), dtype=torch.float32, device=device())
    reused = torch.empty((B, Hkv), dtype=torch.int32, device=device())
    wi.wi_decode_gated(p, view, Qt.data_ptr(), Qpt.data_ptr(), sp.data_ptr(), 0.9, out.data_ptr(), lse.data_ptr(),
                       sel.data_ptr(), reused.data_ptr(), ws.data_ptr(), need, stream)
    done = torch.cuda.Event()
    done.record()
    side = torch.cuda.Stream()
    side.wait_event(done)
    wi.wi_select_refresh(p, view, Qt.data_ptr(), sel.data_ptr(), ws.data_ptr(), need, side.cuda_stream)
    torch.cuda.synchronize()
    _check(out, lse, sel, reused, ro, rl, rs, rr, dtype)


def test_refresh_long_lists_and_half_size_select_blocks():
    # top_k = 5000 (lists in global memory), then 272 heads (512-thread select)
    for (B, Hkv, G, C, tpc, k, dtype, seed) in ((1, 1, 2, 8192, 1, 5000, "bf16", 24),
                                                (1, 34, 8, 512, 2, 24, "f32", 25)):
        rng = np.random.default_rng(seed)
        Hq = Hkv * G
        idx = _index(C, tpc, Hkv, dtype, seed=seed)
        gi = upload_index(idx, dtype, device())
        Qp = 8.0 * rng.standard_normal((B, Hq, D)) / math.sqrt(D)
        Qpt, Qp64 = _queries(Qp, dtype)
        Qt, Q64 = _queries(_drift(rng, Qp, [(0, 0)] if Hkv > 1 else [], G, small=0.1), dtype)
        _, _, rs_prev = oracle.decode(Qp64, idx, Hq, k)
        ro, rl, rs, rr = oracle.decode_gated(Q64, Qp64, rs_prev, idx, Hq, k, tau=0.9, refresh=True)
        sp = torch.from_numpy(rs_prev.astype(np.int32)).to(device())
        o, lse, sel, reused = wi.decode_gated(gi, Qt, Qpt, sp, k, 0.9, refresh=True)
        torch.cuda.synchronize()
        _check(o, lse, sel, reused, ro, rl, rs, rr, dtype)


def test_gated_full_size_sampled_heads():
    """The benchmarked shape (B=1, 32/8 heads, 128K, top 164 of 8192 clusters) on an index the
    oracle finalizes from the generator's blob labels; the previous step's queries are the
    generator's, the current ones drift by N(0, 0.1^2) per coordinate, and sel_prev is the
    oracle's own top-k of the previous queries.  Sampled heads of a kept and (by moving one
    group's queries far) a re-selected group are checked against the oracle one by one."""
    dev = device()
    w = synth.WORKLOADS["gqa_128k_bf16"]
    from wi_testutil import inputs
    Kt, Vt, Qpt, K64, V64, Qp64, labels = inputs(w, 0, dev, with_labels=True)
    lo, hi = oracle.clustered_range(w.N, w.sink, w.window)
    lab = (np.arange(hi - lo) // w.seg_len) * w.clusters_per_seg + labels[:, :, lo:hi] % w.clusters_per_seg
    C = len(oracle.segment_bounds(hi - lo, w.seg_len)) * w.clusters_per_seg
    idx = oracle.finalize_index(K64, V64, lab, w.sink, w.window, C, w.dtype)
    gi = upload_index(idx, w.dtype, dev)
    G = w.Hq // w.Hkv
    rng = np.random.default_rng(31)
    Qn = Qp64 + 0.1 * rng.standard_normal(Qp64.shape)
    Qn[0, 3 * G:4 * G] = 3.0 * rng.standard_normal((G, w.d))       # group 3 moves away
    Qt, Q64 = _queries(Qn, w.dtype)
    scale = 1 / math.sqrt(w.d)
    # the oracle's top-k of the previous queries, for every head
    sel_prev = np.full((1, w.Hq, w.top_k), -1, dtype=np.int64)
    for h in range(w.Hq):
        R = oracle.decode_head(Qp64[0, h], idx, 0, h // G, w.top_k, scale)[2]
        sel_prev[0, h, :R.size] = R
    o, lse, sel, reused = _run(gi, Qt, Qpt, sel_prev, w.top_k, 0.9)
    r = reused.cpu().numpy()[0]
    heads = [(0, 0), (0, 5), (0, 13), (0, 14), (0, 31)]
    want_reuse = [all(oracle.query_cosine(Q64[0, j], Qp64[0, j]) >= 0.9 for j in range(g * G, (g + 1) * G))
                  for g in range(w.Hkv)]
    np.testing.assert_array_equal(r.astype(bool), want_reuse)
    assert not want_reuse[3] and sum(want_reuse) >= 6
    res = []
    for b, h in heads:
        g = h // G
        R = np.unique(sel_prev[b, h][sel_prev[b, h] >= 0]) if want_reuse[g] else None
        res.append(oracle.decode_head(Q64[b, h], idx, b, g, w.top_k, scale, R))
    ro = np.stack([x[0] for x in res])
    rl = np.array([x[1] for x in res])
    rs = np.stack([np.concatenate([x[2], -np.ones(w.top_k - x[2].size, dtype=np.int64)]) for x in res])
    assert_decode_parity(o, lse, sel, ro, rl, rs, w.dtype, heads=heads)
