"""GPU parity of wi_decode against the CPU oracle (decode side only, on oracle-built indexes).

Gates: selected cluster ids bit-exact (ascending, -1 padded); max |o - oracle| <= 1e-4 (fp32) or
1e-2 (bf16 inputs, fp32 accumulation); |lse - oracle| <= 1e-4; relative RMS error of o <= 1e-3.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from kv_vector_index_amd import synth
from kv_vector_index_amd import wave_index as wi
from wi_testutil import assert_decode_parity, device, inputs, upload_index

pytestmark = pytest.mark.gpu


def _small(**kw):
    # several score tiles (C = 6 x 48 = 288), a ragged last segment, several attention chunks
    w = synth.Workload("small", 2, 8, 2, 128, 6000, "bf16", 40, 4, 32, 1024, 48, 3, 7)
    return w.replace(**kw)


def _run(w, seed, top_k=None, q_scale_override=None, build_seed=5):
    dev = device()
    Kt, Vt, Qt, K64, V64, Q64 = inputs(w, seed, dev)
    idx = oracle.build_index(K64, V64, w.sink, w.window, w.seg_len, w.clusters_per_seg, w.iters,
                             build_seed, w.dtype)
    k = w.top_k if top_k is None else top_k
    gi = upload_index(idx, w.dtype, dev)
    o, lse, sel = wi.decode(gi, Qt, k)
    torch.cuda.synchronize()
    ro, rl, rs = oracle.decode(Q64, idx, w.Hq, k, 1 / math.sqrt(w.d))
    return assert_decode_parity(o, lse, sel, ro, rl, rs, w.dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("G", [1, 4, 8])
def test_decode_parity_small(dtype, G):
    _run(_small(dtype=dtype, Hq=2 * G), seed=10 + G)


@pytest.mark.parametrize("top_k", [0, 1, 13, 287, 288, 400])
def test_decode_parity_top_k_range(top_k):
    _run(_small(B=1, Hq=8), seed=3, top_k=top_k)


@pytest.mark.parametrize("top_k", [1000, 3000])
def test_decode_many_partials_per_head(top_k):
    # one query head per KV group over 60 000 tokens (59 segments x 48 = 2832 clusters): with this
    # many retrieved tokens a head gets 354 (top 1000) or 390 (all) partials, past the merge's
    # 256 (m, den) pairs held in registers and, for 390, past its first round of numerators
    w = synth.Workload("many", 1, 2, 2, 128, 60000, "bf16", 40, 4, 32, 1024, 48, 3, top_k)
    _run(w, seed=17)


def test_decode_sharpened_queries_bf16():
    # a query scale of 12 concentrates attention (max logit ~ 12) so that the 1e-2 gate bites
    _run(_small(q_scale=12.0, q_noise=0.5), seed=4)


def test_decode_all_retrieved_equals_dense_attention():
    dev = device()
    w = _small(B=1, Hq=4, dtype="f32")
    Kt, Vt, Qt, K64, V64, Q64 = inputs(w, 21, dev)
    idx = oracle.build_index(K64, V64, w.sink, w.window, w.seg_len, w.clusters_per_seg, w.iters, 1, "f32")
    gi = upload_index(idx, "f32", dev)
    o, lse, _ = wi.decode(gi, Qt, idx.C)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(128)
    for h in range(w.Hq):
        g = h // (w.Hq // w.Hkv)
        q = torch.from_numpy(Q64[0, h])
        Kd, Vd = torch.from_numpy(K64[0, g]), torch.from_numpy(V64[0, g])
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[None, None, None], Kd[None, None], Vd[None, None], scale=scale)[0, 0, 0].numpy()
        assert np.abs(o[0, h].cpu().numpy() - ref).max() <= 1e-5
        assert abs(float(lse[0, h]) - float(torch.logsumexp(Kd @ q * scale, 0))) <= 1e-5


def test_decode_ties_broken_by_lower_id():
    dev = device()
    rng = np.random.default_rng(7)
    C, d = 300, 128
    mu = oracle.round_to_dtype(rng.standard_normal((C, d)) * 0.1, "bf16")
    for c in range(0, C, 3):
        mu[c + 1] = mu[c]          # every score appears at least twice
    mu[10:40] = mu[9]
    sizes = rng.integers(1, 5, C)
    sizes[::17] = 0                # some empty clusters (never selectable)
    off = np.concatenate([[0], np.cumsum(sizes)])
    Nc = int(off[-1])
    kp = oracle.round_to_dtype(rng.standard_normal((Nc, d)) * 0.1, "bf16")
    vp = oracle.round_to_dtype(rng.standard_normal((Nc, d)), "bf16")
    sv = np.zeros((C, d))
    for c in range(C):
        if sizes[c]:
            sv[c] = oracle.round_to_dtype(vp[off[c]:off[c + 1]].sum(0), "bf16")
    ks = oracle.round_to_dtype(rng.standard_normal((3, d)) * 0.1, "bf16")
    vs = oracle.round_to_dtype(rng.standard_normal((3, d)), "bf16")
    idx = oracle.Index(centroids=mu[None, None], value_sums=sv[None, None], sizes=sizes[None, None],
                       offsets=off[None, None], perm=np.arange(Nc)[None, None] + 3,
                       k_perm=kp[None, None], v_perm=vp[None, None], k_steady=ks[None, None],
                       v_steady=vs[None, None], C=C, Nc=Nc)
    Q64 = oracle.round_to_dtype(rng.standard_normal((1, 4, d)), "bf16")
    Q64[0, 3] = mu[9] * 4          # the 31 tied clusters 9..39 top this head's ranking
    gi = upload_index(idx, "bf16", dev)
    Qt = synth.cast(Q64, "bf16", dev)
    for k in (1, 5, 20, 31, 45, 150):
        o, lse, sel = wi.decode(gi, Qt, k)
        torch.cuda.synchronize()
        ro, rl, rs = oracle.decode(Q64, idx, 4, k, 1 / math.sqrt(d))
        assert_decode_parity(o, lse, sel, ro, rl, rs, "bf16")


def test_decode_steady_only_context():
    dev = device()
    w = _small(B=1, Hq=4, N=50, sink=8, window=64)
    Kt, Vt, Qt, K64, V64, Q64 = inputs(w, 2, dev)
    idx = oracle.build_index(K64, V64, w.sink, w.window, w.seg_len, w.clusters_per_seg, w.iters, 1, "bf16")
    assert idx.C == 0
    gi = upload_index(idx, "bf16", dev)
    o, lse, sel = wi.decode(gi, Qt, 4)
    torch.cuda.synchronize()
    ro, rl, rs = oracle.decode(Q64, idx, w.Hq, 4, 1 / math.sqrt(128))
    assert_decode_parity(o, lse, sel, ro, rl, rs, "bf16")


def test_decode_single_head_8k_f32_workload():
    # one head, fp32, 8192 keys from 64 blobs, 64 clusters, 10 iterations, top 8, 4 + 256 steady
    w = synth.WORKLOADS["single_head_8k_f32"]
    _run(w, seed=0, build_seed=0)


@pytest.mark.parametrize("q_scale", [1.5, 12.0])
def test_decode_gqa_128k_bf16_full_size_every_head(q_scale):
    """The benchmarked launch (B=1, 32/8 heads, 128K, top 164 of 8192 clusters), on an index the
    oracle finalizes from the generator's blob labels (folded into 512 clusters per segment);
    every query head is checked against the oracle.  q_scale 12 sharpens the queries (max logit
    about 12) so that the 1e-2 output gate bites."""
    dev = device()
    w = synth.WORKLOADS["gqa_128k_bf16"].replace(q_scale=q_scale)
    Kt, Vt, Qt, K64, V64, Q64, labels = inputs(w, 0, dev, with_labels=True)
    del Kt, Vt
    lo, hi = oracle.clustered_range(w.N, w.sink, w.window)
    ci = np.arange(hi - lo)
    lab = (ci // w.seg_len) * w.clusters_per_seg + labels[:, :, lo:hi] % w.clusters_per_seg
    C = len(oracle.segment_bounds(hi - lo, w.seg_len)) * w.clusters_per_seg
    idx = oracle.finalize_index(K64, V64, lab, w.sink, w.window, C, w.dtype)
    del K64, V64
    gi = upload_index(idx, w.dtype, dev)
    o, lse, sel = wi.decode(gi, Qt, w.top_k)
    torch.cuda.synchronize()
    ro, rl, rs = oracle.decode(Q64, idx, w.Hq, w.top_k, 1 / math.sqrt(w.d))
    err, _, _ = assert_decode_parity(o, lse, sel, ro, rl, rs, w.dtype)
    if q_scale > 2:
        assert float(np.abs(ro).max()) > 0.1, "sharpened queries should give outputs above the gate"
    G = w.Hq // w.Hkv
    s = sel.cpu().numpy()
    for h in range(w.Hq):
        ids = s[0, h][s[0, h] >= 0]
        assert ids.size == w.top_k and np.all(np.diff(ids) > 0) and np.all(idx.sizes[0, h // G, ids] > 0)


def _oracle_index_slice(gi, b, g):
    """The oracle's view of KV group (b, g) of a device index: exact float64 copies of its arrays
    with leading dimensions of one."""
    f = lambda t: t[b:b + 1, g:g + 1].detach().cpu().to(torch.float64).numpy()
    i = lambda t: t[b:b + 1, g:g + 1].detach().cpu().numpy().astype(np.int64)
    return oracle.Index(centroids=f(gi.centroids), value_sums=f(gi.value_sums), sizes=i(gi.sizes),
                        offsets=i(gi.offsets), perm=i(gi.perm), k_perm=f(gi.k_perm), v_perm=f(gi.v_perm),
                        k_steady=f(gi.k_steady), v_steady=f(gi.v_steady), C=gi.C, Nc=gi.Nc)


def _check_every_head(gi, w, results):
    """results: list of (Q64 [B,Hq,d], o, lse, sel) device results of decode steps on index gi;
    every (b, query head) of every step is decoded by the oracle on the same index, one KV group
    at a time, and held to the parity gates."""
    G = w.Hq // w.Hkv
    scale = 1 / math.sqrt(w.d)
    got = [(o.cpu().numpy().astype(np.float64), l.cpu().numpy().astype(np.float64),
            s.cpu().numpy().astype(np.int64)) for _, o, l, s in results]
    ro = np.zeros((len(results), w.B, w.Hq, w.d))
    rl = np.zeros((len(results), w.B, w.Hq))
    rs = np.full((len(results), w.B, w.Hq, w.top_k), -1, dtype=np.int64)
    for b in range(w.B):
        for g in range(w.Hkv):
            sl = _oracle_index_slice(gi, b, g)
            for t, (Q64, _, _, _) in enumerate(results):
                for h in range(g * G, (g + 1) * G):
                    oh, lh, R = oracle.decode_head(Q64[b, h], sl, 0, 0, w.top_k, scale)
                    ro[t, b, h], rl[t, b, h] = oh, lh
                    rs[t, b, h, :R.size] = R
            del sl
    for t, (o, l, s) in enumerate(got):
        assert_decode_parity(torch.from_numpy(o), torch.from_numpy(l), torch.from_numpy(s),
                             ro[t], rl[t], rs[t], w.dtype)


def test_decode_gqa_128k_b16_drifting_steps_every_head():
    """Batch 16 at 128K context, 100 decode steps whose queries drift by N(0, 0.1) per step, on
    the device-built index of the full batch; the oracle checks all 16 x 32 query heads at the
    first, a middle and the last step, on the same index (build parity is tested on its own)."""
    dev = device()
    w = synth.WORKLOADS["gqa_128k_b16_bf16"]
    Kt, Vt, Qt = synth.make_instance_device(w, 0, dev)
    gi = wi.build_index(Kt, Vt, w.sink, w.window, w.seg_len, w.clusters_per_seg, w.iters, 1)
    del Kt, Vt
    qm = synth.drift_queries_device(Qt, w.steps, w.drift, 0)
    checks = {0: None, 50: None, w.steps - 1: None}
    for t in range(w.steps):
        q = qm[t].to(torch.float32).to(Qt.dtype)
        o, lse, sel = wi.decode(gi, q, w.top_k)
        if t in checks:
            checks[t] = (synth.as_float64(q), o.clone(), lse.clone(), sel.clone())
    torch.cuda.synchronize()
    print(f"[decode b16] 100 steps done; oracle over {w.B * w.Hq} heads x 3 steps", flush=True)
    _check_every_head(gi, w, list(checks.values()))


def test_decode_gqa_1m_bf16_every_head():
    """One million tokens per KV head (65536 clusters, top 656): the device-built index decoded
    once, every query head checked against the oracle on the same index."""
    dev = device()
    w = synth.WORKLOADS["gqa_1m_bf16"]
    Kt, Vt, Qt = synth.make_instance_device(w, 0, dev)
    gi = wi.build_index(Kt, Vt, w.sink, w.window, w.seg_len, w.clusters_per_seg, w.iters, 1)
    del Kt, Vt
    o, lse, sel = wi.decode(gi, Qt, w.top_k)
    torch.cuda.synchronize()
    _check_every_head(gi, w, [(synth.as_float64(Qt), o, lse, sel)])


def test_decode_graph_replay_matches_eager():
    """Decode steps captured in a HIP graph and replayed several times, with eager work and
    synchronisations between replays, give the eager result every time (the kernels zero their
    own counters, so nothing in the graph is a memset)."""
    dev = device()
    w = _small(B=2, Hq=8)
    Kt, Vt, Qt, K64, V64, Q64 = inputs(w, 31, dev)
    idx = oracle.build_index(K64, V64, w.sink, w.window, w.seg_len, w.clusters_per_seg, w.iters, 2, w.dtype)
    gi = upload_index(idx, w.dtype, dev)
    q2 = (Qt.float() * 1.3).to(Qt.dtype)
    p = wi.decode_params(gi, w.B, w.Hq, w.Hkv, w.top_k, Qt.dtype)
    ws = torch.empty(wi.wi_decode_workspace_bytes(p), dtype=torch.uint8, device=dev)
    outs = [torch.empty((w.B, w.Hq, 128), dtype=torch.float32, device=dev) for _ in range(2)]
    lses = [torch.empty((w.B, w.Hq), dtype=torch.float32, device=dev) for _ in range(2)]
    sels = [torch.empty((w.B, w.Hq, w.top_k), dtype=torch.int32, device=dev) for _ in range(2)]
    view = gi.view()

    def steps():
        for j, q in enumerate((Qt, q2)):
            wi.wi_decode(p, view, q.data_ptr(), outs[j].data_ptr(), lses[j].data_ptr(), sels[j].data_ptr(),
                         ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)

    steps()
    torch.cuda.synchronize()
    ref = [(o.clone(), l.clone(), s.clone()) for o, l, s in zip(outs, lses, sels)]
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            steps()
    torch.cuda.current_stream().wait_stream(st)
    for r in range(4):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        _ = (torch.randn(1000, device=dev) * 2).sum()     # eager work between replays
        torch.cuda.synchronize()
        for (o, l, s), (ro, rl, rs) in zip(zip(outs, lses, sels), ref):
            assert torch.equal(s, rs)
            assert torch.equal(o, ro) and torch.equal(l, rl)


def test_decode_repeated_launches_and_back_to_back_calls_agree():
    # every decode kernel is a pure function of its inputs and of what the earlier kernels of
    # the same call wrote: repeated launches (the profiling hook's repeat mode) and consecutive
    # calls on one workspace give identical results
    dev = device()
    w = _small(B=1, Hq=8)
    Kt, Vt, Qt, K64, V64, Q64 = inputs(w, 31, dev)
    idx = oracle.build_index(K64, V64, w.sink, w.window, w.seg_len, w.clusters_per_seg, w.iters, 2,
                             w.dtype)
    gi = upload_index(idx, w.dtype, dev)
    o1, l1, s1 = wi.decode(gi, Qt, w.top_k)
    copies = [gi.clone(), gi.clone()]
    wi.wi_profile_rotate([c.view() for c in copies])       # repeats read copies at other addresses
    wi.wi_profile_enable(True, 3)
    o2, l2, s2 = wi.decode(gi, Qt, w.top_k)
    torch.cuda.synchronize()
    launches = wi.wi_profile_read()["attend"][1]
    wi.wi_profile_enable(False)
    wi.wi_profile_rotate([])
    o3, l3, s3 = wi.decode(gi, Qt, w.top_k)
    torch.cuda.synchronize()
    assert launches == 3
    for o, l, s in ((o2, l2, s2), (o3, l3, s3)):
        assert torch.equal(o, o1) and torch.equal(l, l1) and torch.equal(s, s1)
    ro, rl, rs = oracle.decode(Q64, idx, w.Hq, w.top_k, 1 / math.sqrt(w.d))
    assert_decode_parity(o1, l1, s1, ro, rl, rs, w.dtype)
