"""GPU tests of the wave buffer (wi_decode_wavebuf): decode over an index whose cluster-major K/V
copies are in pinned host memory, through a GPU block cache and an execution buffer.

Every step's out, lse and sel_ids meet the oracle's gates on the same index (the oracle decodes
every head of every step), and where the rows come from must not change what is computed: they
equal wi_decode's on the same index in device memory, bit for bit, whatever the cache holds.
The cache's behaviour is checked against a plain LRU model fed with the blocks that the oracle's
retrieval zones touch (16-row blocks of the cluster-major rows, once per (b, KV head) and step):
per step the hits, the staged misses, the admissions and the evictions.
"""
from collections import OrderedDict

import numpy as np
import pytest
import torch

import oracle
from kv_vector_index_amd import synth
from kv_vector_index_amd import wave_index as wi
from wi_testutil import assert_decode_parity, device, upload_index

pytestmark = pytest.mark.gpu

D = 128
BLK = wi.WB_BLOCK


def _setup(dtype, seed, N=2048, Hq=8, Hkv=2, top_k=12, B=1):
    w = synth.Workload("wb", B, Hq, Hkv, D, N, dtype, 24, 4, 32, 512, 32, 4, top_k)
    K, V, Q = synth.make_instance(w, seed)
    dev = device()
    Kt, Vt, Qt = (synth.cast(x, dtype, dev) for x in (K, V, Q))
    K64, V64, Q64 = (synth.as_float64(t) for t in (Kt, Vt, Qt))
    idx = oracle.build_index(K64, V64, w.sink, w.window, 512, 32, w.iters, 7, dtype)
    gi = upload_index(idx, dtype, dev)
    qm = synth.drift_queries(Q64, 6, 0.15, seed)
    qs = [synth.cast(qm[t], dtype, dev) for t in range(6)]
    return w, idx, gi, qs


def _needed(idx, sel, G):
    """Per step: the sorted block keys (bg * nblk + block) the zones of sel [B,Hq,k] touch."""
    B, Hkv = idx.sizes.shape[:2]
    nblk = -(-max(idx.Nc, 1) // BLK)
    keys = set()
    for b in range(B):
        for g in range(Hkv):
            off = idx.offsets[b, g]
            for c in np.unique(sel[b, g * G:(g + 1) * G]):
                if c < 0 or off[c + 1] == off[c]:
                    continue
                for blk in range(off[c] // BLK, (off[c + 1] - 1) // BLK + 1):
                    keys.add((b * Hkv + g) * nblk + blk)
    return sorted(keys)


def _lru_model(steps, capacity):
    """Per step (hits, staged, admitted, evicted).  The host decides from each step's log in step
    order: hits refresh their recency in key order, then every miss not cached since is admitted
    in key order into a free slot or over the least recently used block (a miss cached since only
    refreshes).  The device applies the decisions from step t at step t + 2, so the lookups of step
    t see the cache as decided through step t - 2."""
    host = OrderedDict()
    snaps = []
    out = []
    for t, keys in enumerate(steps):
        dev = snaps[t - 2] if t >= 2 else set()
        hits = [k for k in keys if k in dev]
        miss = [k for k in keys if k not in dev]
        adm = ev = 0
        for k in hits:
            if k in host:
                host.move_to_end(k)
        if capacity > 0:
            for k in miss:
                if k in host:
                    host.move_to_end(k)
                    continue
                if len(host) >= capacity:
                    host.popitem(last=False)
                    ev += 1
                host[k] = None
                adm += 1
        snaps.append(set(host))
        out.append((len(hits), len(miss), adm, ev))
    return out


def _run(w, idx, gi, qs, cache_blocks, exec_blocks, dtype):
    host = wi.with_host_kv(gi)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    wb = wi.WaveBuffer(host, w.B, w.Hq, w.Hkv, w.top_k, tdt, cache_blocks, exec_blocks)
    per_step = []
    prev = wb.stats()
    for q in qs:
        o1, l1, s1 = wb.decode(q)
        o2, l2, s2 = wi.decode(gi, q, w.top_k)
        torch.cuda.synchronize()
        # the oracle's decode on the same index, then the device-resident decode bit for bit
        ro, rl, rs = oracle.decode(synth.as_float64(q), idx, w.Hq, w.top_k)
        assert_decode_parity(o1, l1, s1, ro, rl, rs, dtype)
        assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(s1, s2)
        st = wb.stats()
        per_step.append({k: st[k] - prev[k] for k in st})
        prev = st
    wb.close()
    return per_step


def _oracle_steps(w, idx, qs):
    G = w.Hq // w.Hkv
    steps = []
    for q in qs:
        _, _, sel = oracle.decode(synth.as_float64(q), idx, w.Hq, w.top_k)
        steps.append(_needed(idx, sel, G))
    return steps


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_wavebuf_equals_device_decode_and_follows_lru(dtype):
    w, idx, gi, qs = _setup(dtype, 1)
    steps = _oracle_steps(w, idx, qs)
    most = max(len(s) for s in steps)
    for cache_blocks in (0, 40, 10_000):
        got = _run(w, idx, gi, qs, cache_blocks, most, dtype)
        want = _lru_model(steps, cache_blocks)
        for t, (g, (h, m, a, e)) in enumerate(zip(got, want)):
            assert (g["hits"], g["staged"], g["host_reads"], g["admitted"], g["evicted"]) == (h, m, 0, a, e), (cache_blocks, t)
            assert g["calls"] == 1


def test_wavebuf_repeated_query_hits_everything_from_the_third_step():
    # decisions from step t reach the device at step t + 2: steps 0 and 1 miss, 2 and 3 hit
    w, idx, gi, qs = _setup("bf16", 2)
    q = qs[0]
    got = _run(w, idx, gi, [q, q, q, q], 10_000, 10_000, "bf16")
    n = len(_oracle_steps(w, idx, [q])[0])
    assert [g["staged"] for g in got] == [n, n, 0, 0] and [g["hits"] for g in got] == [0, 0, n, n]
    assert [g["admitted"] for g in got] == [n, 0, 0, 0]


def test_wavebuf_full_execution_buffer_reads_host_memory_in_place():
    # 8 execution-buffer blocks: the rest of each step's misses are read over PCIe by the
    # attention kernel itself; which blocks those are depends on the order the zones are
    # resolved in, their number does not
    w, idx, gi, qs = _setup("bf16", 3)
    steps = _oracle_steps(w, idx, qs)
    got = _run(w, idx, gi, qs, 0, 8, "bf16")
    for g, keys in zip(got, steps):
        assert g["hits"] == 0 and g["staged"] == min(8, len(keys))
        assert g["host_reads"] == len(keys) - g["staged"] and g["admitted"] == 0
    got = _run(w, idx, gi, qs, 0, 0, "bf16")
    assert all(g["host_reads"] == len(k) for g, k in zip(got, steps))


def test_wavebuf_batch_and_many_heads():
    w, idx, gi, qs = _setup("bf16", 4, N=1536, Hq=16, Hkv=4, B=2, top_k=20)
    steps = _oracle_steps(w, idx, qs)
    most = max(len(s) for s in steps)
    got = _run(w, idx, gi, qs, 100, most, "bf16")
    want = _lru_model(steps, 100)
    for g, (h, m, a, e) in zip(got, want):
        assert (g["hits"], g["staged"], g["admitted"], g["evicted"]) == (h, m, a, e)


def test_wavebuf_back_to_back_steps_without_waiting():
    # the steps are enqueued without reading the counters in between (the host decides from each
    # log two calls later, as in a serving loop); every step's results and the totals
    w, idx, gi, qs = _setup("bf16", 5)
    steps = _oracle_steps(w, idx, qs)
    most = max(len(s) for s in steps)
    host = wi.with_host_kv(gi)
    wb = wi.WaveBuffer(host, w.B, w.Hq, w.Hkv, w.top_k, torch.bfloat16, 60, most)
    res = [wb.decode(q) for q in qs + qs]
    torch.cuda.synchronize()
    for q, (o1, l1, s1) in zip(qs + qs, res):
        ro, rl, rs = oracle.decode(synth.as_float64(q), idx, w.Hq, w.top_k)
        assert_decode_parity(o1, l1, s1, ro, rl, rs, "bf16")
        o2, l2, s2 = wi.decode(gi, q, w.top_k)
        assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(s1, s2)
    st = wb.stats()
    want = _lru_model(steps + steps, 60)
    assert st["calls"] == 2 * len(qs)
    assert (st["hits"], st["staged"], st["admitted"], st["evicted"]) == tuple(sum(x[i] for x in want) for i in range(4))
    wb.close()


def test_wavebuf_full_size_equals_device_decode():
    """The benchmarked shape (B=1, 32/8 heads, 128K, top 164 of 8192 clusters), the clustered K/V
    in pinned host memory and a cache of 30% of the blocks: five drifting steps, each equal to
    wi_decode on the device-resident index bit for bit; the third step onwards hits the cache."""
    from wi_testutil import inputs
    dev = device()
    w = synth.WORKLOADS["gqa_128k_bf16"]
    Kt, Vt, Qt, K64, V64, Q64, labels = inputs(w, 0, dev, with_labels=True)
    lo, hi = oracle.clustered_range(w.N, w.sink, w.window)
    lab = (np.arange(hi - lo) // w.seg_len) * w.clusters_per_seg + labels[:, :, lo:hi] % w.clusters_per_seg
    C = len(oracle.segment_bounds(hi - lo, w.seg_len)) * w.clusters_per_seg
    idx = oracle.finalize_index(K64, V64, lab, w.sink, w.window, C, w.dtype)
    gi = upload_index(idx, w.dtype, dev)
    nblk = -(-idx.Nc // BLK)
    host = wi.with_host_kv(gi)
    wb = wi.WaveBuffer(host, w.B, w.Hq, w.Hkv, w.top_k, torch.bfloat16, int(0.3 * w.Hkv * nblk),
                       w.Hq * w.top_k * 2)
    qm = synth.drift_queries(Q64, 5, 0.1, 3)
    prev = wb.stats()
    for t in range(5):
        q = synth.cast(qm[t], "bf16", dev)
        o1, l1, s1 = wb.decode(q)
        o2, l2, s2 = wi.decode(gi, q, w.top_k)
        torch.cuda.synchronize()
        ro, rl, rs = oracle.decode(synth.as_float64(q), idx, w.Hq, w.top_k)
        assert_decode_parity(o1, l1, s1, ro, rl, rs, "bf16")
        assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(s1, s2), t
        st = wb.stats()
        if t >= 2:
            assert st["hits"] - prev["hits"] > 0.5 * (st["hits"] - prev["hits"] + st["staged"] - prev["staged"])
        prev = st
    assert st["host_reads"] == 0
    wb.close()
