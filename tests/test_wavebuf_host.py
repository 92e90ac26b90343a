"""The wave buffer's cache policy on the host alone: the library's LRU (csrc/wi_lru.h), compiled
with g++ into a small shim that emulates the device side of the protocol (decisions applied two
calls later, misses staged while the execution buffer has room, every hit checked to read a slot
that holds its block), against an independent model of the policy on random block streams."""
import ctypes
import os
import shutil
import subprocess
from collections import OrderedDict

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def shim(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("shim") / "libwbshim.so")
    subprocess.run([gxx, "-O2", "-std=c++17", "-shared", "-fPIC", "-I", os.path.join(ROOT, "kv_vector_index_amd", "csrc"),
                    os.path.join(ROOT, "tests", "wavebuf_protocol_shim.cpp"), "-o", out], check=True)
    lib = ctypes.CDLL(out)
    lib.wb_protocol.restype = ctypes.c_int
    return lib


def _model(steps, cache, exec_blocks):
    """Per step (hits, staged, host reads, admitted, evicted): lookups see the decisions through
    step t - 2; misses are staged in resolve order while the execution buffer has room; the host
    refreshes hits still cached (key order), then admits staged misses not cached yet (key order)
    into a free slot or over the least recently used one."""
    host = OrderedDict()
    snaps = []
    out = []
    for t, keys in enumerate(steps):
        dev = snaps[t - 2] if t >= 2 else set()
        hits = [k for k in keys if k in dev]
        miss = [k for k in keys if k not in dev]
        staged, reads = miss[:exec_blocks], miss[exec_blocks:]
        adm = ev = 0
        for k in sorted(hits):
            if k in host:
                host.move_to_end(k)
        if cache > 0:
            for k in sorted(staged):
                if k in host:
                    host.move_to_end(k)
                    continue
                if len(host) >= cache:
                    host.popitem(last=False)
                    ev += 1
                host[k] = None
                adm += 1
        snaps.append(set(host))
        out.append((len(hits), len(staged), len(reads), adm, ev))
    return out


def _streams(seed, n_keys=600, n_steps=40, width=120):
    """Blocks of a drifting window (the temporal locality the cache exploits), a few far jumps,
    each step in a random resolve order."""
    rng = np.random.default_rng(seed)
    steps = []
    centre = n_keys // 2
    for t in range(n_steps):
        centre = int(np.clip(centre + rng.integers(-15, 16), width, n_keys - width))
        if t % 13 == 7:
            centre = int(rng.integers(width, n_keys - width))
        cand = np.arange(centre - width, centre + width)
        keys = rng.choice(cand, size=int(rng.integers(40, 140)), replace=False)
        steps.append([int(k) for k in keys])
    return n_keys, steps


@pytest.mark.parametrize("cache,exec_blocks", [(0, 200), (16, 200), (60, 200), (1000, 200), (60, 30), (500, 0)])
@pytest.mark.parametrize("seed", [1, 2])
def test_policy_matches_the_model_and_hits_read_their_blocks(shim, cache, exec_blocks, seed):
    n_keys, steps = _streams(seed)
    off = np.concatenate([[0], np.cumsum([len(s) for s in steps])]).astype(np.int32)
    keys = np.concatenate([np.array(s, dtype=np.int32) for s in steps])
    out = np.zeros((len(steps), 5), dtype=np.int64)
    rc = shim.wb_protocol(cache, exec_blocks, n_keys, len(steps), off.ctypes.data_as(ctypes.c_void_p),
                          keys.ctypes.data_as(ctypes.c_void_p), out.ctypes.data_as(ctypes.c_void_p))
    assert rc == 0, f"step {-rc - 1}: a hit's slot did not hold its block"
    want = _model(steps, cache, exec_blocks)
    for t, (g, w) in enumerate(zip(out.tolist(), want)):
        assert tuple(g) == w, (t, g, w)
    if cache >= 1000 and exec_blocks >= 200:
        assert sum(w[0] for w in want) > 0.5 * sum(len(s) for s in steps)   # locality pays off


def test_a_batch_that_refills_a_slot_keeps_the_directory_consistent(shim):
    # a 4-block cache and 40 misses a step: every batch evicts its own admissions and, with keys
    # revisited, re-admits blocks it evicted a moment before (the case that needs one directory
    # update per key); every hit must still read its own block
    rng = np.random.default_rng(9)
    steps = [[int(k) for k in rng.permutation(np.arange(t % 3 * 10, t % 3 * 10 + 40))] for t in range(30)]
    off = np.concatenate([[0], np.cumsum([len(s) for s in steps])]).astype(np.int32)
    keys = np.concatenate([np.array(s, dtype=np.int32) for s in steps])
    out = np.zeros((len(steps), 5), dtype=np.int64)
    rc = shim.wb_protocol(4, 64, 80, len(steps), off.ctypes.data_as(ctypes.c_void_p),
                          keys.ctypes.data_as(ctypes.c_void_p), out.ctypes.data_as(ctypes.c_void_p))
    assert rc == 0
    assert [tuple(r) for r in out.tolist()] == _model(steps, 4, 64)
