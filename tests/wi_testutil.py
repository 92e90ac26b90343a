"""Helpers shared by the GPU parity tests: moving oracle-built indexes to the device and the
parity gates (bit-exact ids and sizes; output tolerances of the decode)."""
import math

import numpy as np
import torch

import oracle
from kv_vector_index_amd import synth
from kv_vector_index_amd import wave_index as wi

# Output gates: max |o - oracle| <= 1e-4 for fp32 inputs, 1e-2 for bf16 inputs (fp32 accumulation);
# in addition |lse - oracle| <= 1e-4 and relative RMS error of o <= 1e-3 for both.
O_TOL = {"f32": 1e-4, "bf16": 1e-2}
LSE_TOL = 1e-4
REL_RMS_TOL = 1e-3


def device():
    assert torch.cuda.is_available(), "GPU test without a GPU"
    return torch.device("cuda:0")


def inputs(w, seed, dev, n_override=None, with_labels=False):
    """Seeded K, V, Q cast to the storage dtype on `dev`, and their exact float64 copies."""
    r = synth.make_instance(w, seed, n_override=n_override, with_labels=with_labels)
    K, V, Q = r[:3]
    Kt, Vt, Qt = (synth.cast(x, w.dtype, dev) for x in (K, V, Q))
    K64, V64, Q64 = (synth.as_float64(t) for t in (Kt, Vt, Qt))
    out = (Kt, Vt, Qt, K64, V64, Q64)
    return out + (r[3],) if with_labels else out


def upload_index(idx: oracle.Index, dtype: str, dev) -> wi.Index:
    """An oracle-built index as device tensors (values are exactly representable in dtype)."""
    cast = lambda a: synth.cast(a, dtype, dev)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a).astype(np.int32)).to(dev)
    return wi.Index(centroids=cast(idx.centroids), value_sums=cast(idx.value_sums),
                    sizes=i32(idx.sizes), offsets=i32(idx.offsets), perm=i32(idx.perm),
                    k_perm=cast(idx.k_perm), v_perm=cast(idx.v_perm),
                    k_steady=cast(idx.k_steady), v_steady=cast(idx.v_steady),
                    C=idx.C, Nc=idx.Nc, n_steady=idx.k_steady.shape[2])


def assert_decode_parity(o, lse, sel, ro, rl, rs, dtype, heads=None):
    """o/lse/sel: device results; ro/rl/rs: oracle results (optionally for a subset of heads,
    given as a list of (b, h))."""
    o = o.detach().cpu().numpy().astype(np.float64)
    lse = lse.detach().cpu().numpy().astype(np.float64)
    sel = sel.detach().cpu().numpy().astype(np.int64)
    if heads is not None:
        o = np.stack([o[b, h] for b, h in heads])
        lse = np.array([lse[b, h] for b, h in heads])
        sel = np.stack([sel[b, h] for b, h in heads])
    np.testing.assert_array_equal(sel, rs)
    err = float(np.abs(o - ro).max())
    assert err <= O_TOL[dtype], f"max |o - oracle| = {err}"
    lerr = float(np.abs(lse - rl).max())
    assert lerr <= LSE_TOL, f"max |lse - oracle| = {lerr}"
    rms = math.sqrt(float(np.mean((o - ro) ** 2))) / max(math.sqrt(float(np.mean(ro ** 2))), 1e-30)
    assert rms <= REL_RMS_TOL, f"relative RMS error {rms}"
    return err, lerr, rms


def index_to_numpy(idx: wi.Index):
    f = lambda t: t.detach().cpu().to(torch.float64).numpy() if t.is_floating_point() else t.detach().cpu().numpy().astype(np.int64)
    return {k: f(getattr(idx, k)) for k in ("centroids", "value_sums", "sizes", "offsets", "perm",
                                            "k_perm", "v_perm", "k_steady", "v_steady")}
