"""Seeded synthetic inputs for the wave index: blob-mixture keys, Gaussian values, shifted queries.

This module only draws random numbers and casts them to the storage dtype. It holds none of the
wave-index arithmetic (no clustering, scoring, selection or attention), so the HIP path and the CPU
oracle can both consume what it produces without sharing any of the method.

Workload shape follows the pages' setting: one attention layer of an 8B-class GQA model (32 query
heads, 8 KV heads, head dim 128) at 128K and 1M tokens of context [RetroInfer technical summary
(gist.science, es), section 4; RetrievalAttention abstract (scholarfeed)]. Query vectors are drawn
off the key distribution on purpose: the RetrievalAttention abstract reports that attention queries
are out-of-distribution with respect to keys, which is what breaks off-the-shelf ANN indexes.

Recipe (all draws in float64 from ``numpy.random.default_rng(SeedSequence([seed, b, g]))``):
  * blob centres   : [n_blobs, d] ~ N(0, 1)
  * token labels   : i.i.d. uniform over the blobs (no positional locality)
  * keys           : centre[label] + key_noise * N(0, I), then scaled to unit length
  * values         : N(0, 1)
  * queries        : q_scale * centre[u] + q_noise * N(0, I), u uniform, one draw per query head
  * drifting steps : q_{t+1} = q_t + drift * N(0, I), kept in a float64 master copy
All "N(0, s)" parameters are standard deviations.  Casting to bf16 goes float64 -> float32 -> bf16,
each step round-to-nearest-even (torch's conversion).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "blob_mixture_head", "make_instance", "drift_queries",
           "cast", "as_float64", "make_instance_device", "drift_queries_device"]


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and generator parameters of one synthetic decode / build workload."""
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    N: int
    dtype: str                 # "f32" or "bf16"
    n_blobs: int
    sink: int
    window: int
    seg_len: int               # 0 = one segment over the clustered range
    clusters_per_seg: int
    iters: int
    top_k: int                 # clusters retrieved per query head
    steps: int = 1
    drift: float = 0.0
    q_scale: float = 1.5
    q_noise: float = 0.5
    key_noise: float = 0.3

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# k for the fractional configurations is ceil(fraction * total clusters):
#   128K: 16 segments x 512 clusters = 8192, 2%  -> 164
#   1M  : 128 segments x 512 clusters = 65536, 1% -> 656
WORKLOADS = {
    # single head, fp32, 8192 keys from 64 blobs, one segment of 64 clusters, top 8
    "single_head_8k_f32": Workload("single_head_8k_f32", 1, 1, 1, 128, 8192, "f32", 64,
                                   4, 256, 0, 64, 10, 8),
    # Llama-3-8B-shaped GQA layer, batch 1, 128K context
    "gqa_128k_bf16": Workload("gqa_128k_bf16", 1, 32, 8, 128, 131072, "bf16", 4096,
                              4, 64, 8192, 512, 10, 164),
    # same layer, batch 16, 100 drifting decode steps
    "gqa_128k_b16_bf16": Workload("gqa_128k_b16_bf16", 16, 32, 8, 128, 131072, "bf16", 4096,
                                  4, 64, 8192, 512, 10, 164, steps=100, drift=0.1),
    # million-token context
    "gqa_1m_bf16": Workload("gqa_1m_bf16", 1, 32, 8, 128, 1048576, "bf16", 65536,
                            4, 64, 8192, 512, 10, 656),
    # index build only (no steady zone)
    "build_128k_bf16": Workload("build_128k_bf16", 1, 32, 8, 128, 131072, "bf16", 4096,
                                0, 0, 8192, 512, 10, 0),
}


def _rng(seed: int, b: int, g: int, stream: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(b), int(g), int(stream)]))


def blob_mixture_head(n: int, d: int, n_blobs: int, rng: np.random.Generator,
                      key_noise: float = 0.3):
    """Keys/values of one (sequence, KV head): returns (K, V, centres, labels), float64."""
    centres = rng.standard_normal((n_blobs, d))
    labels = rng.integers(0, n_blobs, size=n)
    K = centres[labels]
    K += key_noise * rng.standard_normal((n, d))
    K /= np.linalg.norm(K, axis=1, keepdims=True)
    V = rng.standard_normal((n, d))
    return K, V, centres, labels


def make_instance(w: Workload, seed: int = 0, n_override: Optional[int] = None,
                  with_labels: bool = False):
    """Draw K, V [B,Hkv,N,d] and q [B,Hq,d] (float64) for workload ``w``.

    Each (b, g) has its own blob mixture; each query head of group g picks its own blob centre.
    """
    N = w.N if n_override is None else int(n_override)
    G = w.Hq // w.Hkv
    K = np.empty((w.B, w.Hkv, N, w.d))
    V = np.empty((w.B, w.Hkv, N, w.d))
    Q = np.empty((w.B, w.Hq, w.d))
    labels = np.empty((w.B, w.Hkv, N), dtype=np.int64) if with_labels else None
    for b in range(w.B):
        for g in range(w.Hkv):
            rng = _rng(seed, b, g)
            k, v, centres, lab = blob_mixture_head(N, w.d, w.n_blobs, rng, w.key_noise)
            K[b, g], V[b, g] = k, v
            if with_labels:
                labels[b, g] = lab
            for j in range(G):
                u = rng.integers(0, w.n_blobs)
                Q[b, g * G + j] = w.q_scale * centres[u] + w.q_noise * rng.standard_normal(w.d)
    if with_labels:
        return K, V, Q, labels
    return K, V, Q


def drift_queries(q0: np.ndarray, steps: int, drift: float, seed: int = 0) -> np.ndarray:
    """[steps, *q0.shape] float64 master copies: q_0 = q0, q_{t+1} = q_t + drift * N(0, I)."""
    rng = _rng(seed, 1 << 20, 0, 7)
    out = np.empty((steps,) + q0.shape)
    out[0] = q0
    for t in range(1, steps):
        out[t] = out[t - 1] + drift * rng.standard_normal(q0.shape)
    return out


def cast(x: np.ndarray, dtype: str, device=None):
    """float64 numpy -> torch tensor of the storage dtype (f32, or bf16 through f32)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return t if device is None else t.to(device)


def _device_generator(device, seed: int, b: int, g: int, stream: int = 0):
    import torch
    key = np.random.SeedSequence([int(seed), int(b), int(g), int(stream)]).generate_state(1, np.uint64)[0]
    gen = torch.Generator(device=device)
    gen.manual_seed(int(key) & ((1 << 63) - 1))
    return gen


def make_instance_device(w: Workload, seed: int, device, n_override: Optional[int] = None):
    """The same recipe as make_instance, drawn on the device with torch's generator (a different
    random stream, so not the same numbers): K, V [B,Hkv,N,d] and q [B,Hq,d] in the storage
    dtype.  For throughput runs whose sizes make host-side float64 generation slow; parity tests
    use make_instance."""
    import torch
    N = w.N if n_override is None else int(n_override)
    G = w.Hq // w.Hkv
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    K = torch.empty((w.B, w.Hkv, N, w.d), dtype=tdt, device=device)
    V = torch.empty_like(K)
    Q = torch.empty((w.B, w.Hq, w.d), dtype=tdt, device=device)
    chunk = 1 << 16
    for b in range(w.B):
        for g in range(w.Hkv):
            gen = _device_generator(device, seed, b, g)
            centres = torch.randn((w.n_blobs, w.d), generator=gen, device=device, dtype=torch.float64)
            for t0 in range(0, N, chunk):
                n = min(chunk, N - t0)
                lab = torch.randint(0, w.n_blobs, (n,), generator=gen, device=device)
                k = centres[lab] + w.key_noise * torch.randn((n, w.d), generator=gen, device=device,
                                                             dtype=torch.float64)
                k /= torch.linalg.vector_norm(k, dim=1, keepdim=True)
                K[b, g, t0:t0 + n] = k.to(torch.float32).to(tdt)
                v = torch.randn((n, w.d), generator=gen, device=device, dtype=torch.float64)
                V[b, g, t0:t0 + n] = v.to(torch.float32).to(tdt)
            u = torch.randint(0, w.n_blobs, (G,), generator=gen, device=device)
            q = w.q_scale * centres[u] + w.q_noise * torch.randn((G, w.d), generator=gen, device=device,
                                                                 dtype=torch.float64)
            Q[b, g * G:(g + 1) * G] = q.to(torch.float32).to(tdt)
    return K, V, Q


def drift_queries_device(q0, steps: int, drift: float, seed: int = 0):
    """[steps, *q0.shape] float64 device master copies: q_0 = q0, q_{t+1} = q_t + drift * N(0, I)."""
    import torch
    gen = _device_generator(q0.device, seed, 1 << 20, 0, 7)
    out = torch.empty((steps,) + tuple(q0.shape), dtype=torch.float64, device=q0.device)
    out[0] = q0.to(torch.float64)
    for t in range(1, steps):
        out[t] = out[t - 1] + drift * torch.randn(tuple(q0.shape), generator=gen, device=q0.device,
                                                  dtype=torch.float64)
    return out


def as_float64(t) -> np.ndarray:
    """torch tensor (any device, f32/bf16) -> float64 numpy holding exactly the stored values."""
    return t.detach().to("cpu").to(__import__("torch").float64).numpy()


assert math.ceil(0.02 * 8192) == 164 and math.ceil(0.01 * 65536) == 656
