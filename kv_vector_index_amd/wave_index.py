"""Python binding of libwave_index.so (the C ABI declared in include/wave_index.h).

Argument marshalling only: every step of the build and of the decode runs in the HIP kernels of
the library.  torch supplies device memory and the HIP stream handle.  The binding fails loudly
when the library is missing; there is no fallback path.

Functions with the C names (``wi_index_shapes_for``, ``wi_build_index``,
``wi_decode_workspace_bytes``, ``wi_decode``, ``wi_status_string``, ``wi_last_error``) take and
return ctypes structures; ``build_index`` and ``decode`` wrap them for torch tensors.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwave_index.so")

WI_OK, WI_ERR_INVALID_ARG, WI_ERR_UNSUPPORTED, WI_ERR_WORKSPACE, WI_ERR_HIP = 0, -1, -2, -3, -4
WI_F32, WI_BF16 = 0, 1
EXPORTED = ("wi_index_shapes_for", "wi_build_index", "wi_index_append_segment",
            "wi_decode_workspace_bytes", "wi_decode", "wi_decode_noalloc", "wi_decode_gated",
            "wi_select_refresh", "wi_bound_data", "wi_decode_bounded", "wi_wavebuf_device_bytes", "wi_wavebuf_create",
            "wi_decode_wavebuf", "wi_wavebuf_stats", "wi_wavebuf_destroy",
            "wi_profile_enable", "wi_profile_rotate", "wi_profile_read", "wi_status_string", "wi_last_error")
STAGES = ("score", "select", "attend", "merge", "prep", "init", "assign", "rescore", "csr", "update",
          "final", "refresh")


class WaveIndexError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"wave-index status {status}: {detail}")
        self.status = status
        self.detail = detail


class BuildParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("N", ctypes.c_int32),
                ("d", ctypes.c_int32), ("sink", ctypes.c_int32), ("window", ctypes.c_int32),
                ("seg_len", ctypes.c_int32), ("clusters_per_seg", ctypes.c_int32),
                ("iters", ctypes.c_int32), ("dtype", ctypes.c_int32), ("seed", ctypes.c_uint64)]


class IndexView(ctypes.Structure):
    _fields_ = [("centroids", ctypes.c_void_p), ("value_sums", ctypes.c_void_p),
                ("sizes", ctypes.c_void_p), ("offsets", ctypes.c_void_p),
                ("perm", ctypes.c_void_p), ("k_perm", ctypes.c_void_p),
                ("v_perm", ctypes.c_void_p), ("k_steady", ctypes.c_void_p),
                ("v_steady", ctypes.c_void_p)]


class IndexShapes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "C", "Nc", "n_steady", "nseg", "centroids", "value_sums", "sizes", "offsets", "perm",
        "k_perm", "v_perm", "k_steady", "v_steady", "build_workspace_bytes")]


class DecodeParams(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("n_steady", ctypes.c_int32), ("C", ctypes.c_int32),
                ("Nc", ctypes.c_int32), ("top_k", ctypes.c_int32), ("scale", ctypes.c_float),
                ("dtype", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        L.wi_index_shapes_for.argtypes = [ctypes.POINTER(BuildParams), ctypes.POINTER(IndexShapes)]
        L.wi_build_index.argtypes = [ctypes.POINTER(BuildParams), vp, vp, ctypes.POINTER(IndexView),
                                     vp, sz, vp]
        L.wi_index_append_segment.argtypes = [ctypes.POINTER(BuildParams), vp, vp, ctypes.POINTER(IndexView),
                                              ctypes.POINTER(IndexView), vp, sz, vp]
        L.wi_decode_workspace_bytes.argtypes = [ctypes.POINTER(DecodeParams), ctypes.POINTER(sz)]
        L.wi_decode.argtypes = [ctypes.POINTER(DecodeParams), ctypes.POINTER(IndexView), vp, vp, vp,
                                vp, vp, sz, vp]
        L.wi_decode_noalloc.argtypes = [ctypes.POINTER(DecodeParams), ctypes.POINTER(IndexView), vp, vp, vp,
                                        vp, vp]
        L.wi_decode_gated.argtypes = [ctypes.POINTER(DecodeParams), ctypes.POINTER(IndexView), vp, vp, vp,
                                      ctypes.c_float, vp, vp, vp, vp, vp, sz, vp]
        L.wi_select_refresh.argtypes = [ctypes.POINTER(DecodeParams), ctypes.POINTER(IndexView), vp, vp, vp, sz,
                                        vp]
        L.wi_bound_data.argtypes = [ctypes.POINTER(DecodeParams), ctypes.POINTER(IndexView), vp, vp, vp, vp]
        L.wi_decode_bounded.argtypes = [ctypes.POINTER(DecodeParams), ctypes.POINTER(IndexView), vp, vp, vp, vp,
                                        ctypes.c_float, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.wi_wavebuf_device_bytes.argtypes = [ctypes.POINTER(DecodeParams), ctypes.c_int32, ctypes.c_int32,
                                              ctypes.POINTER(ctypes.c_size_t)]
        L.wi_wavebuf_create.argtypes = [ctypes.POINTER(DecodeParams), ctypes.c_int32, ctypes.c_int32, vp, sz, vp,
                                        ctypes.POINTER(ctypes.c_void_p)]
        L.wi_decode_wavebuf.argtypes = [vp, ctypes.POINTER(DecodeParams), ctypes.POINTER(IndexView), vp, vp, vp, vp,
                                        vp, sz, vp]
        L.wi_wavebuf_stats.argtypes = [vp, ctypes.POINTER(ctypes.c_int64)]
        L.wi_wavebuf_destroy.argtypes = [vp]
        L.wi_status_string.argtypes = [ctypes.c_int]
        L.wi_profile_enable.argtypes = [ctypes.c_int]
        L.wi_profile_enable.restype = ctypes.c_int
        L.wi_profile_rotate.argtypes = [ctypes.POINTER(IndexView), ctypes.c_int]
        L.wi_profile_rotate.restype = ctypes.c_int
        L.wi_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
        L.wi_profile_read.restype = ctypes.c_int
        for name in ("wi_index_shapes_for", "wi_build_index", "wi_index_append_segment",
                     "wi_decode_workspace_bytes", "wi_decode", "wi_decode_noalloc", "wi_decode_gated",
                     "wi_select_refresh", "wi_bound_data", "wi_decode_bounded", "wi_wavebuf_device_bytes",
                     "wi_wavebuf_create", "wi_decode_wavebuf", "wi_wavebuf_stats", "wi_wavebuf_destroy"):
            getattr(L, name).restype = ctypes.c_int
        L.wi_status_string.restype = ctypes.c_char_p
        L.wi_last_error.restype = ctypes.c_char_p
        L.wi_last_error.argtypes = []
        _lib = L
    return _lib


def wi_status_string(status: int) -> str:
    return lib().wi_status_string(int(status)).decode()


def wi_last_error() -> str:
    return lib().wi_last_error().decode()


def _check(status: int) -> int:
    if status != WI_OK:
        raise WaveIndexError(status, f"{wi_status_string(status)}: {wi_last_error()}")
    return status


def wi_index_shapes_for(p: BuildParams) -> IndexShapes:
    out = IndexShapes()
    _check(lib().wi_index_shapes_for(ctypes.byref(p), ctypes.byref(out)))
    return out


def wi_build_index(p: BuildParams, k_ptr: int, v_ptr: int, view: IndexView, ws_ptr: int,
                   ws_bytes: int, stream: int) -> int:
    return _check(lib().wi_build_index(ctypes.byref(p), k_ptr, v_ptr, ctypes.byref(view), ws_ptr,
                                       ws_bytes, stream))


def wi_index_append_segment(p: BuildParams, k_ptr: int, v_ptr: int, prev: IndexView, out: IndexView,
                            ws_ptr: int, ws_bytes: int, stream: int) -> int:
    return _check(lib().wi_index_append_segment(ctypes.byref(p), k_ptr, v_ptr, ctypes.byref(prev),
                                                ctypes.byref(out), ws_ptr, ws_bytes, stream))


def wi_decode_workspace_bytes(p: DecodeParams) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().wi_decode_workspace_bytes(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def wi_decode(p: DecodeParams, view: IndexView, q_ptr: int, out_ptr: int, lse_ptr: Optional[int],
              sel_ptr: Optional[int], ws_ptr: int, ws_bytes: int, stream: int) -> int:
    return _check(lib().wi_decode(ctypes.byref(p), ctypes.byref(view), q_ptr, out_ptr, lse_ptr,
                                  sel_ptr, ws_ptr, ws_bytes, stream))


def wi_decode_noalloc(p: DecodeParams, view: IndexView, q_ptr: int, out_ptr: int, lse_ptr: Optional[int],
                      sel_ptr: Optional[int], stream: int) -> int:
    return _check(lib().wi_decode_noalloc(ctypes.byref(p), ctypes.byref(view), q_ptr, out_ptr, lse_ptr,
                                          sel_ptr, stream))


def wi_decode_gated(p: DecodeParams, view: IndexView, q_ptr: int, q_prev_ptr: int, sel_prev_ptr: int,
                    tau: float, out_ptr: int, lse_ptr: Optional[int], sel_ptr: Optional[int],
                    reused_ptr: Optional[int], ws_ptr: int, ws_bytes: int, stream: int) -> int:
    return _check(lib().wi_decode_gated(ctypes.byref(p), ctypes.byref(view), q_ptr, q_prev_ptr, sel_prev_ptr,
                                        tau, out_ptr, lse_ptr, sel_ptr, reused_ptr, ws_ptr, ws_bytes, stream))


def wi_select_refresh(p: DecodeParams, view: IndexView, q_ptr: int, sel_ptr: Optional[int], ws_ptr: int,
                      ws_bytes: int, stream: int) -> int:
    return _check(lib().wi_select_refresh(ctypes.byref(p), ctypes.byref(view), q_ptr, sel_ptr, ws_ptr, ws_bytes,
                                          stream))


def wi_bound_data(p: DecodeParams, view: IndexView, radius_ptr: Optional[int], vnorm_ptr: Optional[int],
                  vmax_ptr: int, stream: int) -> int:
    return _check(lib().wi_bound_data(ctypes.byref(p), ctypes.byref(view), radius_ptr, vnorm_ptr, vmax_ptr, stream))


def wi_decode_bounded(p: DecodeParams, view: IndexView, radius_ptr: Optional[int], vnorm_ptr: Optional[int],
                      vmax_ptr: int, q_ptr: int, eps: float, out_ptr: int, lse_ptr: Optional[int],
                      sel_ptr: Optional[int], k_ptr: Optional[int], err_ptr: Optional[int],
                      n_exact_ptr: Optional[int], ws_ptr: int, ws_bytes: int, stream: int) -> int:
    return _check(lib().wi_decode_bounded(ctypes.byref(p), ctypes.byref(view), radius_ptr, vnorm_ptr, vmax_ptr,
                                          q_ptr, eps, out_ptr, lse_ptr, sel_ptr, k_ptr, err_ptr, n_exact_ptr, ws_ptr,
                                          ws_bytes, stream))


def wi_wavebuf_device_bytes(p: DecodeParams, cache_blocks: int, exec_blocks: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().wi_wavebuf_device_bytes(ctypes.byref(p), cache_blocks, exec_blocks, ctypes.byref(n)))
    return n.value


def wi_wavebuf_create(p: DecodeParams, cache_blocks: int, exec_blocks: int, mem_ptr: Optional[int], nbytes: int,
                      stream: int) -> int:
    h = ctypes.c_void_p(0)
    _check(lib().wi_wavebuf_create(ctypes.byref(p), cache_blocks, exec_blocks, mem_ptr, nbytes, stream, ctypes.byref(h)))
    return h.value


def wi_decode_wavebuf(handle: int, p: DecodeParams, view: IndexView, q_ptr: int, out_ptr: int, lse_ptr: Optional[int],
                      sel_ptr: Optional[int], ws_ptr: int, ws_bytes: int, stream: int) -> int:
    return _check(lib().wi_decode_wavebuf(handle, ctypes.byref(p), ctypes.byref(view), q_ptr, out_ptr, lse_ptr, sel_ptr,
                                          ws_ptr, ws_bytes, stream))


def wi_wavebuf_stats(handle: int) -> dict:
    st = (ctypes.c_int64 * 6)()
    _check(lib().wi_wavebuf_stats(handle, st))
    return dict(zip(("calls", "hits", "staged", "host_reads", "admitted", "evicted"), list(st)))


def wi_wavebuf_destroy(handle: int) -> int:
    return _check(lib().wi_wavebuf_destroy(handle))


def wi_profile_enable(enable, repeats: int = 1) -> int:
    """Turn the per-kernel timing hook on or off; with repeats > 1 every decode kernel is
    launched that many times back to back between its events."""
    return _check(lib().wi_profile_enable(max(1, int(repeats)) if enable else 0))


def wi_profile_rotate(views) -> int:
    """Rotation list of the profiling hook's repeats: IndexViews of bit-identical copies of the
    decoded index (an empty list clears it)."""
    arr = (IndexView * max(1, len(views)))(*views)
    return _check(lib().wi_profile_rotate(arr, len(views)))


def wi_profile_read() -> dict:
    """{stage name: (total kernel ms, launches)} accumulated since wi_profile_enable(True)."""
    n = len(STAGES)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check(lib().wi_profile_read(ms, cnt))
    return {STAGES[i]: (ms[i], cnt[i]) for i in range(n)}


# ---------------------------------------------------------------------------- torch convenience
def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return WI_BF16
    if t.dtype == torch.float32:
        return WI_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


@dataclasses.dataclass
class Index:
    """Device tensors of a built wave index (layouts as in include/wave_index.h)."""
    centroids: object
    value_sums: object
    sizes: object
    offsets: object
    perm: object
    k_perm: object
    v_perm: object
    k_steady: object
    v_steady: object
    C: int
    Nc: int
    n_steady: int

    def view(self) -> IndexView:
        return IndexView(*[_ptr(getattr(self, f)) for f in (
            "centroids", "value_sums", "sizes", "offsets", "perm", "k_perm", "v_perm",
            "k_steady", "v_steady")])

    def clone(self) -> "Index":
        return dataclasses.replace(self, **{f: getattr(self, f).clone() for f in (
            "centroids", "value_sums", "sizes", "offsets", "perm", "k_perm", "v_perm",
            "k_steady", "v_steady")})


def allocate_index(B: int, Hkv: int, N: int, sink: int, window: int, seg_len: int,
                   clusters_per_seg: int, dtype, device) -> tuple:
    """Index tensors (uninitialised) and the BuildParams skeleton for the given shape."""
    import torch
    p = BuildParams(B, Hkv, N, 128, sink, window, seg_len, clusters_per_seg, 1,
                    WI_BF16 if dtype == torch.bfloat16 else WI_F32, 0)
    sh = wi_index_shapes_for(p)
    C, Nc, NS = sh.C, sh.Nc, sh.n_steady
    e = dict(device=device)
    idx = Index(
        centroids=torch.empty((B, Hkv, C, 128), dtype=dtype, **e),
        value_sums=torch.empty((B, Hkv, C, 128), dtype=dtype, **e),
        sizes=torch.empty((B, Hkv, C), dtype=torch.int32, **e),
        offsets=torch.empty((B, Hkv, C + 1), dtype=torch.int32, **e),
        perm=torch.empty((B, Hkv, Nc), dtype=torch.int32, **e),
        k_perm=torch.empty((B, Hkv, Nc, 128), dtype=dtype, **e),
        v_perm=torch.empty((B, Hkv, Nc, 128), dtype=dtype, **e),
        k_steady=torch.empty((B, Hkv, NS, 128), dtype=dtype, **e),
        v_steady=torch.empty((B, Hkv, NS, 128), dtype=dtype, **e),
        C=C, Nc=Nc, n_steady=NS)
    return idx, p, sh


def build_index(K, V, sink: int, window: int, seg_len: int, clusters_per_seg: int, iters: int,
                seed: int, workspace=None) -> Index:
    """Build the wave index of K, V ([B,Hkv,N,128] device tensors, fp32 or bf16)."""
    import torch
    assert K.is_cuda and K.shape == V.shape and K.dtype == V.dtype and K.is_contiguous() and V.is_contiguous()
    B, Hkv, N, d = K.shape
    idx, p, sh = allocate_index(B, Hkv, N, sink, window, seg_len, clusters_per_seg, K.dtype, K.device)
    p.d = d
    p.iters = iters
    p.seed = seed & ((1 << 64) - 1)
    p.dtype = _dtype_code(K)
    need = max(int(sh.build_workspace_bytes), 256)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=K.device)
    wi_build_index(p, K.data_ptr(), V.data_ptr(), idx.view(), workspace.data_ptr(), workspace.numel(),
                   _stream(K.device))
    return idx


def append_segment(prev: Index, K, V, sink: int, window: int, seg_len: int, clusters_per_seg: int,
                   iters: int, seed: int, workspace=None) -> Index:
    """The index of K, V ([B,Hkv,N,128]) grown from `prev`, the index of their first N - seg_len
    tokens built with the same parameters: the tokens that left the window form one new segment."""
    import torch
    assert K.is_cuda and K.shape == V.shape and K.dtype == V.dtype and K.is_contiguous() and V.is_contiguous()
    B, Hkv, N, d = K.shape
    idx, p, sh = allocate_index(B, Hkv, N, sink, window, seg_len, clusters_per_seg, K.dtype, K.device)
    p.d = d
    p.iters = iters
    p.seed = seed & ((1 << 64) - 1)
    p.dtype = _dtype_code(K)
    need = max(int(sh.build_workspace_bytes), 256)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=K.device)
    wi_index_append_segment(p, K.data_ptr(), V.data_ptr(), prev.view(), idx.view(), workspace.data_ptr(),
                            workspace.numel(), _stream(K.device))
    return idx


def decode_params(index: Index, B: int, Hq: int, Hkv: int, top_k: int, dtype,
                  scale: Optional[float] = None) -> DecodeParams:
    import torch
    if scale is None:
        scale = 1.0 / math.sqrt(128)
    return DecodeParams(B, Hq, Hkv, 128, index.n_steady, index.C, index.Nc, top_k, scale,
                        WI_BF16 if dtype == torch.bfloat16 else WI_F32)


def decode(index: Index, q, top_k: int, scale: Optional[float] = None, workspace=None,
           want_lse: bool = True, want_sel: bool = True, out=None):
    """One decode step: q [B,Hq,128] -> (out fp32 [B,Hq,128], lse [B,Hq] or None, sel [B,Hq,k])."""
    import torch
    assert q.is_cuda and q.is_contiguous()
    B, Hq, d = q.shape
    Hkv = index.centroids.shape[1]
    p = decode_params(index, B, Hq, Hkv, top_k, q.dtype, scale)
    p.d = d
    p.dtype = _dtype_code(q)
    need = wi_decode_workspace_bytes(p)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if want_lse else None
    sel = torch.empty((B, Hq, top_k), dtype=torch.int32, device=q.device) if want_sel else None
    wi_decode(p, index.view(), q.data_ptr(), out.data_ptr(), _ptr(lse), _ptr(sel),
              workspace.data_ptr(), workspace.numel(), _stream(q.device))
    return out, lse, sel


def decode_gated(index: Index, q, q_prev, sel_prev, top_k: int, tau: float, scale: Optional[float] = None,
                 workspace=None, refresh: bool = False):
    """Decode step attending over sel_prev ([B,Hq,k] int32) for every KV head whose query heads
    all moved by a cosine >= tau.  Returns (out, lse, sel, reused [B,Hkv]): sel holds the zones
    attended over, or with refresh=True the top-k of q for every head (wi_select_refresh)."""
    import torch
    assert q.is_cuda and q.is_contiguous() and q_prev.shape == q.shape and q_prev.dtype == q.dtype
    assert q_prev.is_contiguous() and sel_prev.dtype == torch.int32 and sel_prev.is_contiguous()
    B, Hq, d = q.shape
    Hkv = index.centroids.shape[1]
    assert tuple(sel_prev.shape) == (B, Hq, top_k)
    p = decode_params(index, B, Hq, Hkv, top_k, q.dtype, scale)
    p.d = d
    p.dtype = _dtype_code(q)
    need = wi_decode_workspace_bytes(p)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    sel = torch.empty((B, Hq, top_k), dtype=torch.int32, device=q.device)
    reused = torch.empty((B, Hkv), dtype=torch.int32, device=q.device)
    view = index.view()
    wi_decode_gated(p, view, q.data_ptr(), q_prev.data_ptr(), sel_prev.data_ptr(), float(tau),
                    out.data_ptr(), lse.data_ptr(), sel.data_ptr(), reused.data_ptr(), workspace.data_ptr(),
                    workspace.numel(), _stream(q.device))
    if refresh:
        wi_select_refresh(p, view, q.data_ptr(), sel.data_ptr(), workspace.data_ptr(), workspace.numel(),
                          _stream(q.device))
    return out, lse, sel, reused


def bound_data(index: Index, B: int, Hkv: int, dtype):
    """Radius [B,Hkv,C], value norms [B,Hkv,C] and largest value norm [B,Hkv] (float32) of an
    index: the per-cluster data of the estimation error bound."""
    import torch
    dev = index.centroids.device
    p = decode_params(index, B, Hkv, Hkv, 0, dtype)
    p.d = index.centroids.shape[-1]
    p.dtype = WI_BF16 if dtype == torch.bfloat16 else WI_F32
    radius = torch.empty((B, Hkv, index.C), dtype=torch.float32, device=dev)
    vnorm = torch.empty((B, Hkv, index.C), dtype=torch.float32, device=dev)
    vmax = torch.empty((B, Hkv), dtype=torch.float32, device=dev)
    wi_bound_data(p, index.view(), _ptr(radius) if index.C else None, _ptr(vnorm) if index.C else None,
                  vmax.data_ptr(), _stream(dev))
    return radius, vnorm, vmax


def decode_bounded(index: Index, q, bound, top_k: int, eps: float, scale: Optional[float] = None,
                   workspace=None, n_exact=None):
    """Decode with the zone of each head sized to meet an error bound eps; ``bound`` is the
    (radius, vnorm, vmax) of bound_data.  Returns (out, lse, sel, k_used [B,Hq], err_bound [B,Hq]).
    ``n_exact``, a one-element int32 device tensor, counts the heads that decided in fp64."""
    import torch
    assert q.is_cuda and q.is_contiguous()
    B, Hq, d = q.shape
    Hkv = index.centroids.shape[1]
    radius, vnorm, vmax = bound
    p = decode_params(index, B, Hq, Hkv, top_k, q.dtype, scale)
    p.d = d
    p.dtype = _dtype_code(q)
    need = wi_decode_workspace_bytes(p)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    sel = torch.empty((B, Hq, top_k), dtype=torch.int32, device=q.device)
    k_used = torch.empty((B, Hq), dtype=torch.int32, device=q.device)
    err = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    wi_decode_bounded(p, index.view(), _ptr(radius) if index.C else None, _ptr(vnorm) if index.C else None,
                      vmax.data_ptr(), q.data_ptr(), float(eps), out.data_ptr(), lse.data_ptr(), _ptr(sel),
                      k_used.data_ptr(), err.data_ptr(), None if n_exact is None else n_exact.data_ptr(),
                      workspace.data_ptr(), workspace.numel(), _stream(q.device))
    return out, lse, sel, k_used, err


WB_BLOCK = 16   # rows per wave-buffer block


def with_host_kv(index: Index) -> Index:
    """The same index with its cluster-major K/V copies moved to pinned host memory."""
    import torch
    hk = torch.empty(index.k_perm.shape, dtype=index.k_perm.dtype, pin_memory=True)
    hv = torch.empty(index.v_perm.shape, dtype=index.v_perm.dtype, pin_memory=True)
    hk.copy_(index.k_perm)
    hv.copy_(index.v_perm)
    return Index(centroids=index.centroids, value_sums=index.value_sums, sizes=index.sizes, offsets=index.offsets,
                 perm=index.perm, k_perm=hk, v_perm=hv, k_steady=index.k_steady, v_steady=index.v_steady,
                 C=index.C, Nc=index.Nc, n_steady=index.n_steady)


class WaveBuffer:
    """A GPU block cache and execution buffer over an index whose K/V copies are in host memory
    (with_host_kv).  decode() runs wi_decode_wavebuf; stats() returns the running counters."""

    def __init__(self, index: Index, B: int, Hq: int, Hkv: int, top_k: int, dtype, cache_blocks: int,
                 exec_blocks: int, device=None):
        import torch
        self.index = index
        self.device = device if device is not None else index.centroids.device
        self.p = decode_params(index, B, Hq, Hkv, top_k, dtype)
        nbytes = wi_wavebuf_device_bytes(self.p, cache_blocks, exec_blocks)
        self.mem = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        self.handle = wi_wavebuf_create(self.p, cache_blocks, exec_blocks, self.mem.data_ptr(), self.mem.numel(),
                                        _stream(self.device))
        self.view = index.view()
        self.ws = torch.empty(max(wi_decode_workspace_bytes(self.p), 256), dtype=torch.uint8, device=self.device)

    def decode(self, q, out=None, lse=None, sel=None):
        import torch
        B, Hq, d = q.shape
        if out is None:
            out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
        if lse is None:
            lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
        if sel is None:
            sel = torch.empty((B, Hq, self.p.top_k), dtype=torch.int32, device=q.device)
        wi_decode_wavebuf(self.handle, self.p, self.view, q.data_ptr(), out.data_ptr(), lse.data_ptr(), _ptr(sel),
                          self.ws.data_ptr(), self.ws.numel(), _stream(q.device))
        return out, lse, sel

    def stats(self) -> dict:
        return wi_wavebuf_stats(self.handle)

    def close(self):
        if self.handle:
            wi_wavebuf_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
