"""CPU checks of the C ABI: the library loads, exports every declared symbol, its structs match
the header's layout, and host-side validation rejects bad arguments before anything is launched."""
import ctypes
import os
import re
import subprocess

import pytest

from kv_vector_index_amd import wave_index as wi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wave_index.h")


def _declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(wi_[a-z_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert set(names) == set(wi.EXPORTED)
    L = wi.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", wi.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (wi_[a-z_]+)\b", out))
    assert set(names) <= exported


def test_struct_layouts_match_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(r'''
#include <stdio.h>
#include <stddef.h>
#include "wave_index.h"
#define P(T, f) printf(#T "." #f " %zu\n", offsetof(T, f))
int main(void) {
  printf("wi_build_params %zu\n", sizeof(wi_build_params));
  printf("wi_index_view %zu\n", sizeof(wi_index_view));
  printf("wi_index_shapes %zu\n", sizeof(wi_index_shapes));
  printf("wi_decode_params %zu\n", sizeof(wi_decode_params));
  P(wi_build_params, seed); P(wi_build_params, dtype); P(wi_build_params, iters);
  P(wi_index_view, v_steady); P(wi_index_shapes, build_workspace_bytes);
  P(wi_decode_params, scale); P(wi_decode_params, dtype); P(wi_decode_params, top_k);
  return 0;
}''')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = dict(l.rsplit(" ", 1) for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                        check=True).stdout.splitlines())
    assert int(got["wi_build_params"]) == ctypes.sizeof(wi.BuildParams)
    assert int(got["wi_index_view"]) == ctypes.sizeof(wi.IndexView)
    assert int(got["wi_index_shapes"]) == ctypes.sizeof(wi.IndexShapes)
    assert int(got["wi_decode_params"]) == ctypes.sizeof(wi.DecodeParams)
    assert int(got["wi_build_params.seed"]) == wi.BuildParams.seed.offset
    assert int(got["wi_build_params.dtype"]) == wi.BuildParams.dtype.offset
    assert int(got["wi_build_params.iters"]) == wi.BuildParams.iters.offset
    assert int(got["wi_index_view.v_steady"]) == wi.IndexView.v_steady.offset
    assert int(got["wi_index_shapes.build_workspace_bytes"]) == wi.IndexShapes.build_workspace_bytes.offset
    assert int(got["wi_decode_params.scale"]) == wi.DecodeParams.scale.offset
    assert int(got["wi_decode_params.dtype"]) == wi.DecodeParams.dtype.offset
    assert int(got["wi_decode_params.top_k"]) == wi.DecodeParams.top_k.offset


@pytest.mark.parametrize("N,S,W,L,Cs,want", [
    (8192, 4, 256, 0, 64, dict(C=64, Nc=7932, n_steady=260, nseg=1)),
    (131072, 4, 64, 8192, 512, dict(C=8192, Nc=131004, n_steady=68, nseg=16)),
    (1048576, 4, 64, 8192, 512, dict(C=65536, Nc=1048508, n_steady=68, nseg=128)),
    (131072, 0, 0, 8192, 512, dict(C=8192, Nc=131072, n_steady=0, nseg=16)),
    (50, 30, 30, 8, 4, dict(C=0, Nc=0, n_steady=50, nseg=0)),
    (100, 10, 10, 30, 7, dict(C=21, Nc=80, n_steady=20, nseg=3)),
])
def test_index_shapes(N, S, W, L, Cs, want):
    p = wi.BuildParams(2, 8, N, 128, S, W, L, Cs, 10, wi.WI_BF16, 0)
    sh = wi.wi_index_shapes_for(p)
    for k, v in want.items():
        assert getattr(sh, k) == v, k
    BG = 16
    assert sh.centroids == BG * want["C"] * 128 and sh.offsets == BG * (want["C"] + 1)
    assert sh.perm == BG * want["Nc"] and sh.k_steady == BG * want["n_steady"] * 128
    # per clustered key: its assignment and a slot of the uncertain-key list (int32 each), plus
    # the bf16 centroid directions
    assert sh.build_workspace_bytes >= BG * want["Nc"] * 8 + BG * want["C"] * 128 * 2


@pytest.mark.parametrize("field,value,status", [
    ("d", 64, wi.WI_ERR_UNSUPPORTED), ("B", 0, wi.WI_ERR_INVALID_ARG),
    ("N", 0, wi.WI_ERR_INVALID_ARG), ("seg_len", 70000, wi.WI_ERR_UNSUPPORTED),
    ("clusters_per_seg", 5000, wi.WI_ERR_UNSUPPORTED), ("clusters_per_seg", 0, wi.WI_ERR_INVALID_ARG),
    ("iters", 0, wi.WI_ERR_INVALID_ARG), ("dtype", 7, wi.WI_ERR_INVALID_ARG),
    ("sink", -1, wi.WI_ERR_INVALID_ARG),
])
def test_shapes_rejects(field, value, status):
    p = wi.BuildParams(1, 8, 131072, 128, 4, 64, 8192, 512, 10, wi.WI_BF16, 0)
    setattr(p, field, value)
    with pytest.raises(wi.WaveIndexError) as e:
        wi.wi_index_shapes_for(p)
    assert e.value.status == status
    assert wi.wi_last_error()


FAKE = 0x7f0000000000  # never dereferenced: every call below fails validation first


def _view():
    return wi.IndexView(*([FAKE] * 9))


def _bparams(**kw):
    # 4 sink + 64 window + 3 segments of 1024 tokens, 64 clusters each
    p = wi.BuildParams(1, 8, 4 + 64 + 3 * 1024, 128, 4, 64, 1024, 64, 10, wi.WI_BF16, 0)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("kw", [dict(N=4 + 64 + 3 * 1024 + 100), dict(seg_len=0), dict(N=40)])
def test_append_segment_rejects_ranges_that_are_not_whole_segments(kw):
    # a clustered range that is not a positive multiple of seg_len (ragged, one implicit segment,
    # or empty) has no previous index of full segments to grow from
    with pytest.raises(wi.WaveIndexError) as e:
        wi.wi_index_append_segment(_bparams(**kw), FAKE, FAKE, _view(), _view(), FAKE, 1 << 40, 0)
    assert e.value.status == wi.WI_ERR_INVALID_ARG


def test_append_segment_rejects_null_overlap_and_small_workspace():
    p = _bparams()
    apart = wi.IndexView(*([FAKE + (1 << 38)] * 9))
    with pytest.raises(wi.WaveIndexError) as e:       # null key rows
        wi.wi_index_append_segment(p, None, FAKE, _view(), apart, FAKE, 1 << 40, 0)
    assert e.value.status == wi.WI_ERR_INVALID_ARG
    prev = _view()
    prev.k_perm = None
    with pytest.raises(wi.WaveIndexError) as e:       # the previous index must be complete
        wi.wi_index_append_segment(p, FAKE, FAKE, prev, apart, FAKE, 1 << 40, 0)
    assert e.value.status == wi.WI_ERR_INVALID_ARG
    with pytest.raises(wi.WaveIndexError) as e:       # same buffers on both sides
        wi.wi_index_append_segment(p, FAKE, FAKE, _view(), _view(), FAKE, 1 << 40, 0)
    assert e.value.status == wi.WI_ERR_INVALID_ARG
    need = int(wi.wi_index_shapes_for(p).build_workspace_bytes)
    with pytest.raises(wi.WaveIndexError) as e:
        wi.wi_index_append_segment(p, FAKE, FAKE, _view(), apart, FAKE, need - 1, 0)
    assert e.value.status == wi.WI_ERR_WORKSPACE


def _dparams(**kw):
    p = wi.DecodeParams(1, 32, 8, 128, 68, 8192, 131004, 164, 0.0883883, wi.WI_BF16)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("kw,status", [
    (dict(d=64), wi.WI_ERR_UNSUPPORTED), (dict(Hq=12), wi.WI_ERR_INVALID_ARG),
    (dict(Hq=24), wi.WI_ERR_UNSUPPORTED), (dict(top_k=-1), wi.WI_ERR_INVALID_ARG),
    (dict(C=0), wi.WI_ERR_INVALID_ARG), (dict(scale=0.0), wi.WI_ERR_INVALID_ARG),
    (dict(n_steady=0, C=0, Nc=0), wi.WI_ERR_INVALID_ARG), (dict(dtype=3), wi.WI_ERR_INVALID_ARG),
])
def test_decode_rejects_bad_params(kw, status):
    p = _dparams(**kw)
    with pytest.raises(wi.WaveIndexError) as e:
        wi.wi_decode(p, _view(), FAKE, FAKE, None, None, FAKE, 1 << 40, 0)
    assert e.value.status == status


def test_decode_rejects_null_pointers_and_small_workspace():
    p = _dparams()
    need = wi.wi_decode_workspace_bytes(p)
    assert need > 0
    with pytest.raises(wi.WaveIndexError) as e:
        wi.wi_decode(p, _view(), None, FAKE, None, None, FAKE, need, 0)
    assert e.value.status == wi.WI_ERR_INVALID_ARG
    v = _view()
    v.k_perm = None
    with pytest.raises(wi.WaveIndexError) as e:
        wi.wi_decode(p, v, FAKE, FAKE, None, None, FAKE, need, 0)
    assert e.value.status == wi.WI_ERR_INVALID_ARG
    with pytest.raises(wi.WaveIndexError) as e:
        wi.wi_decode(p, _view(), FAKE, FAKE, None, None, FAKE, need - 1, 0)
    assert e.value.status == wi.WI_ERR_WORKSPACE
    with pytest.raises(wi.WaveIndexError) as e:
        wi.wi_decode(p, _view(), FAKE, FAKE, None, None, FAKE + 8, need, 0)
    assert e.value.status == wi.WI_ERR_WORKSPACE


def test_decode_gated_rejects_missing_gate_inputs_and_aliasing():
    p = _dparams()
    need = wi.wi_decode_workspace_bytes(p)
    sel_bytes = p.B * p.Hq * p.top_k * 4
    far = FAKE + (1 << 30)

    def call(**kw):
        a = dict(q_prev=FAKE + 4096, sel_prev=far, tau=0.9, sel=far + sel_bytes, ws=FAKE, ws_bytes=need, p=p)
        a.update(kw)
        with pytest.raises(wi.WaveIndexError) as e:
            wi.wi_decode_gated(a["p"], _view(), FAKE, a["q_prev"], a["sel_prev"], a["tau"], FAKE, None,
                               a["sel"], None, a["ws"], a["ws_bytes"], 0)
        return e.value.status

    assert call(q_prev=None) == wi.WI_ERR_INVALID_ARG
    assert call(sel_prev=None) == wi.WI_ERR_INVALID_ARG
    assert call(tau=float("nan")) == wi.WI_ERR_INVALID_ARG
    assert call(sel=None) == wi.WI_ERR_INVALID_ARG
    assert call(sel=far + sel_bytes - 4) == wi.WI_ERR_INVALID_ARG      # last row shared
    assert call(ws_bytes=need - 1) == wi.WI_ERR_WORKSPACE
    assert call(p=_dparams(Hq=12)) == wi.WI_ERR_INVALID_ARG              # same checks as wi_decode


def test_select_refresh_rejects_null_sel_ids_and_does_nothing_for_top_k_zero():
    p = _dparams()
    need = wi.wi_decode_workspace_bytes(p)
    with pytest.raises(wi.WaveIndexError) as e:
        wi.wi_select_refresh(p, _view(), FAKE, None, FAKE, need, 0)
    assert e.value.status == wi.WI_ERR_INVALID_ARG
    with pytest.raises(wi.WaveIndexError) as e:
        wi.wi_select_refresh(p, _view(), FAKE, FAKE, FAKE, need - 1, 0)
    assert e.value.status == wi.WI_ERR_WORKSPACE
    assert wi.wi_select_refresh(_dparams(top_k=0), _view(), FAKE, None, FAKE, need, 0) == wi.WI_OK


def test_bound_data_and_bounded_decode_reject_bad_arguments():
    p = _dparams()
    with pytest.raises(wi.WaveIndexError) as e:            # vmax is required
        wi.wi_bound_data(p, _view(), FAKE, FAKE, None, 0)
    assert e.value.status == wi.WI_ERR_INVALID_ARG
    with pytest.raises(wi.WaveIndexError) as e:            # radius is required when C > 0
        wi.wi_bound_data(p, _view(), None, FAKE, FAKE, 0)
    assert e.value.status == wi.WI_ERR_INVALID_ARG
    with pytest.raises(wi.WaveIndexError) as e:
        wi.wi_bound_data(_dparams(d=64), _view(), FAKE, FAKE, FAKE, 0)
    assert e.value.status == wi.WI_ERR_UNSUPPORTED
    need = wi.wi_decode_workspace_bytes(p)

    def bounded(pp=p, radius=FAKE, vmax=FAKE, eps=0.1, ws_bytes=need):
        with pytest.raises(wi.WaveIndexError) as e:
            wi.wi_decode_bounded(pp, _view(), radius, FAKE, vmax, FAKE, eps, FAKE, None, None, None, None,
                                 None, FAKE, ws_bytes, 0)
        return e.value.status

    assert bounded(radius=None) == wi.WI_ERR_INVALID_ARG
    assert bounded(vmax=None) == wi.WI_ERR_INVALID_ARG
    assert bounded(eps=-1.0) == wi.WI_ERR_INVALID_ARG
    assert bounded(eps=float("nan")) == wi.WI_ERR_INVALID_ARG
    assert bounded(pp=_dparams(top_k=2049)) == wi.WI_ERR_UNSUPPORTED
    assert bounded(ws_bytes=need - 1) == wi.WI_ERR_WORKSPACE


def test_wavebuf_rejects_bad_sizes_and_small_memory():
    p = _dparams()
    for cache, exe, status in ((-1, 8, wi.WI_ERR_INVALID_ARG), (8, -1, wi.WI_ERR_INVALID_ARG),
                               (1 << 25, 1, wi.WI_ERR_UNSUPPORTED),
                               # cache + both execution-buffer regions past 2^29 rows, although
                               # cache + one region is within it
                               ((1 << 24), (1 << 23) + 1, wi.WI_ERR_UNSUPPORTED)):
        with pytest.raises(wi.WaveIndexError) as e:
            wi.wi_wavebuf_device_bytes(p, cache, exe)
        assert e.value.status == status
    # exactly 2^29 rows: cache 2^24 blocks + 2 x 2^23 blocks of 16 rows
    assert wi.wi_wavebuf_device_bytes(p, 1 << 24, 1 << 23) > 0
    need = wi.wi_wavebuf_device_bytes(p, 1000, 100)
    # pool blocks of 16 rows of K and V, directory, claims and locations per block, the log
    assert need >= 1100 * 16 * 128 * 2 * 2 + 3 * 8 * -(-131004 // 16) * 4
    with pytest.raises(wi.WaveIndexError) as e:
        wi.wi_wavebuf_create(p, 1000, 100, FAKE, need - 1, 0)
    assert e.value.status == wi.WI_ERR_WORKSPACE
    with pytest.raises(wi.WaveIndexError) as e:
        wi.wi_decode_wavebuf(None, p, _view(), FAKE, FAKE, None, None, FAKE, 1 << 40, 0)
    assert e.value.status == wi.WI_ERR_INVALID_ARG


def test_build_rejects_null_inputs_and_small_workspace():
    p = wi.BuildParams(1, 8, 4096, 128, 4, 64, 1024, 64, 3, wi.WI_BF16, 1)
    need = wi.wi_index_shapes_for(p).build_workspace_bytes
    with pytest.raises(wi.WaveIndexError) as e:
        wi.wi_build_index(p, None, FAKE, _view(), FAKE, need, 0)
    assert e.value.status == wi.WI_ERR_INVALID_ARG
    with pytest.raises(wi.WaveIndexError) as e:
        wi.wi_build_index(p, FAKE, FAKE, _view(), FAKE, need - 1, 0)
    assert e.value.status == wi.WI_ERR_WORKSPACE


def test_status_strings():
    for s in (wi.WI_OK, wi.WI_ERR_INVALID_ARG, wi.WI_ERR_UNSUPPORTED, wi.WI_ERR_WORKSPACE, wi.WI_ERR_HIP):
        assert wi.wi_status_string(s)
    assert wi.wi_status_string(-99) == "unknown status"


def test_profile_hook_modes():
    L = wi.lib()
    assert L.wi_profile_enable(-1) == wi.WI_ERR_INVALID_ARG
    assert L.wi_profile_enable(5) == wi.WI_OK           # five back-to-back launches per decode kernel
    stages = wi.wi_profile_read()                         # nothing recorded yet
    assert all(v == (0.0, 0) for v in stages.values())
    assert L.wi_profile_enable(0) == wi.WI_OK
    assert L.wi_profile_rotate(None, -1) == wi.WI_ERR_INVALID_ARG
    assert L.wi_profile_rotate(None, 2) == wi.WI_ERR_INVALID_ARG
    assert wi.wi_profile_rotate([_view(), _view()]) == wi.WI_OK
    assert wi.wi_profile_rotate([]) == wi.WI_OK


def test_decode_noalloc_rejects_workspaces_beyond_its_static_array():
    # batch 16 at 128K needs ~86 MiB of workspace, more than the 64 MiB static array; the call is
    # rejected on the host, before the device is looked up
    p = _dparams(B=16)
    assert wi.wi_decode_workspace_bytes(p) > 64 << 20
    with pytest.raises(wi.WaveIndexError) as e:
        wi.wi_decode_noalloc(p, _view(), FAKE, FAKE, None, None, 0)
    assert e.value.status == wi.WI_ERR_UNSUPPORTED
    with pytest.raises(wi.WaveIndexError) as e:
        wi.wi_decode_noalloc(_dparams(top_k=-1), _view(), FAKE, FAKE, None, None, 0)
    assert e.value.status == wi.WI_ERR_INVALID_ARG
