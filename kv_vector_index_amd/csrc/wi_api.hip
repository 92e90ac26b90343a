// C ABI of the wave-index library: host-side validation, buffer sizing, workspace carving and
// launch order.  No device memory is allocated here; every buffer comes from the caller.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "wave_index.h"
#include "wi_device.h"
#include "wi_internal.h"

namespace {

thread_local char g_err[512] = "";

wi_status fail(wi_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

bool sync_debug() {
  static int v = -1;
  if (v < 0) {
    const char* e = std::getenv("WI_SYNC_DEBUG");
    v = (e && e[0] == '1') ? 1 : 0;
  }
  return v == 1;
}

wi_status check_hip(hipError_t e, const char* what, hipStream_t s) {
  if (e == hipSuccess && sync_debug()) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(WI_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return WI_OK;
}

constexpr int64_t kMaxRows = (int64_t)1 << 31;   // rows (of d elements) per buffer

struct Derived {
  int64_t NS, Nc, lo, L, nseg, C;
};

wi_status derive_build(const wi_build_params* p, Derived* d) {
  if (!p) return fail(WI_ERR_INVALID_ARG, "params is null");
  if (p->B < 1 || p->Hkv < 1 || p->N < 1)
    return fail(WI_ERR_INVALID_ARG, "B, Hkv and N must be >= 1 (got %d, %d, %d)", p->B, p->Hkv, p->N);
  if (p->d != wi::kD) return fail(WI_ERR_UNSUPPORTED, "head dim %d unsupported (only 128)", p->d);
  if (p->sink < 0 || p->window < 0 || p->seg_len < 0)
    return fail(WI_ERR_INVALID_ARG, "sink, window and seg_len must be >= 0");
  if (p->clusters_per_seg < 1) return fail(WI_ERR_INVALID_ARG, "clusters_per_seg must be >= 1");
  if (p->clusters_per_seg > wi::kMaxClustersPerSeg)
    return fail(WI_ERR_UNSUPPORTED, "clusters_per_seg %d > %d", p->clusters_per_seg, wi::kMaxClustersPerSeg);
  if (p->iters < 1) return fail(WI_ERR_INVALID_ARG, "iters must be >= 1");
  if (p->dtype != WI_F32 && p->dtype != WI_BF16) return fail(WI_ERR_INVALID_ARG, "bad dtype %d", p->dtype);
  const int64_t N = p->N;
  d->NS = std::min<int64_t>(N, (int64_t)p->sink + p->window);
  if ((int64_t)p->sink + p->window >= N) { d->Nc = 0; d->lo = N; }
  else { d->Nc = N - p->sink - p->window; d->lo = p->sink; }
  d->L = (p->seg_len == 0) ? d->Nc : p->seg_len;
  if (d->L > wi::kMaxSegLen)
    return fail(WI_ERR_UNSUPPORTED, "segment length %lld > %d", (long long)d->L, wi::kMaxSegLen);
  d->nseg = d->Nc > 0 ? wi::ceil_div(d->Nc, d->L) : 0;
  d->C = d->nseg * p->clusters_per_seg;
  const int64_t BG = (int64_t)p->B * p->Hkv;
  if (BG * N >= kMaxRows || BG * (d->C + 1) >= kMaxRows)
    return fail(WI_ERR_UNSUPPORTED, "an index buffer would exceed 2^31 rows");
  return WI_OK;
}

}  // namespace

namespace wi {

bool g_prof_on = false;
int g_prof_reps = 1;
static std::vector<wi_index_view> g_prof_views;   // rotation list of the repeats (host copies)

DecodeArgs prof_args(const DecodeArgs& a, int r) {
  if (!g_prof_on || g_prof_views.empty() || a.paged) return a;
  const wi_index_view& v = g_prof_views[(size_t)r % g_prof_views.size()];
  DecodeArgs x = a;
  x.mu = v.centroids; x.sv = v.value_sums; x.offsets = v.offsets; x.sizes = v.sizes;
  x.k_perm = v.k_perm; x.v_perm = v.v_perm; x.k_steady = v.k_steady; x.v_steady = v.v_steady;
  return x;
}

namespace {
struct ProfRec {
  int stage;
  hipEvent_t a, b;
  int reps;            // launches of the stage between a and b
};
std::mutex g_prof_mu;
std::vector<ProfRec> g_prof_recs;
hipEvent_t g_prof_open[WI_NUM_STAGES] = {};
}  // namespace

void prof_record(int stage, bool begin, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  hipEvent_t ev;
  if (hipEventCreate(&ev) != hipSuccess) return;
  (void)hipEventRecord(ev, s);
  if (begin) {
    g_prof_open[stage] = ev;
  } else if (g_prof_open[stage]) {
    g_prof_recs.push_back({stage, g_prof_open[stage], ev, g_prof_reps});
    g_prof_open[stage] = nullptr;
  } else {
    (void)hipEventDestroy(ev);
  }
}

BuildLayout build_layout(const wi_build_params& p) {
  BuildLayout L{};
  Derived d{};
  derive_build(&p, &d);
  L.C = d.C; L.Nc = d.Nc; L.NS = d.NS; L.nseg = d.nseg; L.L = d.L;
  const int64_t BG = (int64_t)p.B * p.Hkv;
  const size_t e = p.dtype == WI_BF16 ? 2 : 4;
  size_t o = 0;
  L.off_mhat = o;      o = align256(o + (size_t)BG * d.C * kD * e);
  L.off_assign = o;    o = align256(o + (size_t)BG * d.Nc * 4);
  L.off_flag_cnt = o;  o = align256(o + (size_t)p.iters * 4);
  L.off_flag_list = o; o = align256(o + (size_t)BG * d.Nc * 4);
  L.total = o;
  return L;
}

DecodeLayout decode_layout(const wi_decode_params& p) {
  DecodeLayout L{};
  L.BG = p.B * p.Hkv;
  L.BH = p.B * p.Hq;
  L.G = p.Hq / p.Hkv;
  L.W32 = (int)ceil_div(p.C, 32);
  L.tiles_g = (int)ceil_div(p.C, kScoreTile);
  // estimation workgroups per KV group: about kEstTarget in all, each over whole score tiles
  const int64_t est_target = select_half_blocks(L.BH, p.C) ? kEstTargetMany : kEstTarget;
  L.est_blocks_g = (int)std::max<int64_t>(
      std::min<int64_t>({L.tiles_g, ceil_div(est_target, L.BG), ceil_div(p.C, kEstMinClusters)}), p.C > 0 ? 1 : 0);
  // Attention workgroups per query head: Sc fold the retrieved clusters' estimation terms (64
  // each); S split the head's exact tokens (steady zone + retrieved clusters, estimated from
  // the mean cluster size).  S fills about one resident wave of the grid (kAttTarget in all)
  // but gives no workgroup fewer than 64 or, when the grid must queue anyway, 336 tokens (1M
  // tokens, batch 1: 32 token workgroups per head, four per CU; attend 34.1 us with 512-token
  // workgroups, 32.9 us with these).
  const int Sc = p.top_k > 0 ? (int)ceil_div(p.top_k, kCorrEntries) : 0;
  const int64_t tok_est = (int64_t)p.n_steady + (p.C > 0 ? ceil_div((int64_t)p.top_k * p.Nc, p.C) : 0);
  const int64_t fill = (int64_t)kAttTarget / L.BH - Sc;
  L.att_split = (int)std::max<int64_t>(1, std::min<int64_t>(ceil_div(tok_est, 64), std::max<int64_t>(ceil_div(tok_est, 336), fill)));
  L.att_items = L.att_split + Sc;
  const size_t BG = L.BG, BH = L.BH, C = p.C, G = L.G, K = p.top_k;
  size_t o = 0;
  L.off_keys = o;       o = align256(o + BH * C * 4);
  L.off_tile_norm = o;  o = align256(o + BG * L.tiles_g * 4);
  L.off_tile_cnt = o;   o = align256(o + BG * L.tiles_g * 4);
  L.off_tile_top = o;   o = align256(o + BH * L.tiles_g * kTileTop * 4);
  L.off_tile_top_id = o; o = align256(o + BH * L.tiles_g * kTileTop * 4);
  L.off_band_ids = o;   o = align256(o + BH * C * 4);
  L.off_band_key = o;   o = align256(o + BH * C * 8);
  L.off_all_sel = o;    o = align256(o + BH * 4);
  L.off_gate = o;       o = align256(o + BG * 4);
  L.off_bnd = o;        o = align256(o + BH * 4 * 4);
  L.off_bnd_redo = o;   o = align256(o + BH * 4);
  L.off_hl_cid = o;     o = align256(o + BH * K * 4);
  L.off_hl_row = o;     o = align256(o + BH * K * 4);
  L.off_hl_pre = o;     o = align256(o + BH * (K + 1) * 4);
  L.off_hl_key = o;     o = align256(o + BH * K * 4);
  L.off_att_bounds = o; o = align256(o + BH * L.att_split * 4);
  L.off_est_md = o;     o = align256(o + BG * L.est_blocks_g * G * 2 * 4);
  L.off_est_num = o;    o = align256(o + BG * L.est_blocks_g * G * kD * 4);
  L.off_att_md = o;     o = align256(o + BH * L.att_items * 2 * 4);
  L.off_att_num = o;    o = align256(o + BH * L.att_items * kD * 4);
  L.total = o;
  return L;
}

}  // namespace wi

// ---- allocation-free decode: the workspace is this file's static device array.  Host code never
// names the array itself (its host-side name is only a registration handle): the device address
// comes from hipGetSymbolAddress, once per device with that device current, and is kept per device.
namespace {
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kScratchMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchMaxDevices] = {};

wi_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(WI_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kScratchMaxDevices)
    return fail(WI_ERR_UNSUPPORTED, "device %d: the static workspace serves devices 0..%d", dev, kScratchMaxDevices - 1);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(WI_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return WI_OK;
}
}  // namespace

extern "C" {

wi_status wi_index_shapes_for(const wi_build_params* p, wi_index_shapes* out) {
  if (!out) return fail(WI_ERR_INVALID_ARG, "out is null");
  Derived d{};
  wi_status s = derive_build(p, &d);
  if (s != WI_OK) return s;
  const int64_t BG = (int64_t)p->B * p->Hkv;
  out->C = d.C;
  out->Nc = d.Nc;
  out->n_steady = d.NS;
  out->nseg = d.nseg;
  out->centroids = BG * d.C * wi::kD;
  out->value_sums = BG * d.C * wi::kD;
  out->sizes = BG * d.C;
  out->offsets = BG * (d.C + 1);
  out->perm = BG * d.Nc;
  out->k_perm = BG * d.Nc * wi::kD;
  out->v_perm = BG * d.Nc * wi::kD;
  out->k_steady = BG * d.NS * wi::kD;
  out->v_steady = BG * d.NS * wi::kD;
  out->build_workspace_bytes = (int64_t)wi::build_layout(*p).total;
  return WI_OK;
}

wi_status wi_build_index(const wi_build_params* p, const void* k, const void* v,
                         const wi_index_view* out, void* workspace, size_t ws_bytes, void* stream) {
  Derived d{};
  wi_status s = derive_build(p, &d);
  if (s != WI_OK) return s;
  if (!k || !v) return fail(WI_ERR_INVALID_ARG, "k and v must be non-null");
  if (!out) return fail(WI_ERR_INVALID_ARG, "index view is null");
  if (!out->offsets || (d.NS > 0 && (!out->k_steady || !out->v_steady)))
    return fail(WI_ERR_INVALID_ARG, "index view has a null offsets or steady-zone pointer");
  if (d.Nc > 0 && (!out->centroids || !out->value_sums || !out->sizes || !out->perm ||
                   !out->k_perm || !out->v_perm))
    return fail(WI_ERR_INVALID_ARG, "index view has a null pointer");
  const wi::BuildLayout L = wi::build_layout(*p);
  if (L.total > 0 && (!workspace || ws_bytes < L.total))
    return fail(WI_ERR_WORKSPACE, "build workspace of %zu bytes given, %zu needed", ws_bytes, L.total);
  if (reinterpret_cast<uintptr_t>(workspace) & 255)
    return fail(WI_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  return check_hip(wi::launch_build(*p, L, k, v, *out, workspace, st), "wi_build_index launch", st);
}

// [a, a + na) and [b, b + nb) share a byte (null ranges never do)
static bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

wi_status wi_index_append_segment(const wi_build_params* p, const void* k, const void* v,
                                  const wi_index_view* prev, const wi_index_view* out,
                                  void* workspace, size_t ws_bytes, void* stream) {
  Derived d{};
  wi_status s = derive_build(p, &d);
  if (s != WI_OK) return s;
  if (p->seg_len < 1) return fail(WI_ERR_INVALID_ARG, "appending a segment needs an explicit seg_len");
  if (d.Nc < d.L || d.Nc % d.L != 0)
    return fail(WI_ERR_INVALID_ARG, "the clustered range (%lld tokens) must be a positive multiple of seg_len (%lld)",
                (long long)d.Nc, (long long)d.L);
  if (!k || !v) return fail(WI_ERR_INVALID_ARG, "k and v must be non-null");
  if (!prev || !out) return fail(WI_ERR_INVALID_ARG, "index view is null");
  if (!out->offsets || (d.NS > 0 && (!out->k_steady || !out->v_steady)) || !out->centroids ||
      !out->value_sums || !out->sizes || !out->perm || !out->k_perm || !out->v_perm)
    return fail(WI_ERR_INVALID_ARG, "output index view has a null pointer");
  const int64_t BG = (int64_t)p->B * p->Hkv, e = p->dtype == WI_BF16 ? 2 : 4;
  const int64_t C0 = (d.nseg - 1) * p->clusters_per_seg, N0 = (d.nseg - 1) * d.L;
  if (C0 > 0 && (!prev->centroids || !prev->value_sums || !prev->sizes || !prev->offsets ||
                 !prev->perm || !prev->k_perm || !prev->v_perm))
    return fail(WI_ERR_INVALID_ARG, "previous index view has a null pointer");
  const size_t rowc = (size_t)(BG * C0 * wi::kD * e), rowc1 = (size_t)(BG * d.C * wi::kD * e);
  const size_t rown = (size_t)(BG * N0 * wi::kD * e), rown1 = (size_t)(BG * d.Nc * wi::kD * e);
  if (overlaps(prev->centroids, rowc, out->centroids, rowc1) ||
      overlaps(prev->value_sums, rowc, out->value_sums, rowc1) ||
      overlaps(prev->sizes, (size_t)(BG * C0 * 4), out->sizes, (size_t)(BG * d.C * 4)) ||
      overlaps(prev->offsets, (size_t)(BG * (C0 + 1) * 4), out->offsets, (size_t)(BG * (d.C + 1) * 4)) ||
      overlaps(prev->perm, (size_t)(BG * N0 * 4), out->perm, (size_t)(BG * d.Nc * 4)) ||
      overlaps(prev->k_perm, rown, out->k_perm, rown1) || overlaps(prev->v_perm, rown, out->v_perm, rown1))
    return fail(WI_ERR_INVALID_ARG, "the previous and the new index buffers overlap");
  const wi::BuildLayout L = wi::build_layout(*p);
  if (L.total > 0 && (!workspace || ws_bytes < L.total))
    return fail(WI_ERR_WORKSPACE, "build workspace of %zu bytes given, %zu needed", ws_bytes, L.total);
  if (reinterpret_cast<uintptr_t>(workspace) & 255)
    return fail(WI_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  return check_hip(wi::launch_build(*p, L, k, v, *out, workspace, st, prev, (int)d.nseg - 1),
                   "wi_index_append_segment launch", st);
}

wi_status wi_decode_workspace_bytes(const wi_decode_params* p, size_t* bytes) {
  if (!p || !bytes) return fail(WI_ERR_INVALID_ARG, "null argument");
  if (p->B < 1 || p->Hq < 1 || p->Hkv < 1 || p->Hq % p->Hkv != 0)
    return fail(WI_ERR_INVALID_ARG, "need B, Hq, Hkv >= 1 and Hkv dividing Hq");
  if (p->C < 0 || p->Nc < 0 || p->n_steady < 0 || p->top_k < 0)
    return fail(WI_ERR_INVALID_ARG, "negative C, Nc, n_steady or top_k");
  *bytes = wi::decode_layout(*p).total;
  return WI_OK;
}

struct Bounded {
  const float* radius;
  const float* vnorm;
  const float* vmax;
  float eps;
  int32_t* k_used;
  float* err_bound;
  uint32_t* n_exact;
};

struct Gate {
  const void* q_prev;
  const int32_t* sel_prev;
  int32_t* reused;
  float tau;
  bool refresh;            // select only, for the groups the last gated call reused
};

static wi_status decode_common(const wi_decode_params* p, const wi_index_view* idx, const void* q, float* out,
                               float* lse, int32_t* sel_ids, void* workspace, size_t ws_bytes, void* stream,
                               const Gate* gate, const Bounded* bnd = nullptr, wi::WaveBuf* wb = nullptr) {
  if (!p || !idx || !q || !out) return fail(WI_ERR_INVALID_ARG, "params, index, q and out must be non-null");
  if (p->B < 1 || p->Hq < 1 || p->Hkv < 1 || p->Hq % p->Hkv != 0)
    return fail(WI_ERR_INVALID_ARG, "need B, Hq, Hkv >= 1 and Hkv dividing Hq");
  if (p->d != wi::kD) return fail(WI_ERR_UNSUPPORTED, "head dim %d unsupported (only 128)", p->d);
  if (p->dtype != WI_F32 && p->dtype != WI_BF16) return fail(WI_ERR_INVALID_ARG, "bad dtype %d", p->dtype);
  const int G = p->Hq / p->Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(WI_ERR_UNSUPPORTED, "query heads per KV head must be 1, 2, 4 or 8 (got %d)", G);
  if ((int64_t)p->B * p->Hkv > wi::kMaxGroupsPerDecode)
    return fail(WI_ERR_UNSUPPORTED, "B * Hkv = %lld > %d", (long long)p->B * p->Hkv, wi::kMaxGroupsPerDecode);
  if (p->C < 0 || p->Nc < 0 || p->n_steady < 0 || p->top_k < 0)
    return fail(WI_ERR_INVALID_ARG, "negative C, Nc, n_steady or top_k");
  if ((int64_t)p->n_steady + p->Nc < 1) return fail(WI_ERR_INVALID_ARG, "empty context");
  if ((p->C == 0) != (p->Nc == 0)) return fail(WI_ERR_INVALID_ARG, "C and Nc must be both zero or both positive");
  if (p->Nc >= (1 << 23) || p->n_steady >= (1 << 23))
    return fail(WI_ERR_UNSUPPORTED, "more than 2^23 clustered or steady tokens per KV head");
  if (p->C > wi::kMaxDecodeClusters)
    return fail(WI_ERR_UNSUPPORTED, "more than %d clusters per KV head", wi::kMaxDecodeClusters);
  if (!(p->scale > 0.f) || !std::isfinite(p->scale)) return fail(WI_ERR_INVALID_ARG, "scale must be finite and > 0");
  const int64_t BG = (int64_t)p->B * p->Hkv;
  if (BG * ((int64_t)p->Nc + p->n_steady) >= kMaxRows || (int64_t)p->B * p->Hq * ((int64_t)p->C + 1) >= kMaxRows)
    return fail(WI_ERR_UNSUPPORTED, "a buffer would exceed 2^31 rows");
  if (!idx->offsets || (p->n_steady > 0 && (!idx->k_steady || !idx->v_steady)))
    return fail(WI_ERR_INVALID_ARG, "index view has a null offsets or steady-zone pointer");
  if (p->C > 0 && (!idx->centroids || !idx->value_sums || !idx->sizes || !idx->k_perm || !idx->v_perm))
    return fail(WI_ERR_INVALID_ARG, "index view has a null pointer");
  if (sel_ids && p->top_k == 0) sel_ids = nullptr;
  const wi::DecodeLayout L = wi::decode_layout(*p);
  if (!workspace || ws_bytes < L.total)
    return fail(WI_ERR_WORKSPACE, "decode workspace of %zu bytes given, %zu needed", ws_bytes, L.total);
  if (reinterpret_cast<uintptr_t>(workspace) & 255)
    return fail(WI_ERR_WORKSPACE, "workspace must be 256-byte aligned");

  wi::DecodeArgs a{};
  a.mu = idx->centroids; a.sv = idx->value_sums; a.offsets = idx->offsets; a.sizes = idx->sizes;
  a.k_perm = idx->k_perm; a.v_perm = idx->v_perm; a.k_steady = idx->k_steady; a.v_steady = idx->v_steady;
  a.q = q; a.out = out; a.lse = lse; a.sel_ids = sel_ids;
  char* base = static_cast<char*>(workspace);
  a.keys = reinterpret_cast<uint32_t*>(base + L.off_keys);
  a.tile_norm = reinterpret_cast<float*>(base + L.off_tile_norm);
  a.tile_cnt = reinterpret_cast<int32_t*>(base + L.off_tile_cnt);
  a.tile_top = reinterpret_cast<uint32_t*>(base + L.off_tile_top);
  a.tile_top_id = reinterpret_cast<int32_t*>(base + L.off_tile_top_id);
  a.band_ids = reinterpret_cast<int32_t*>(base + L.off_band_ids);
  a.band_key = reinterpret_cast<uint64_t*>(base + L.off_band_key);
  a.all_sel = reinterpret_cast<int32_t*>(base + L.off_all_sel);
  a.gate = reinterpret_cast<int32_t*>(base + L.off_gate);
  a.bnd = reinterpret_cast<float*>(base + L.off_bnd);
  a.bnd_redo = reinterpret_cast<int32_t*>(base + L.off_bnd_redo);
  a.hl_cid = reinterpret_cast<int32_t*>(base + L.off_hl_cid);
  a.hl_row = reinterpret_cast<int32_t*>(base + L.off_hl_row);
  a.hl_pre = reinterpret_cast<int32_t*>(base + L.off_hl_pre);
  a.hl_key = reinterpret_cast<uint32_t*>(base + L.off_hl_key);
  a.att_bounds = reinterpret_cast<int32_t*>(base + L.off_att_bounds);
  a.est_md = reinterpret_cast<float*>(base + L.off_est_md);
  a.est_num = reinterpret_cast<float*>(base + L.off_est_num);
  a.att_md = reinterpret_cast<float*>(base + L.off_att_md);
  a.att_num = reinterpret_cast<float*>(base + L.off_att_num);
  a.B = p->B; a.Hq = p->Hq; a.Hkv = p->Hkv; a.G = G; a.C = p->C; a.Nc = p->Nc; a.NS = p->n_steady;
  a.top_k = p->top_k; a.W32 = L.W32; a.tiles_g = L.tiles_g; a.est_blocks_g = L.est_blocks_g;
  a.att_split = L.att_split; a.att_items = L.att_items;
  a.scale = p->scale;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (gate && gate->refresh) {
    a.refresh = 1;
    return check_hip(wi::launch_refresh(*p, a, st), "wi_select_refresh launch", st);
  }
  if (gate) {
    a.gated = 1; a.q_prev = gate->q_prev; a.sel_prev = gate->sel_prev; a.reused = gate->reused;
    a.tau = gate->tau;
  }
  if (wb) {
    if (!wi::wavebuf_matches(wb, *p)) return fail(WI_ERR_INVALID_ARG, "wave buffer made for other B, Hkv, Nc or dtype");
    if (p->Nc > 0) {
      // the device's view of the host copies; memory the device cannot read is an error here
      // rather than a fault in the attention kernel
      void* dk = nullptr;
      void* dv = nullptr;
      if (hipHostGetDevicePointer(&dk, idx->k_perm, 0) != hipSuccess ||
          hipHostGetDevicePointer(&dv, idx->v_perm, 0) != hipSuccess || !dk || !dv) {
        (void)hipGetLastError();
        return fail(WI_ERR_INVALID_ARG, "k_perm and v_perm must be pinned host memory (hipHostMalloc)");
      }
      a.k_perm = dk;
      a.v_perm = dv;
    }
    const hipError_t e = wi::wavebuf_begin(wb, st, a);
    if (e != hipSuccess) return check_hip(e, "wave buffer admission", st);
  }
  if (bnd) {
    a.bounded = 1; a.radius = bnd->radius; a.vnorm = bnd->vnorm; a.vmax = bnd->vmax; a.eps = bnd->eps;
    a.k_used = bnd->k_used; a.err_bound = bnd->err_bound; a.bnd_fallback = bnd->n_exact;
    a.u = p->dtype == WI_BF16 ? 0x1.0002p-8f : 0x1p-24f;     // 2^-8 + 2^-23 for bfloat16 sums
  }
  return check_hip(wi::launch_decode(*p, a, st),
                   gate ? "wi_decode_gated launch" : bnd ? "wi_decode_bounded launch"
                   : wb ? "wi_decode_wavebuf launch" : "wi_decode launch", st);
}

wi_status wi_decode(const wi_decode_params* p, const wi_index_view* idx, const void* q, float* out,
                    float* lse, int32_t* sel_ids, void* workspace, size_t ws_bytes, void* stream) {
  return decode_common(p, idx, q, out, lse, sel_ids, workspace, ws_bytes, stream, nullptr);
}

wi_status wi_decode_noalloc(const wi_decode_params* p, const wi_index_view* idx, const void* q, float* out,
                            float* lse, int32_t* sel_ids, void* stream) {
  size_t need = 0;
  wi_status s = wi_decode_workspace_bytes(p, &need);
  if (s != WI_OK) return s;
  if (need > kScratchBytes)
    return fail(WI_ERR_UNSUPPORTED, "this decode needs %zu workspace bytes; the static workspace holds %zu",
                need, kScratchBytes);
  void* ws = nullptr;
  if ((s = scratch_for_current_device(&ws)) != WI_OK) return s;
  return decode_common(p, idx, q, out, lse, sel_ids, ws, kScratchBytes, stream, nullptr);
}

wi_status wi_decode_gated(const wi_decode_params* p, const wi_index_view* idx, const void* q,
                          const void* q_prev, const int32_t* sel_prev, float tau, float* out, float* lse,
                          int32_t* sel_ids, int32_t* reused, void* workspace, size_t ws_bytes, void* stream) {
  if (!q_prev || !sel_prev) return fail(WI_ERR_INVALID_ARG, "q_prev and sel_prev must be non-null");
  if (std::isnan(tau)) return fail(WI_ERR_INVALID_ARG, "tau is NaN");
  if (p && p->top_k > 0 && !sel_ids)
    return fail(WI_ERR_INVALID_ARG, "sel_ids must be non-null: it is the next step's sel_prev");
  if (p && p->top_k > 0 && p->B > 0 && p->Hq > 0) {
    const size_t nb = (size_t)p->B * p->Hq * p->top_k * sizeof(int32_t);
    if (overlaps(sel_prev, nb, sel_ids, nb)) return fail(WI_ERR_INVALID_ARG, "sel_prev and sel_ids overlap");
  }
  const Gate gate{q_prev, sel_prev, reused, tau, false};
  return decode_common(p, idx, q, out, lse, sel_ids, workspace, ws_bytes, stream, &gate);
}

wi_status wi_decode_bounded(const wi_decode_params* p, const wi_index_view* idx, const float* radius,
                            const float* vnorm, const float* vmax, const void* q, float eps, float* out, float* lse,
                            int32_t* sel_ids, int32_t* k_used, float* err_bound, uint32_t* n_exact,
                            void* workspace, size_t ws_bytes, void* stream) {
  if (p && p->C > 0 && (!radius || !vnorm)) return fail(WI_ERR_INVALID_ARG, "radius and vnorm must be non-null");
  if (!vmax) return fail(WI_ERR_INVALID_ARG, "vmax must be non-null");
  if (!(eps >= 0.f)) return fail(WI_ERR_INVALID_ARG, "eps must be >= 0 (got %g)", (double)eps);
  if (p && p->top_k > wi::kBoundedMaxTopK)
    return fail(WI_ERR_UNSUPPORTED, "top_k %d > %d for bounded zone sizing", p->top_k, wi::kBoundedMaxTopK);
  const Bounded bnd{radius, vnorm, vmax, eps, k_used, err_bound, n_exact};
  return decode_common(p, idx, q, out, lse, sel_ids, workspace, ws_bytes, stream, nullptr, &bnd);
}

wi_status wi_select_refresh(const wi_decode_params* p, const wi_index_view* idx, const void* q,
                            int32_t* sel_ids, void* workspace, size_t ws_bytes, void* stream) {
  if (p && p->top_k > 0 && !sel_ids) return fail(WI_ERR_INVALID_ARG, "sel_ids must be non-null");
  if (p && p->top_k == 0) return WI_OK;       // nothing to select
  const Gate gate{nullptr, nullptr, nullptr, 0.f, true};
  // out is not written; any non-null pointer passes the shared checks
  return decode_common(p, idx, q, reinterpret_cast<float*>(workspace), nullptr, sel_ids, workspace, ws_bytes,
                       stream, &gate);
}

const char* wi_status_string(wi_status s) {
  switch (s) {
    case WI_OK: return "ok";
    case WI_ERR_INVALID_ARG: return "invalid argument";
    case WI_ERR_UNSUPPORTED: return "unsupported configuration";
    case WI_ERR_WORKSPACE: return "workspace too small or misaligned";
    case WI_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* wi_last_error(void) { return g_err; }

wi_status wi_bound_data(const wi_decode_params* p, const wi_index_view* idx, float* radius, float* vnorm,
                        float* vmax, void* stream) {
  if (!p || !idx || !vmax) return fail(WI_ERR_INVALID_ARG, "params, index and vmax must be non-null");
  if (p->B < 1 || p->Hkv < 1) return fail(WI_ERR_INVALID_ARG, "need B, Hkv >= 1");
  if (p->d != wi::kD) return fail(WI_ERR_UNSUPPORTED, "head dim %d unsupported (only 128)", p->d);
  if (p->dtype != WI_F32 && p->dtype != WI_BF16) return fail(WI_ERR_INVALID_ARG, "bad dtype %d", p->dtype);
  if (p->C < 0 || p->Nc < 0 || p->n_steady < 0) return fail(WI_ERR_INVALID_ARG, "negative C, Nc or n_steady");
  if ((p->C == 0) != (p->Nc == 0)) return fail(WI_ERR_INVALID_ARG, "C and Nc must be both zero or both positive");
  const int64_t BG = (int64_t)p->B * p->Hkv;
  if (BG > wi::kMaxGroupsPerDecode) return fail(WI_ERR_UNSUPPORTED, "B * Hkv = %lld > %d", (long long)BG, wi::kMaxGroupsPerDecode);
  if (BG * ((int64_t)p->Nc + p->n_steady) >= kMaxRows || BG * ((int64_t)p->C + 1) >= kMaxRows)
    return fail(WI_ERR_UNSUPPORTED, "a buffer would exceed 2^31 rows");
  if (p->n_steady > 0 && !idx->v_steady) return fail(WI_ERR_INVALID_ARG, "index view has a null v_steady");
  if (p->C > 0 && (!idx->centroids || !idx->offsets || !idx->k_perm || !idx->v_perm || !radius || !vnorm))
    return fail(WI_ERR_INVALID_ARG, "null index buffer, radius or vnorm");
  hipStream_t st = static_cast<hipStream_t>(stream);
  return check_hip(wi::launch_bound_data(*p, *idx, radius, vnorm, vmax, st), "wi_bound_data launch", st);
}

static wi_status wavebuf_check(const wi_decode_params* p, int32_t cache_blocks, int32_t exec_blocks) {
  if (!p) return fail(WI_ERR_INVALID_ARG, "null params");
  if (p->B < 1 || p->Hkv < 1) return fail(WI_ERR_INVALID_ARG, "need B, Hkv >= 1");
  if (p->d != wi::kD) return fail(WI_ERR_UNSUPPORTED, "head dim %d unsupported (only 128)", p->d);
  if (p->dtype != WI_F32 && p->dtype != WI_BF16) return fail(WI_ERR_INVALID_ARG, "bad dtype %d", p->dtype);
  if (p->Nc < 0 || cache_blocks < 0 || exec_blocks < 0)
    return fail(WI_ERR_INVALID_ARG, "negative Nc, cache_blocks or exec_blocks");
  // the pool holds the cache and two execution-buffer regions (one per call parity); the
  // attention kernel addresses its rows with 29 bits
  if (((int64_t)cache_blocks + 2 * (int64_t)exec_blocks) * wi::kWbBlock > wi::kWbMaxPoolRows)
    return fail(WI_ERR_UNSUPPORTED, "a wave-buffer pool (cache + 2 x execution buffer) holds at most 2^29 rows");
  if ((int64_t)p->B * p->Hkv * wi::ceil_div(std::max(p->Nc, 1), wi::kWbBlock) >= kMaxRows)
    return fail(WI_ERR_UNSUPPORTED, "too many blocks");
  return WI_OK;
}

wi_status wi_wavebuf_device_bytes(const wi_decode_params* p, int32_t cache_blocks, int32_t exec_blocks,
                                  size_t* bytes) {
  const wi_status st = wavebuf_check(p, cache_blocks, exec_blocks);
  if (st != WI_OK) return st;
  if (!bytes) return fail(WI_ERR_INVALID_ARG, "null output");
  *bytes = wi::wavebuf_device_bytes(*p, cache_blocks, exec_blocks);
  return WI_OK;
}

wi_status wi_wavebuf_create(const wi_decode_params* p, int32_t cache_blocks, int32_t exec_blocks, void* device_mem,
                            size_t bytes, void* stream, wi_wavebuf** out) {
  const wi_status st = wavebuf_check(p, cache_blocks, exec_blocks);
  if (st != WI_OK) return st;
  if (!out) return fail(WI_ERR_INVALID_ARG, "null output");
  const size_t need = wi::wavebuf_device_bytes(*p, cache_blocks, exec_blocks);
  if (!device_mem || bytes < need) return fail(WI_ERR_WORKSPACE, "wave buffer memory of %zu bytes given, %zu needed", bytes, need);
  if (reinterpret_cast<uintptr_t>(device_mem) & 255) return fail(WI_ERR_WORKSPACE, "wave buffer memory must be 256-byte aligned");
  wi::WaveBuf* w = nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const wi_status r = check_hip(wi::wavebuf_create(*p, cache_blocks, exec_blocks, device_mem, s, &w), "wi_wavebuf_create", s);
  if (r != WI_OK) return r;
  *out = reinterpret_cast<wi_wavebuf*>(w);
  return WI_OK;
}

wi_status wi_decode_wavebuf(wi_wavebuf* wb, const wi_decode_params* p, const wi_index_view* idx, const void* q,
                            float* out, float* lse, int32_t* sel_ids, void* workspace, size_t ws_bytes,
                            void* stream) {
  if (!wb) return fail(WI_ERR_INVALID_ARG, "null wave buffer");
  return decode_common(p, idx, q, out, lse, sel_ids, workspace, ws_bytes, stream, nullptr, nullptr,
                       reinterpret_cast<wi::WaveBuf*>(wb));
}

wi_status wi_wavebuf_stats(wi_wavebuf* wb, int64_t* stats) {
  if (!wb || !stats) return fail(WI_ERR_INVALID_ARG, "null wave buffer or output");
  wi::WaveBuf* w = reinterpret_cast<wi::WaveBuf*>(wb);
  const hipError_t e = wi::wavebuf_sync_log(w);
  if (e != hipSuccess) return fail(WI_ERR_HIP, "wave buffer log: %s", hipGetErrorString(e));
  std::memcpy(stats, wi::wavebuf_stats(w), 6 * sizeof(int64_t));
  return WI_OK;
}

wi_status wi_wavebuf_destroy(wi_wavebuf* wb) {
  wi::wavebuf_destroy(reinterpret_cast<wi::WaveBuf*>(wb));
  return WI_OK;
}

static void prof_clear() {
  for (auto& r : wi::g_prof_recs) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  wi::g_prof_recs.clear();
  for (auto& e : wi::g_prof_open)
    if (e) { (void)hipEventDestroy(e); e = nullptr; }
}

wi_status wi_profile_enable(int enable) {
  std::lock_guard<std::mutex> lk(wi::g_prof_mu);
  if (enable < 0) return fail(WI_ERR_INVALID_ARG, "negative profiling mode %d", enable);
  if (enable) prof_clear();
  wi::g_prof_on = enable != 0;
  wi::g_prof_reps = enable > 1 ? enable : 1;
  return WI_OK;
}

wi_status wi_profile_rotate(const wi_index_view* views, int n) {
  std::lock_guard<std::mutex> lk(wi::g_prof_mu);
  if (n < 0 || (n > 0 && !views)) return fail(WI_ERR_INVALID_ARG, "rotation list: need n >= 0 and views for n > 0");
  wi::g_prof_views.assign(views, views + n);
  return WI_OK;
}

wi_status wi_profile_read(double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return fail(WI_ERR_INVALID_ARG, "null output array");
  std::lock_guard<std::mutex> lk(wi::g_prof_mu);
  for (int i = 0; i < WI_NUM_STAGES; ++i) { total_ms[i] = 0.0; launches[i] = 0; }
  for (auto& r : wi::g_prof_recs) {
    hipError_t e = hipEventSynchronize(r.b);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) return fail(WI_ERR_HIP, "profiling events: %s", hipGetErrorString(e));
    // a decode stage launched `reps` times back to back between its events counts as that many
    const int reps = (r.stage <= WI_STAGE_MERGE || r.stage == WI_STAGE_REFRESH) ? r.reps : 1;
    total_ms[r.stage] += ms;
    launches[r.stage] += reps;
  }
  return WI_OK;
}

}  // extern "C"
