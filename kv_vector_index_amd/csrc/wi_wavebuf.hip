// Wave buffer: decode over an index whose cluster-major K/V copies live in host memory (RetroInfer
// technical summary, section 2.B; Arabic summary, section 2.b).  The pages describe a GPU-side
// cache of KV blocks that exploits the temporal locality of the retrieved tokens, management that
// runs on the CPU off the attention's critical path (LRU replacement, metadata), and an execution
// buffer that holds the retrieved vectors for the attention kernel.
//
// Here (MI355X): index metadata (centroids, value sums, sizes, offsets) and the steady zone stay in
// HBM; the clustered rows are split into blocks of kWbBlock rows.  One device pool holds the cache
// (slots [0, cache_blocks)) and the execution buffer (slots [cache_blocks, cache_blocks +
// exec_blocks)).  Each decode call, in stream order:
//   k_wb_admit    copies the previous call's staged misses that the host LRU admitted from the
//                 execution buffer into cache slots and updates the block directory;
//   score, select (unchanged);
//   k_wb_resolve  for every block a head's retrieval zone touches (each once per call, claimed
//                 with an epoch): a cached block is used in place; a missing one is copied from
//                 host memory over PCIe into an execution-buffer slot, or, when the buffer is
//                 full, left in host memory for the attention to read there; every block is
//                 logged;
//   attend (reads rows through the per-call block locations), merge.
// The log goes back to the host on a copy stream while attention runs.  The host decides two
// calls later: the logs, their counters and the execution buffer are double-buffered by call
// parity, so call t applies the admissions decided from call t - 2's log, and the host never waits
// for the call just enqueued.  Deciding means: update the LRU order (hits first, then misses, each
// in ascending block key) and admit every staged miss not cached since, into a free slot or in
// place of the least recently used block.
#include <algorithm>
#include <cstring>
#include <vector>

#include "wi_device.h"
#include "wi_internal.h"
#include "wi_lru.h"

namespace wi {

constexpr int kWbThreads = 256;

__global__ __launch_bounds__(kWbThreads) void k_wb_init(int32_t* dir, int32_t* claim, int64_t n_keys, int32_t* ctr) {
  const int64_t i = (int64_t)blockIdx.x * kWbThreads + threadIdx.x;
  if (i < n_keys) { dir[i] = -1; claim[i] = 0; }
  if (i < 4) ctr[i] = 0;
}

// one 16-row block of K and of V (rows past `rows` are not copied); the whole workgroup or wave
// of `nt` threads takes part, thread t moving 16-byte pieces t, t + nt, ...
template <typename T>
__device__ __forceinline__ void copy_block(const T* __restrict__ sk, const T* __restrict__ sv, T* __restrict__ dk,
                                           T* __restrict__ dv, int rows, int t, int nt) {
  constexpr int per_row = kD * (int)sizeof(T) / 16;      // 16-byte pieces per row
  const int n = rows * per_row;
  for (int i = t; i < n; i += nt) {
    reinterpret_cast<u32x4_t*>(dk)[i] = reinterpret_cast<const u32x4_t*>(sk)[i];
    reinterpret_cast<u32x4_t*>(dv)[i] = reinterpret_cast<const u32x4_t*>(sv)[i];
  }
}

// one batch of admissions: workgroup i copies pool block cp[2 i] (execution buffer) into cache
// slot cp[2 i + 1]; the directory entries up[2 j] take the values up[2 j + 1] (each key once, so
// the writes do not race).  Workgroup 0 also clears the counters this call's resolve uses.
template <typename T>
__global__ __launch_bounds__(kWbThreads) void k_wb_admit(const int32_t* __restrict__ cp, int n_cp,
                                                         const int32_t* __restrict__ up, int n_up, T* pool_k,
                                                         T* pool_v, int32_t* dir, int32_t* ctr) {
  if (blockIdx.x == 0 && threadIdx.x < 4) ctr[threadIdx.x] = 0;
  for (int j = blockIdx.x * kWbThreads + threadIdx.x; j < n_up; j += gridDim.x * kWbThreads) dir[up[2 * j]] = up[2 * j + 1];
  if ((int)blockIdx.x >= n_cp) return;
  const int src = cp[2 * blockIdx.x], dst = cp[2 * blockIdx.x + 1];
  const size_t bs = (size_t)kWbBlock * kD;
  copy_block<T>(pool_k + src * bs, pool_v + src * bs, pool_k + dst * bs, pool_v + dst * bs, kWbBlock, threadIdx.x,
                kWbThreads);
}

struct WbResolveArgs {
  const int32_t* hl_cid;     // the heads' published zones (decode workspace)
  const int32_t* hl_row;
  const int32_t* hl_pre;
  const void* host_k;        // [BG, Nc, d] in host memory
  const void* host_v;
  void* pool_k;
  void* pool_v;
  const int32_t* dir;
  int32_t* claim;
  int32_t* loc;
  int32_t* ctr;              // [0] staged misses, [1] log entries, [2] reads left in host memory
  int32_t* log;              // [log_cap, 2]: block key, pool slot of a staged miss / -1 hit / -2 host
  int log_cap, exec_base, exec_blocks, nblk, epoch;
  int B, Hq, Hkv, G, K, Nc;
};

// grid (B*Hq, ceil(K / 4)): wave w of workgroup (bh, y) takes list entry 4 y + w of head bh
template <typename T>
__global__ __launch_bounds__(kWbThreads) void k_wb_resolve(WbResolveArgs r) {
  const int bh = blockIdx.x, lane = threadIdx.x & 63;
  const int e = blockIdx.y * (kWbThreads / 64) + (threadIdx.x >> 6);
  if (e >= r.K) return;
  const int b = bh / r.Hq, h = bh - b * r.Hq, bg = b * r.Hkv + h / r.G;
  const int32_t* pre = r.hl_pre + (size_t)bh * (r.K + 1);
  const int nrow = pre[e + 1] - pre[e];
  if (nrow <= 0) return;                                 // padding past the list
  const int row0 = r.hl_row[(size_t)bh * r.K + e];
  const int blk0 = row0 / kWbBlock, blk1 = (row0 + nrow - 1) / kWbBlock;
  const size_t bs = (size_t)kWbBlock * kD;
  for (int blk = blk0; blk <= blk1; ++blk) {
    const int key = bg * r.nblk + blk;
    int slot = -3;                                       // -3: another wave claimed the block
    if (lane == 0) {
      const int old = atomicMax(&r.claim[key], r.epoch);
      if (old < r.epoch) {
        const int cached = r.dir[key];
        if (cached >= 0) {
          slot = cached;
        } else {
          const int x = atomicAdd(&r.ctr[0], 1);
          if (x < r.exec_blocks) slot = r.exec_base + x;
          else { slot = -1; atomicAdd(&r.ctr[2], 1); }
        }
        r.loc[key] = slot >= 0 ? slot : -1;
        const int li = atomicAdd(&r.ctr[1], 1);
        if (li < r.log_cap) {
          r.log[2 * li] = key;
          r.log[2 * li + 1] = cached >= 0 ? -1 : (slot >= 0 ? slot - r.exec_base : -2);
        }
        if (cached >= 0) slot = -4;                      // hit: nothing to copy
      }
    }
    slot = __shfl(slot, 0);
    if (slot >= 0) {
      const int rows = min(kWbBlock, r.Nc - blk * kWbBlock);
      const size_t src = ((size_t)bg * r.Nc + (size_t)blk * kWbBlock) * kD;
      copy_block<T>(static_cast<const T*>(r.host_k) + src, static_cast<const T*>(r.host_v) + src,
                    static_cast<T*>(r.pool_k) + slot * bs, static_cast<T*>(r.pool_v) + slot * bs, rows, lane, 64);
    }
  }
}

// ------------------------------------------------------------------ host side
struct WaveBuf {
  int B, Hkv, BG, Nc, nblk, dtype, esize;
  int cache_blocks, exec_blocks, log_cap;
  // device; per call parity: counters, log, admission list, execution-buffer region
  void *pool_k = nullptr, *pool_v = nullptr;
  int32_t *dir = nullptr, *claim = nullptr, *loc = nullptr;
  int32_t *ctr[2] = {nullptr, nullptr}, *log[2] = {nullptr, nullptr}, *adm[2] = {nullptr, nullptr};
  // host (pinned) copies; the counters sit right before the log on both sides, so that one copy
  // brings both back
  int32_t *log_h[2] = {nullptr, nullptr}, *ctr_h[2] = {nullptr, nullptr}, *adm_h[2] = {nullptr, nullptr};
  int copied[2] = {0, 0};                    // log entries each pending copy brings back
  int n_cp[2] = {0, 0}, n_up[2] = {0, 0};    // pending admissions: copies, directory updates
  int last_count = 0;
  hipStream_t copy_stream = nullptr;
  hipEvent_t resolved = nullptr;
  hipEvent_t log_ready[2] = {nullptr, nullptr};
  int64_t enqueued = 0;                      // calls enqueued
  int64_t processed = 0;                     // calls whose log has been processed
  int epoch = 0;
  WbLru* lru = nullptr;                      // the policy (and the counters)

  // the log of call `processed` (parity q): the decisions applied two calls later
  void process_log(int q) {
    const int n = std::min(ctr_h[q][1], log_cap);
    if (n > copied[q])       // more entries than the copy brought back: fetch the rest now
      (void)hipMemcpy(log_h[q] + 2 * (size_t)copied[q], log[q] + 2 * (size_t)copied[q], (size_t)(n - copied[q]) * 8,
                      hipMemcpyDeviceToHost);
    last_count = n;
    lru->decide(log_h[q], n, q, adm_h[q], &n_cp[q], adm_h[q] + 2 * (size_t)std::max(exec_blocks, 1), &n_up[q]);
    ++processed;
  }
  hipError_t process_through(int64_t last) {  // every log up to call `last` (inclusive)
    while (processed <= last && processed < enqueued) {
      const int q = (int)(processed & 1);
      const hipError_t e = hipEventSynchronize(log_ready[q]);
      if (e != hipSuccess) return e;
      process_log(q);
    }
    return hipSuccess;
  }
};

struct WbLayout {
  size_t pool_k, pool_v, dir, claim, loc, log, log_stride, adm, total;
};

static WbLayout wb_layout(int64_t BG, int64_t nblk, int64_t pool_blocks, int64_t exec_blocks, int esize,
                          int64_t log_cap) {
  WbLayout L{};
  size_t o = 0;
  const size_t blk_bytes = (size_t)kWbBlock * kD * esize;
  L.pool_k = o; o = align256(o + pool_blocks * blk_bytes);
  L.pool_v = o; o = align256(o + pool_blocks * blk_bytes);
  L.dir = o;    o = align256(o + BG * nblk * 4);
  L.claim = o;  o = align256(o + BG * nblk * 4);
  L.loc = o;    o = align256(o + BG * nblk * 4);
  L.log_stride = align256(16 + (size_t)log_cap * 8);   // per parity: 4 counters, then the log
  L.log = o;    o = align256(o + 2 * L.log_stride);
  L.adm = o;    o = align256(o + 2 * std::max<int64_t>(exec_blocks, 1) * 24);   // copies + updates
  L.total = o;
  return L;
}

static int64_t wb_nblk(int Nc) { return ceil_div(std::max(Nc, 1), kWbBlock); }

// the pool: cache_blocks cached blocks, then two execution-buffer regions of exec_blocks
size_t wavebuf_device_bytes(const wi_decode_params& p, int cache_blocks, int exec_blocks) {
  const int64_t BG = (int64_t)p.B * p.Hkv, nblk = wb_nblk(p.Nc);
  const int esize = p.dtype == WI_BF16 ? 2 : 4;
  return wb_layout(BG, nblk, (int64_t)cache_blocks + 2 * (int64_t)exec_blocks, exec_blocks, esize, BG * nblk).total;
}

hipError_t wavebuf_create(const wi_decode_params& p, int cache_blocks, int exec_blocks, void* mem, hipStream_t s,
                          WaveBuf** out) {
  WaveBuf* w = new WaveBuf();
  w->B = p.B; w->Hkv = p.Hkv; w->BG = p.B * p.Hkv; w->Nc = p.Nc; w->nblk = (int)wb_nblk(p.Nc);
  w->dtype = p.dtype; w->esize = p.dtype == WI_BF16 ? 2 : 4;
  w->cache_blocks = cache_blocks; w->exec_blocks = exec_blocks;
  w->log_cap = w->BG * w->nblk;
  const WbLayout L = wb_layout(w->BG, w->nblk, (int64_t)cache_blocks + 2 * (int64_t)exec_blocks, exec_blocks,
                               w->esize, w->log_cap);
  char* base = static_cast<char*>(mem);
  w->pool_k = base + L.pool_k; w->pool_v = base + L.pool_v;
  w->dir = reinterpret_cast<int32_t*>(base + L.dir);
  w->claim = reinterpret_cast<int32_t*>(base + L.claim);
  w->loc = reinterpret_cast<int32_t*>(base + L.loc);
  const size_t ea = (size_t)std::max(exec_blocks, 1);
  for (int q = 0; q < 2; ++q) {
    w->ctr[q] = reinterpret_cast<int32_t*>(base + L.log + L.log_stride * q);
    w->log[q] = w->ctr[q] + 4;
    w->adm[q] = reinterpret_cast<int32_t*>(base + L.adm) + 6 * ea * q;
  }
  w->lru = new WbLru(cache_blocks, exec_blocks, (int64_t)w->BG * w->nblk);
  hipError_t e = hipSuccess;
  for (int q = 0; q < 2 && e == hipSuccess; ++q) {
    e = hipHostMalloc(reinterpret_cast<void**>(&w->ctr_h[q]), (size_t)w->log_cap * 8 + 16, hipHostMallocDefault);
    if (e == hipSuccess) e = hipHostMalloc(reinterpret_cast<void**>(&w->adm_h[q]), ea * 24, hipHostMallocDefault);
    if (e == hipSuccess) { std::memset(w->ctr_h[q], 0, 16); w->log_h[q] = w->ctr_h[q] + 4; }
    if (e == hipSuccess) e = hipEventCreateWithFlags(&w->log_ready[q], hipEventDisableTiming);
  }
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&w->copy_stream, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&w->resolved, hipEventDisableTiming);
  if (e == hipSuccess) {
    const int64_t nk = (int64_t)w->BG * w->nblk;
    hipLaunchKernelGGL(k_wb_init, dim3((unsigned)ceil_div(std::max<int64_t>(nk, 8), kWbThreads)), dim3(kWbThreads), 0, s,
                       w->dir, w->claim, nk, w->ctr[0]);
    e = hipGetLastError();
  }
  if (e != hipSuccess) { wavebuf_destroy(w); return e; }
  *out = w;
  return hipSuccess;
}

void wavebuf_destroy(WaveBuf* w) {
  if (!w) return;
  if (w->copy_stream) (void)hipStreamSynchronize(w->copy_stream);
  for (int q = 0; q < 2; ++q) {
    if (w->ctr_h[q]) (void)hipHostFree(w->ctr_h[q]);
    if (w->adm_h[q]) (void)hipHostFree(w->adm_h[q]);
    if (w->log_ready[q]) (void)hipEventDestroy(w->log_ready[q]);
  }
  if (w->resolved) (void)hipEventDestroy(w->resolved);
  if (w->copy_stream) (void)hipStreamDestroy(w->copy_stream);
  delete w->lru;
  delete w;
}

hipError_t wavebuf_sync_log(WaveBuf* w) { return w->process_through(w->enqueued - 1); }

const int64_t* wavebuf_stats(WaveBuf* w) { return w->lru->stats; }

bool wavebuf_matches(const WaveBuf* w, const wi_decode_params& p) {
  return w->B == p.B && w->Hkv == p.Hkv && w->Nc == p.Nc && w->dtype == p.dtype;
}

// before the decode kernels of call t (parity q): the logs through call t - 2, and the admissions
// decided from call t - 2 (whose staged misses are still in region q of the execution buffer)
hipError_t wavebuf_begin(WaveBuf* w, hipStream_t s, DecodeArgs& a) {
  const int64_t t = w->enqueued;
  const int q = (int)(t & 1);
  hipError_t e = w->process_through(t - 2);
  if (e != hipSuccess) return e;
  const int ncp = w->n_cp[q], nup = w->n_up[q];
  const size_t ea = (size_t)std::max(w->exec_blocks, 1);
  // the block copies, then the directory updates (decided after 2 ea ints, moved up to follow the
  // copies), in one transfer
  if (nup > 0 && ncp < (int)ea) std::memmove(w->adm_h[q] + 2 * (size_t)ncp, w->adm_h[q] + 2 * ea, (size_t)nup * 8);
  if (ncp + nup > 0 &&
      (e = hipMemcpyAsync(w->adm[q], w->adm_h[q], (size_t)(ncp + nup) * 8, hipMemcpyHostToDevice, s)) != hipSuccess)
    return e;
  const int32_t* cp = w->adm[q];
  const int32_t* up = w->adm[q] + 2 * (size_t)ncp;
  if (w->dtype == WI_BF16)
    hipLaunchKernelGGL(k_wb_admit<uint16_t>, dim3(std::max(ncp, 1)), dim3(kWbThreads), 0, s, cp, ncp, up, nup,
                       static_cast<uint16_t*>(w->pool_k), static_cast<uint16_t*>(w->pool_v), w->dir, w->ctr[q]);
  else
    hipLaunchKernelGGL(k_wb_admit<float>, dim3(std::max(ncp, 1)), dim3(kWbThreads), 0, s, cp, ncp, up, nup,
                       static_cast<float*>(w->pool_k), static_cast<float*>(w->pool_v), w->dir, w->ctr[q]);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // adm_h[q] is rewritten when call t's log is processed, which waits for an event recorded after
  // this copy in stream order
  w->n_cp[q] = 0;
  w->n_up[q] = 0;
  ++w->epoch;
  ++w->lru->stats[0];
  ++w->enqueued;
  a.paged = 1;
  a.wb_nblk = w->nblk;
  a.wb_loc = w->loc;
  a.pool_k = w->pool_k;
  a.pool_v = w->pool_v;
  a.wb = w;
  return hipSuccess;
}

// between select and attend (call enqueued - 1, parity q)
hipError_t launch_wb_resolve(const DecodeArgs& a, hipStream_t s) {
  WaveBuf* w = static_cast<WaveBuf*>(a.wb);
  const int q = (int)((w->enqueued - 1) & 1);
  WbResolveArgs r{};
  r.hl_cid = a.hl_cid; r.hl_row = a.hl_row; r.hl_pre = a.hl_pre;
  r.host_k = a.k_perm; r.host_v = a.v_perm; r.pool_k = w->pool_k; r.pool_v = w->pool_v;
  r.dir = w->dir; r.claim = w->claim; r.loc = w->loc; r.ctr = w->ctr[q]; r.log = w->log[q];
  r.log_cap = w->log_cap; r.exec_base = w->cache_blocks + q * w->exec_blocks; r.exec_blocks = w->exec_blocks;
  r.nblk = w->nblk; r.epoch = w->epoch;
  r.B = a.B; r.Hq = a.Hq; r.Hkv = a.Hkv; r.G = a.G; r.K = a.top_k; r.Nc = a.Nc;
  if (a.top_k > 0 && a.C > 0) {
    const dim3 grid((unsigned)(a.B * a.Hq), (unsigned)ceil_div(a.top_k, kWbThreads / 64));
    if (w->dtype == WI_BF16) hipLaunchKernelGGL(k_wb_resolve<uint16_t>, grid, dim3(kWbThreads), 0, s, r);
    else hipLaunchKernelGGL(k_wb_resolve<float>, grid, dim3(kWbThreads), 0, s, r);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // the counters and the log (right after them) go back in one copy on the copy stream while the
  // attention runs: as many entries as the last processed log held, with room to spare (a longer
  // log is fetched in full when it is processed)
  const int ncopy = std::min(w->log_cap, 2 * w->last_count + 4096);
  w->copied[q] = ncopy;
  hipError_t e = hipEventRecord(w->resolved, s);
  if (e == hipSuccess) e = hipStreamWaitEvent(w->copy_stream, w->resolved, 0);
  if (e == hipSuccess)
    e = hipMemcpyAsync(w->ctr_h[q], w->ctr[q], 16 + (size_t)ncopy * 8, hipMemcpyDeviceToHost, w->copy_stream);
  if (e == hipSuccess) e = hipEventRecord(w->log_ready[q], w->copy_stream);
  return e;
}

}  // namespace wi
