// Internal host/device declarations of the wave-index library: workspace layouts and launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include <algorithm>
#include <cmath>
#include <stdint.h>

#include "wave_index.h"

namespace wi {

constexpr int kScoreTile = 128;     // clusters per workgroup of the score kernel
constexpr int kEstTarget = 224;     // estimation workgroups a decode aims for: the CUs the select's
                                    // 1024-thread workgroups leave free at batch 1 (256 - 32), or,
constexpr int kEstTargetMany = 512; // with 512-thread select blocks, two workgroups per CU
constexpr int kEstMinClusters = 512; // clusters an estimation workgroup streams at least (fewer,
                                     // longer workgroups leave the merge fewer partials)
constexpr int kTileTop = 8;         // best scores per head the score kernel keeps of each tile
constexpr int kMaxGroup = 8;        // query heads per KV head supported by the decode kernels
constexpr int kMaxSegLen = 65536;   // tokens per k-means segment
constexpr int kMaxClustersPerSeg = 4096;
constexpr int kMaxGroupsPerDecode = 65535;  // B * Hkv of one decode call (a grid dimension)
constexpr int kCorrEntries = 64;    // retrieved clusters per correction workgroup
constexpr int kSelectBitmapLds = 65536;   // dynamic LDS of the select kernel: 2 bitmaps over C
constexpr int kMaxDecodeClusters = kSelectBitmapLds / 8 * 32;   // C per KV head (262144)
constexpr int kBoundedMaxTopK = 2048;    // clusters the bounded select ranks in LDS
constexpr int kWbBlock = 16;        // rows per wave-buffer block
constexpr int64_t kWbMaxPoolRows = (int64_t)1 << 29;   // rows a wave-buffer pool may hold
constexpr int kAttTarget = 768;     // attention workgroups a batch-1 step aims for (3 per CU)

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The select launch runs 512-thread workgroups beyond 256 query heads (two heads a CU), and also
// at fewer heads when two of its workgroups fit one CU's LDS (the static arrays and the
// bitmaps over at most 16384 clusters): smaller blocks synchronise faster (128K tokens, batch 1:
// select 12.1 -> 10.6 us).  With more clusters a workgroup needs most of a CU's LDS, and the
// 1024-thread form streams the estimation faster (1M tokens: 30.9 against 41.3 us).
inline bool select_half_blocks(int BH, int C) { return BH > 256 || C <= 16384; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ------------------------------------------------------------------ decode workspace
struct DecodeLayout {
  int BG, BH, G, W32, tiles_g, est_blocks_g, att_split, att_items;
  size_t off_keys, off_tile_norm, off_tile_cnt, off_tile_top, off_tile_top_id, off_band_ids, off_band_key, off_all_sel, off_gate, off_bnd, off_bnd_redo,
      off_hl_cid, off_hl_row, off_hl_pre, off_hl_key, off_att_bounds, off_est_md, off_est_num,
      off_att_md, off_att_num, total;
};
DecodeLayout decode_layout(const wi_decode_params& p);

// Device pointers of one decode call.
struct DecodeArgs {
  const void* mu;          // [BG, C, d]
  const void* sv;          // [BG, C, d]
  const int32_t* offsets;  // [BG, C+1]
  const int32_t* sizes;    // [BG, C]
  const void* k_perm;      // [BG, Nc, d]
  const void* v_perm;
  const void* k_steady;    // [BG, NS, d]
  const void* v_steady;
  const void* q;           // [BH, d]
  float* out;              // [BH, d]
  float* lse;              // [BH] or null
  int32_t* sel_ids;        // [BH, top_k] or null
  // workspace
  uint32_t* keys;          // [BH, C] order key of the fp32 score <q, mu_c> (0: empty cluster)
  float* tile_norm;        // [BG, tiles_g] largest centroid norm of each 128-cluster tile
  int32_t* tile_cnt;       // [BG, tiles_g] non-empty clusters of each tile
  uint32_t* tile_top;      // [BH, tiles_g, kTileTop] best score keys of each tile, descending
  int32_t* tile_top_id;    // [BH, tiles_g, kTileTop] their cluster ids
  int32_t* band_ids;       // [BH, C]
  uint64_t* band_key;      // [BH, C]
  int32_t* all_sel;        // [BH] 1 when every non-empty cluster was retrieved
  // the head's retrieval zone, ascending cluster id, padded to top_k (cid 0, row 0, key 0 and
  // first token = n_tok past the list)
  int32_t* hl_cid;         // [BH, top_k]
  int32_t* hl_row;         // [BH, top_k]    first k_perm row
  int32_t* hl_pre;         // [BH, top_k+1]  first token (steady zone first); [top_k] = n_tok
  uint32_t* hl_key;        // [BH, top_k]    order key of the fp32 score
  int32_t* att_bounds;     // [BH, S]        list entry holding the first retrieved token of
                           //                token workgroup s
  float* est_md;           // [BG, est_blocks_g, G, 2] (m, den) of each estimation workgroup's tiles
  float* est_num;          // [BG, est_blocks_g, G, d]
  float* att_md;           // [BH, S + Sc, 2]
  float* att_num;          // [BH, S + Sc, d]
  // selection reuse (gated decode; gated == 0 otherwise)
  const void* q_prev;      // [BH, d] the previous step's queries
  const int32_t* sel_prev; // [BH, top_k] the previous step's retrieved ids
  int32_t* reused;         // [BG] or null: 1 where the KV head reused its heads' zones
  int32_t* gate;           // [BG] workspace: the same flags, kept for a later refresh
  float tau;
  int gated;
  int refresh;             // select only: fresh zones for the groups gate[] marks, into sel_ids
  // accuracy-bounded zone sizing (bounded == 0 otherwise)
  const float* radius;     // [BG, C] cluster radius around the stored centroid
  const float* vnorm;      // [BG, C] largest member value norm
  const float* vmax;       // [BG]    largest value norm of the context
  float eps;               // error bound the zone must meet
  float u;                 // relative rounding bound of the stored value sums
  int bounded;
  int32_t* k_used;         // [BH] or null: zone size chosen
  uint32_t* bnd_fallback;  // [1] or null: incremented once per head whose zone size was decided in fp64
  int32_t* bnd_redo;       // [BH] workspace: 1 where the bounded select left the head to its fp64 launch
  float* err_bound;        // [BH] or null: bound on |out - dense attention|
  float* bnd;              // [BH, 4] workspace: m*, sum a, sum (a V + w u V), sum lo over the estimation zone
  // wave buffer (paged == 0 otherwise): k_perm / v_perm are then the copies in host memory
  int paged;
  int wb_nblk;             // blocks of kWbBlock rows per (b, KV head)
  const int32_t* wb_loc;   // [BG, wb_nblk] this step's pool block of every needed block, -1: host
  const void* pool_k;      // [pool blocks, kWbBlock, d] cache and execution buffer
  const void* pool_v;
  void* wb;                // the wave buffer's host state (read by the launcher only)
  // shapes
  int B, Hq, Hkv, G, C, Nc, NS, top_k, W32, tiles_g, est_blocks_g, att_split, att_items;
  float scale;
};

hipError_t launch_decode(const wi_decode_params& p, const DecodeArgs& a, hipStream_t s);
hipError_t launch_refresh(const wi_decode_params& p, const DecodeArgs& a, hipStream_t s);
struct WaveBuf;
size_t wavebuf_device_bytes(const wi_decode_params& p, int cache_blocks, int exec_blocks);
hipError_t wavebuf_create(const wi_decode_params& p, int cache_blocks, int exec_blocks, void* mem, hipStream_t s,
                          WaveBuf** out);
void wavebuf_destroy(WaveBuf* w);
hipError_t wavebuf_sync_log(WaveBuf* w);
const int64_t* wavebuf_stats(WaveBuf* w);
bool wavebuf_matches(const WaveBuf* w, const wi_decode_params& p);
hipError_t wavebuf_begin(WaveBuf* w, hipStream_t s, DecodeArgs& a);
hipError_t launch_wb_resolve(const DecodeArgs& a, hipStream_t s);
hipError_t launch_bound_data(const wi_decode_params& p, const wi_index_view& idx, float* radius, float* vnorm,
                             float* vmax, hipStream_t s);

// ------------------------------------------------------------------ profiling hook
extern bool g_prof_on;
extern int g_prof_reps;   // decode kernels launched this many times back to back while profiling
inline int prof_reps() { return g_prof_on ? g_prof_reps : 1; }
// The arguments of repeat r of a decode kernel while profiling: with a rotation list set
// (wi_profile_rotate), the index pointers of list entry r mod n (copies of the call's index at
// other addresses); otherwise, and for a wave-buffer decode, the call's own arguments.
DecodeArgs prof_args(const DecodeArgs& a, int r);
void prof_record(int stage, bool begin, hipStream_t s);
inline void prof_begin(int stage, hipStream_t s) { if (g_prof_on) prof_record(stage, true, s); }
inline void prof_end(int stage, hipStream_t s) { if (g_prof_on) prof_record(stage, false, s); }

// ------------------------------------------------------------------ build workspace
struct BuildLayout {
  int64_t C, Nc, NS, nseg, L;
  size_t off_mhat, off_assign, off_flag_cnt, off_flag_list, total;
};
BuildLayout build_layout(const wi_build_params& p);

// Build segments [seg0, nseg) of the index of *p into `out`; with seg0 > 0, segments [0, seg0)
// are copied from `prev`, an index of the same parameters over seg0 full segments.
hipError_t launch_build(const wi_build_params& p, const BuildLayout& L, const void* k,
                        const void* v, const wi_index_view& out, void* ws, hipStream_t st,
                        const wi_index_view* prev = nullptr, int seg0 = 0);

}  // namespace wi
